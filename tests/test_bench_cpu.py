"""The measurement script's host-side pieces, on the CPU: the refusal of multi-GPU
runs, the algorithmic work model behind the roofline figures, and the reading of
the committed counter summaries."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_layer_17_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("wid", [1, 2, 3, 5])
def test_gemm_work_is_eighteen_r_d_f(wid):
    """Forward 6·R·d·f (gate, up, down) plus backward 12·R·d·f (two products per forward GEMM)."""
    w = wl.WORKLOADS[wid]
    total = sum(bench.kernel_work(f"G{i}_x", w, 2)[1] for i in range(1, 7))
    assert total == 18.0 * w.R * w.d * w.f
    assert all(bench.kernel_work(f"G{i}_x", w, 2)[0] == "mfma" for i in range(1, 7))


def test_data_movement_bytes():
    w = wl.WORKLOADS[2]
    T, d, R = w.T, w.d, w.R
    assert bench.kernel_work("dispatch", w, 2) == ("hbm", float(T * d * 2 + R * d * 2 + 4 * R))
    assert bench.kernel_work("combine", w, 2) == ("hbm", float(R * d * 2 + T * d * 2 + 8 * R))
    assert bench.kernel_work("combine_bwd", w, 2) == ("hbm", float(T * d * 2 + 2 * R * d * 2 + 12 * R))
    # MXFP8: the combine backward computes dgates only (dout and y_perm read, the permutation and gates read,
    # dgates written); mx_gather reads every expert row from its token row and writes it in the rows layout and
    # in the token-axis layout (R rows padded per expert segment to whole 32-row blocks, then to 128-token groups
    # plus one), one E4M3 byte and 1/32 of a scale byte per element each
    w5 = wl.WORKLOADS[5]
    T5, d5, R5, E5 = w5.T, w5.d, w5.R, w5.E
    assert bench.kernel_work("combine_bwd", w5, 2)[1] == T5 * d5 * 2 + R5 * d5 * 2 + 12 * R5
    rp = 128 * ((R5 // 32 + E5 + 3) // 4 + 1)
    assert rp >= R5 + 32 * E5 // 4 and rp % 128 == 0
    o = 1 + 1 / 32
    f5 = w5.f
    per_launch = [R5 * d5 * 2 + 4 * R5 + (R5 + rp) * d5 * o,          # X: rows read from their tokens, permutation
                  R5 * d5 * 2 + 8 * R5 + (R5 + rp) * d5 * o,          # dY: and the gates
                  R5 * f5 * 2 + (R5 + rp) * f5 * o,                   # dHg, dHu: read in place
                  R5 * f5 * 2 + (R5 + rp) * f5 * o]
    assert bench.kernel_work("mx_gather", w5, 2)[1] == pytest.approx(sum(per_launch) / 4)
    assert bench.kernel_work("no_such_kernel", w, 2) == ("other", 0.0)


def test_counted_traffic_reads_the_committed_summary():
    digest = bench.source_digest()
    assert digest == bench.source_digest() and len(digest) == 16
    path = os.path.join(ROOT, "profiles", "bf16_e8_T8192_hbm_traffic.md")
    with open(path) as fh:
        current = f"source-digest: {digest}" in fh.read()
    got = bench.counted_traffic("bf16_e8_T8192", "G1_bf16")
    if not current:
        assert got is None  # counters taken on other sources are not reported
        return
    w = wl.WORKLOADS[2]
    operands = (w.R * w.d + 2 * w.E * w.d * w.f) * 2  # X_perm and the gate/up weights, read once
    outputs = 3 * w.R * w.f * 2                      # Hg, Hu, A
    assert got is not None and got >= operands + outputs
    assert bench.counted_traffic("no_such_workload", "G1_bf16") is None
    assert bench.counted_traffic("bf16_e8_T8192", "G9_bf16") is None


def test_gemm_bytes_and_binding_roof():
    """Algorithmic bytes per GEMM launch: operands read once, outputs written once; the MXFP8 weight gradients
    (bf16 dW of all 128 experts written) are bound by HBM, the forward gate/up GEMM by the matrix cores."""
    w5 = wl.WORKLOADS[5]
    R, d, f, E = w5.R, w5.d, w5.f, w5.E
    o = 1 + 1 / 32
    assert bench.gemm_bytes("G6_mx", w5, E) == pytest.approx(R * d * o + 2 * R * f * o + 2 * E * d * f * 2)
    assert bench.gemm_bytes("G1_mx", w5, 64) == pytest.approx(R * d * o + 2 * 64 * d * f * o + 3 * R * f * 2)
    r = {"per_step_us": {"G6_mx": 1000.0, "G1_mx": 900.0}, "per_launch_us": {"G6_mx": 1000.0, "G1_mx": 900.0},
         "s": 2}
    roof = bench.roofline(w5, r, E)
    assert roof["kernel"] == "G6_mx" and roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["achieved"] == pytest.approx(bench.gemm_bytes("G6_mx", w5, E) / 1e-3 / 1e9)
    roofs = bench.gemm_roofs(w5, r, E)
    assert roofs["G1_mx"]["bound"] == "mfma" and roofs["G6_mx"]["bound"] == "hbm"
    w2 = wl.WORKLOADS[2]  # bf16, E = 8: every GEMM bound by the matrix cores
    r2 = {"per_step_us": {"G1_bf16": 300.0}, "per_launch_us": {"G1_bf16": 300.0}, "s": 2}
    assert bench.roofline(w2, r2, 8)["bound"] == "mfma"
