"""Layer parity on the GPU: the HIP path through the C ABI against the fp64 oracle.

Small cases keep every workload's distributions but shrink the sizes so the
oracle finishes in seconds while the grids still span several tiles, ragged M
and N tails, empty experts and partial routing blocks.  The full-size cases
(the shapes the bench times) compare every routing integer bit-exactly and
sample token outputs and expert weight gradients that the oracle computes one
by one.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_17_amd import workloads as wl
from oracle import moe_mx_oracle as mxl
from oracle import moe_oracle as mo

import gpu_util as gu

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS

SMALL = {
    "tiny-fp32": W[1],
    "fp32-e16-ragged": wl.scaled(W[1], name="fp32-e16", T=333, E=16, k=4, d=128, f=192),
    "bf16-e8-ragged": wl.scaled(W[2], T=1000, d=256, f=320),
    "bf16-e128": wl.scaled(W[3], T=1536, d=256, f=192),
    "bf16-e128-zipf": wl.scaled(W[4], T=2048, d=256, f=128),
    "bf16-one-token": wl.scaled(W[3], T=1, d=128, f=128, E=8),
    "bf16-single-expert": wl.scaled(W[3], T=130, d=128, f=128, E=1, k=1),
    "bf16-k-equals-E": wl.scaled(W[3], T=96, d=128, f=128, E=8, k=8),
    "bf16-e256-k8": wl.scaled(W[3], T=300, d=128, f=64, E=256, k=8),
    # >= 1024 rows per expert and d, f multiples of 256: the 256 x 256 tile path
    "bf16-big-tiles": wl.scaled(W[3], T=2300, d=512, f=256, E=2, k=1),
    "bf16-big-tiles-k2": wl.scaled(W[3], T=2100, d=256, f=512, E=4, k=2),
    "mxfp8-e16": wl.scaled(W[5], T=700, d=256, f=384, E=16),
    "mxfp8-e128": wl.scaled(W[5], T=1536, d=256, f=256),
    # >= 1024 rows per expert and d, f multiples of 256: the 256 x 256 MX tiles, ragged segment ends
    "mxfp8-big-tiles": wl.scaled(W[5], T=2300, d=512, f=256, E=2, k=1),
    # 569 and 581 rows: three 256-row tiles per expert taken as one triple, last tiles of 57 and 69 rows (the K loop
    # for at most two valid 32-row blocks per wave, and the full one)
    "mxfp8-short-tails": wl.scaled(W[5], T=1150, d=512, f=256, E=2, k=1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity_small(gpu, name):
    w = SMALL[name]
    gu.say(f"case {name}")
    inp = wl.make_inputs(w)
    g, _ = gu.run_gpu_step(w, inp)
    ref = gu.run_oracle(w, inp, g["logits"])
    gu.check_layer(w, g, ref, inp)
    if w.prec == "mxfp8":
        gu.check_mx_against_bf16_oracle(w, g, ref, inp,
                                        ("out", "dgates", "dx", "dw_gate", "dw_up", "dw_down", "dlogits"))


def test_layer_deterministic(gpu):
    w = SMALL["bf16-e128-zipf"]
    gu.say("case determinism")
    inp = wl.make_inputs(w)
    a, _ = gu.run_gpu_step(w, inp)
    b, _ = gu.run_gpu_step(w, inp)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


@pytest.mark.parametrize("name", ["mxfp8-e16", "mxfp8-big-tiles"])
def test_mx_fused_movement_bit_identical(gpu, name):
    """X and dY quantised inside the dispatch and the combine backward, in the rows layout only
    (moe_dispatch_mx, moe_combine_bwd_mx) or in both layouts from the routing permutation
    (moe_dispatch_mx_tok, moe_combine_bwd_mx_tok, with and without the bf16 expert rows), give the same bits as
    letting the FFN quantise them."""
    w = SMALL[name]
    gu.say(f"case fused MX movement {name}")
    inp = wl.make_inputs(w)
    a, step_a = gu.run_gpu_step(w, inp, mx_movement="none")
    assert step_a.x_mx is None
    for movement, keep in (("rows", True), ("tok", True), ("tok", False)):
        b, step_b = gu.run_gpu_step(w, inp, mx_movement=movement, keep_rows=keep)
        assert step_b.x_mx is not None and (step_b.x_mxt is not None) == (movement == "tok")
        assert (step_b.x_perm is None) == (not keep)
        for key in b:
            np.testing.assert_array_equal(a[key], b[key], err_msg=f"{movement} {keep} {key}")
        assert set(a) - set(b) <= {"x_perm"}


@pytest.mark.parametrize("name", ["mxfp8-e16", "mxfp8-big-tiles"])
def test_mx_weight_cache_bit_identical(gpu, name):
    """A step on pre-quantised weights (moe_mx_weight_cache_build) gives the same bits as one that quantises
    the weights itself."""
    w = SMALL[name]
    gu.say(f"case weight cache {name}")
    inp = wl.make_inputs(w)
    a, _ = gu.run_gpu_step(w, inp)
    b, step = gu.run_gpu_step(w, inp, mx_weight_cache=True)
    assert step.mx_wcache is not None
    c, step_c = gu.run_gpu_step(w, inp, mx_weights_per_step=True)  # rebuilt inside the step
    assert step_c.mx_wcache is not None
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
        np.testing.assert_array_equal(a[key], c[key], err_msg=key)


def _sampled_full(w, n_tok=48, seed=0):
    gu.say(f"case full-size {w.name}")
    inp = wl.make_inputs(w)
    g, step = gu.run_gpu_step(w, inp)
    logits = g["logits"].astype(np.float32)
    if "w_router" in inp:
        rows = np.random.default_rng(seed).choice(w.T, 64, replace=False)
        e = gu.rel_err(g["logits"][rows], mo.router_logits(inp["x"][rows], inp["w_router"]))
        assert e <= 1e-5, e
    # every routing integer, full size, bit-exact
    idx = mo.topk_select(logits, w.k)
    meta = mo.routing_metadata(idx, w.E)
    np.testing.assert_array_equal(g["topk_idx"], idx)
    for key in ("counts", "offsets", "perm_src", "perm_dst", "mx_blk_offsets"):
        np.testing.assert_array_equal(g[key], meta[key], err_msg=key)
    assert gu.rel_err(g["gates"], mo.topk_gates(logits, idx)) <= 1e-5
    np.testing.assert_array_equal(g["x_perm"], inp["x"][meta["perm_src"] // w.k])
    # sampled tokens: out, dgates, dx and dlogits depend on the token alone
    # (the router weight gradient does not, and is checked on the small cases)
    r = np.random.default_rng(seed)
    toks = np.sort(r.choice(w.T, n_tok, replace=False))
    mx = w.prec == "mxfp8"
    sub_inp = {key: inp[key][toks] for key in ("x", "dout")}
    sub_inp.update({key: inp[key] for key in ("w_gate", "w_up", "w_down")})
    if mx:
        sub_inp["logits"] = logits[toks]
        sub = mxl.mx_layer_forward_backward(sub_inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], sub_inp["dout"],
                                            w.k, logits=logits[toks], want_dw=False)
    else:
        sub = mo.layer_forward_backward(sub_inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], sub_inp["dout"],
                                        w.k, logits=logits[toks], w_router=inp.get("w_router"), want_dw=False)
    errs = {}
    for key in ("out", "dgates", "dlogits", "dx"):
        errs[key] = gu.rel_err(g[key][toks], sub[key])
    if mx:
        gu.check_mx_against_bf16_oracle(w, g, sub, sub_inp, ("out", "dgates", "dlogits", "dx"), rows=toks,
                                        label=f", {n_tok} sampled tokens, full size")
    # sampled experts, each checked over its whole segment: every row of y_perm
    # and dx_perm, and its three weight gradients.  The hottest, a median one,
    # the coldest non-empty one and (if any) an empty one.  The oracle sees each
    # expert as a one-expert, k = 1 problem over the tokens routed to it, with
    # the oracle's own gates.
    counts = meta["counts"]
    order = np.argsort(counts, kind="stable")
    nonempty = order[counts[order] > 0]
    experts = sorted({int(nonempty[-1]), int(nonempty[len(nonempty) // 2]), int(nonempty[0]), int(order[0])})
    gates = mo.topk_gates(logits, idx)
    for e in experts:
        lo, hi = int(meta["offsets"][e]), int(meta["offsets"][e + 1])
        gu.say(f"  expert {e}: {hi - lo} rows")
        if hi == lo:
            for key in ("dw_gate", "dw_up", "dw_down"):
                assert np.all(g[key][e] == 0.0)
            continue
        slots = meta["perm_src"][lo:hi]
        tk, js = slots // w.k, slots % w.k
        n = hi - lo
        we = [inp[key][e:e + 1] for key in ("w_gate", "w_up", "w_down")]
        dy_e, _ = mo.combine_backward(inp["dout"][tk], np.zeros((n, w.d)), gates[tk, js][:, None],
                                      np.arange(n), 1)
        if mx:
            fwd = mxl.mx_expert_ffn_forward(inp["x"][tk], [0, n], *we)
            ref = mxl.mx_expert_ffn_backward(dy_e, inp["x"][tk], [0, n], *we, fwd=fwd)
        else:
            fwd = mo.expert_ffn_forward(inp["x"][tk], [0, n], *we)
            ref = mo.expert_ffn_backward(dy_e, inp["x"][tk], [0, n], *we)
        errs[f"y_perm[{e}]"] = gu.rel_err(g["y_perm"][lo:hi], fwd["y_perm"])
        errs[f"dx_perm[{e}]"] = gu.rel_err(g["dx_perm"][lo:hi], ref["dx_perm"])
        for key in ("dw_gate", "dw_up", "dw_down"):
            errs[f"{key}[{e}]"] = gu.rel_err(g[key][e], ref[key][0])
    gu.report(f"| {w.name} T={w.T} d={w.d} E={w.E} k={w.k} f={w.f}, full size: {n_tok} tokens, experts "
              f"{experts} ({', '.join(str(int(counts[e])) for e in experts)} rows) | vs oracle "
              f"({'MX' if mx else 'plain'}) | " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + " |")
    bad = {k: v for k, v in errs.items() if v > gu.tol_for(w, k.split("[")[0])}
    assert not bad, f"above tolerance: {bad}"
    del step
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_layer_parity_full_size_sampled(gpu, wid):
    # the fp64 MX oracle encodes every touched expert's weights six times (about 10 s per expert at
    # d = 4096, f = 1536): four sampled tokens touch at most 16 experts
    _sampled_full(W[wid], n_tok=48 if wid != 5 else 4)


def test_mx_forward_gemm_matches_dequantised_operands(gpu):
    """The MX gate/up GEMM equals the fp64 product of the oracle's quantise ->
    dequantise of the same operands, up to the bf16 rounding of its output."""
    from mixture_experts_layer_17_amd import binding as B
    from oracle import mx_oracle as mxo
    w = wl.scaled(W[5], T=600, d=256, f=256, E=8)
    gu.say("case mx gemm vs dequantised operands")
    inp = wl.make_inputs(w)
    idx = mo.topk_select(inp["logits"], w.k)
    meta = mo.routing_metadata(idx, w.E)
    xp = inp["x"][meta["perm_src"] // w.k]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    out = B.moe_grouped_ffn_fwd(dev(xp), torch.from_numpy(meta["offsets"]).cuda(), dev(inp["w_gate"]),
                                dev(inp["w_up"]), dev(inp["w_down"]), "mxfp8")
    torch.cuda.synchronize()
    hg = gu.host(out["h_gate"])
    ref = mxl.mx_expert_ffn_forward(xp, meta["offsets"], inp["w_gate"], inp["w_up"], inp["w_down"])["h_gate"]
    err = gu.rel_err(hg, ref)
    gu.say(f"  mx gemm G1 vs dequantised-operand product: {err:.2e}")
    # bf16 output rounding (2^-9 relative) and the matrix core's own accumulation
    assert err <= 4e-3


def test_mx_down_gemm_matches_dequantised_operands_fused_act(gpu):
    """On 256 x 256 tiles G1's epilogue encodes A for G2 itself (no quantiser pass over the stored A): the MX
    down GEMM equals the fp64 product of the oracle's quantise -> dequantise of the GPU's own bf16 A (along f)
    and of W_down, up to the bf16 rounding of its output.  A misplaced code or scale byte shows well above that."""
    from mixture_experts_layer_17_amd import binding as B
    w = wl.scaled(W[5], T=2300, d=512, f=256, E=2, k=1)  # >= 512 rows per expert: the 256 x 256 tiles
    gu.say("case mx down gemm with the fused A encoding")
    inp = wl.make_inputs(w)
    idx = mo.topk_select(inp["logits"], w.k)
    meta = mo.routing_metadata(idx, w.E)
    xp = inp["x"][meta["perm_src"] // w.k]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    out = B.moe_grouped_ffn_fwd(dev(xp), torch.from_numpy(meta["offsets"]).cuda(), dev(inp["w_gate"]),
                                dev(inp["w_up"]), dev(inp["w_down"]), "mxfp8")
    torch.cuda.synchronize()
    a = gu.host(out["a_act"]).astype(np.float64)
    y = gu.host(out["y_perm"])
    aq = mxl.q_along(a, 1)
    ref = np.zeros(y.shape)
    mag = np.zeros(y.shape)  # sum over f of |a_q w_q|: the scale of the fp32 accumulation's rounding
    off = meta["offsets"]
    for e in range(w.E):
        s = slice(int(off[e]), int(off[e + 1]))
        wq = mxl.q_along(np.asarray(inp["w_down"][e], np.float64), 0)
        ref[s] = aq[s] @ wq
        mag[s] = np.abs(aq[s]) @ np.abs(wq)
    err = gu.rel_err(y, ref)
    gu.say(f"  mx gemm G2 (A encoded by G1) vs dequantised-operand product: {err:.2e}")
    assert err <= 4e-3
    # element by element: the output's bf16 rounding (2^-9 relative) with room for the accumulation order; a
    # scale byte or an 8-column run of codes in the wrong place moves whole rows far past this
    bad = np.abs(y - ref) > 2.0**-8 * np.abs(ref) + 2.0**-12 * mag
    assert not bad.any(), f"{int(bad.sum())} outputs off, first at {np.argwhere(bad)[0]}"
