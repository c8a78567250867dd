"""Per-call parity of the ABI entry points on the GPU against the oracle.

Routing integers, dispatch and the MX quantiser are bit-exact; floats are
compared with max|gpu - oracle| / max|oracle| at the precision's tolerance.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_17_amd import binding as B
from mixture_experts_layer_17_amd import workloads as wl
from oracle import moe_oracle as mo
from oracle import mx_oracle as mxo

import gpu_util as gu

pytestmark = pytest.mark.gpu


def _adversarial(T, E, seed):
    r = np.random.default_rng(seed)
    lg = r.integers(-2, 3, (T, E)).astype(np.float32)   # heavy exact ties
    special = [np.zeros(E, np.float32), np.where(np.arange(E) % 2 == 0, -0.0, 0.0).astype(np.float32),
               np.full(E, 1e30, np.float32), np.full(E, -1e30, np.float32)]
    special[3][E // 2] = 5.0
    for i, row in enumerate(special[:T]):
        lg[i] = row                                       # all-equal rows, +-0.0 ties, extremes
    return lg


ROUTE_CASES = [(1, 8, 2), (63, 8, 4), (64, 8, 4), (65, 16, 4), (1000, 128, 4), (4097, 256, 8), (200, 1, 1),
               (130, 8, 8), (16384, 128, 4),
               (203, 1, 1), (7, 3, 2), (129, 5, 3),  # logit tiles whose size is not a multiple of four
               (97, 9, 2), (50, 7, 1), (33, 6, 3)]  # rows split unevenly over two or four scanning lanes


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_route_topk_bit_exact(gpu, T, E, k, kind):
    gu.say(f"case route T={T} E={E} k={k} {kind}")
    r = np.random.default_rng(T * 7 + E)
    lg = r.standard_normal((T, E)).astype(np.float32) if kind == "normal" else _adversarial(T, E, T)
    out = B.moe_route_topk(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    idx = mo.topk_select(lg, k)
    meta = mo.routing_metadata(idx, E)
    np.testing.assert_array_equal(out["topk_idx"].cpu().numpy(), idx)
    for key in ("counts", "offsets", "perm_src", "perm_dst", "mx_blk_offsets"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), meta[key], err_msg=key)
    assert gu.rel_err(out["gates"].cpu().numpy(), mo.topk_gates(lg, idx)) <= 1e-5


@pytest.mark.parametrize("T,E,k", [(300, 8, 4), (1000, 128, 4), (97, 256, 8), (70, 5, 5)])
def test_route_topk_nan_logits(gpu, T, E, k):
    """NaN logits rank below every number (-inf included), NaNs among themselves by index: indices and
    metadata stay bit-exact; gates agree where no NaN was chosen and the largest chosen logit is finite (a
    chosen -inf then gets gate 0), and are NaN on both sides otherwise."""
    gu.say(f"case route NaN T={T} E={E} k={k}")
    r = np.random.default_rng(T + 3 * E)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[r.random((T, E)) < 0.2] = np.nan
    lg[r.random((T, E)) < 0.03] = -np.inf
    lg[0] = np.nan                       # every logit NaN
    lg[1, : E - 1] = np.nan              # a single number
    out = B.moe_route_topk(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    idx = mo.topk_select(lg, k)
    meta = mo.routing_metadata(idx, E)
    np.testing.assert_array_equal(out["topk_idx"].cpu().numpy(), idx)
    for key in ("counts", "offsets", "perm_src", "perm_dst", "mx_blk_offsets"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), meta[key], err_msg=key)
    chosen = np.take_along_axis(lg, idx.astype(np.int64), axis=1)
    bad = np.any(np.isnan(chosen), axis=1) | ~np.isfinite(chosen[:, 0])
    g = out["gates"].cpu().numpy()
    ref = mo.topk_gates(lg, idx)
    assert (~bad).sum() > T // 4 and bad.sum() > 0
    assert gu.rel_err(g[~bad], ref[~bad]) <= 1e-5
    assert np.all(np.isnan(g[bad])) and np.all(np.isnan(ref[bad]))


@pytest.mark.parametrize("T,E,k,bias", [(1000, 8, 4, 0.0), (2048, 128, 4, 3.0), (333, 256, 8, 3.0), (50, 1, 1, 0.0)])
def test_route_stats_bit_exact(gpu, T, E, k, bias):
    """Load statistics from the device routing equal the oracle's from its own routing (uniform and
    zipf-biased logits, the latter with empty experts)."""
    r = np.random.default_rng(T + E)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg += (bias * np.log(1.0 / (r.permutation(E) + 1))).astype(np.float32)
    out = B.moe_route_topk(torch.from_numpy(lg).cuda(), k)
    st = B.moe_route_stats(out["counts"])
    torch.cuda.synchronize()
    ref = mo.routing_stats(mo.routing_metadata(mo.topk_select(lg, k), E)["counts"])
    np.testing.assert_array_equal(st.cpu().numpy(), ref)


@pytest.mark.parametrize("T,E,k", [(1000, 128, 4), (203, 5, 3)])
def test_route_topk_unaligned_logits(gpu, T, E, k):
    """Logits at a 4-byte (not 16-byte) aligned address take the scalar staging loads: same routing."""
    gu.say(f"case route unaligned T={T} E={E} k={k}")
    lg = np.random.default_rng(T + 5 * E).standard_normal((T, E)).astype(np.float32)
    flat = torch.empty(T * E + 1, dtype=torch.float32, device="cuda")
    view = flat[1:].view(T, E)
    view.copy_(torch.from_numpy(lg))
    assert view.data_ptr() % 16 != 0
    out = B.moe_route_topk(view, k)
    torch.cuda.synchronize()
    idx = mo.topk_select(lg, k)
    meta = mo.routing_metadata(idx, E)
    np.testing.assert_array_equal(out["topk_idx"].cpu().numpy(), idx)
    for key in ("counts", "offsets", "perm_src", "perm_dst", "mx_blk_offsets"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), meta[key], err_msg=key)


def test_route_topk_empty_batch(gpu):
    lg = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    out = B.moe_route_topk(lg, 4)
    torch.cuda.synchronize()
    assert out["offsets"].cpu().numpy().tolist() == [0] * 17
    assert out["counts"].cpu().numpy().tolist() == [0] * 16


@pytest.mark.parametrize("prec", ["f32", "bf16", "mxfp8"])
def test_grouped_ffn_empty_batch(gpu, prec):
    """No routed rows (R = 0): the forward has nothing to write and the backward overwrites every expert's
    weight gradients with exact zeros (the buffers start out holding a non-zero pattern)."""
    gu.say(f"case ffn empty batch {prec}")
    E, d, f = 4, 256, 256
    dt = torch.float32 if prec == "f32" else torch.bfloat16
    gen = torch.Generator().manual_seed(5)
    w = [(0.02 * torch.randn((E, d, f), generator=gen)).to(dt).cuda(),
         (0.02 * torch.randn((E, d, f), generator=gen)).to(dt).cuda(),
         (0.02 * torch.randn((E, f, d), generator=gen)).to(dt).cuda()]
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    x = torch.empty((0, d), dtype=dt, device="cuda")
    fwd = B.moe_grouped_ffn_fwd(x, offsets, *w, prec)
    grads = {"dx_perm": torch.empty((0, d), dtype=dt, device="cuda"),
             "dw_gate": torch.full_like(w[0], 7.0), "dw_up": torch.full_like(w[1], 7.0),
             "dw_down": torch.full_like(w[2], 7.0)}
    B.moe_grouped_ffn_bwd(torch.empty((0, d), dtype=dt, device="cuda"), x, fwd["h_gate"], fwd["h_up"], fwd["a_act"],
                          offsets, offsets, *w, prec, out=grads)
    torch.cuda.synchronize()
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert torch.count_nonzero(grads[key]).item() == 0, key


@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (1000, 128, 4), (77, 256, 8)])
def test_route_topk_bwd(gpu, T, E, k):
    r = np.random.default_rng(3)
    lg = r.standard_normal((T, E)).astype(np.float32)
    dg = r.standard_normal((T, k)).astype(np.float32)
    idx = mo.topk_select(lg, k)
    g = mo.topk_gates(lg, idx).astype(np.float32)
    dl = B.moe_route_topk_bwd(torch.from_numpy(g).cuda(), torch.from_numpy(dg).cuda(),
                              torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    ref = mo.topk_gates_backward(g, dg, idx, E)
    got = dl.cpu().numpy()
    assert gu.rel_err(got, ref) <= 1e-5
    assert np.all(got[ref == 0] == 0.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,d,E,k", [(333, 64, 8, 2), (1000, 2048, 128, 4), (77, 4096, 16, 8)])
def test_dispatch_combine_and_backward(gpu, dtype, T, d, E, k):
    gu.say(f"case permute T={T} d={d} E={E} k={k} {dtype}")
    r = np.random.default_rng(T + d)
    lg = r.standard_normal((T, E)).astype(np.float32)
    idx = mo.topk_select(lg, k)
    meta = mo.routing_metadata(idx, E)
    g = mo.topk_gates(lg, idx).astype(np.float32)
    x = torch.randn((T, d), generator=torch.Generator().manual_seed(1)).to(dtype)
    y = torch.randn((T * k, d), generator=torch.Generator().manual_seed(2)).to(dtype)
    dout = torch.randn((T, d), generator=torch.Generator().manual_seed(3)).to(dtype)
    xd, yd, dd = x.cuda(), y.cuda(), dout.cuda()
    pd = torch.from_numpy(meta["perm_dst"]).cuda()
    gd = torch.from_numpy(g).cuda()
    xp = B.moe_dispatch(xd, pd, k)
    out = B.moe_combine(yd, gd, pd)
    dy, dgt = B.moe_combine_bwd(dd, yd, gd, pd)
    dx = B.moe_dispatch_bwd(yd, pd, k)
    torch.cuda.synchronize()
    xf, yf, df = x.float().numpy(), y.float().numpy(), dout.float().numpy()
    np.testing.assert_array_equal(gu.host(xp), mo.dispatch(xf, meta["perm_src"], k))
    tol = 1e-5 if dtype == torch.float32 else 1e-2
    assert gu.rel_err(gu.host(out), mo.combine(yf, g, meta["perm_dst"], k)) <= tol
    rdy, rdg = mo.combine_backward(df, yf, g, meta["perm_dst"], k)
    assert gu.rel_err(gu.host(dy), rdy) <= tol
    assert gu.rel_err(gu.host(dgt), rdg) <= 1e-5  # fp32 dots of exactly representable values
    assert gu.rel_err(gu.host(dx), mo.dispatch_backward(yf, meta["perm_dst"], k)) <= tol


def _mx_act_host(buf, R, d):
    """MX activation buffer -> (codes [R, d], scales [R, d/32] in the public row-major order)."""
    q, sg = B.mx_act_split(buf, R, d)
    q, sg = q.cpu().numpy(), sg.cpu().numpy()
    r = np.arange(R)[:, None]
    b = np.arange(d // 32)[None, :]
    return q, sg[((b // 4) * R + r) * 4 + b % 4]  # grouped byte of (row r, block b)


@pytest.mark.parametrize("T,d,E,k", [(333, 256, 8, 2), (1000, 2048, 128, 4), (77, 4096, 16, 8), (5, 128, 4, 1)])
def test_dispatch_and_combine_bwd_mx_bit_exact(gpu, T, d, E, k):
    """The MX-writing dispatch and combine backward: bf16 outputs identical to the plain calls, E4M3 codes and
    E8M0 scales identical to the oracle's quantiser applied to those bf16 rows."""
    gu.say(f"case permute MX T={T} d={d} E={E} k={k}")
    r = np.random.default_rng(7 + T + d)
    lg = r.standard_normal((T, E)).astype(np.float32)
    idx = mo.topk_select(lg, k)
    meta = mo.routing_metadata(idx, E)
    g = mo.topk_gates(lg, idx).astype(np.float32)
    scale = np.exp2(r.integers(-20, 20, (T, 1))).astype(np.float32)  # a spread of block exponents
    x = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32) * scale).to(torch.bfloat16)
    y = torch.randn((T * k, d), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    dout = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32) * scale).to(torch.bfloat16)
    pd = torch.from_numpy(meta["perm_dst"]).cuda()
    gd = torch.from_numpy(g).cuda()
    xd, yd, dd = x.cuda(), y.cuda(), dout.cuda()
    xp_ref = B.moe_dispatch(xd, pd, k)
    dy_ref, dg_ref = B.moe_combine_bwd(dd, yd, gd, pd)
    xp, xmx = B.moe_dispatch_mx(xd, pd, k)
    dy, dg, dymx = B.moe_combine_bwd_mx(dd, yd, gd, pd)
    torch.cuda.synchronize()
    R = T * k
    np.testing.assert_array_equal(gu.host(xp), gu.host(xp_ref))
    np.testing.assert_array_equal(gu.host(dy), gu.host(dy_ref))
    np.testing.assert_array_equal(dg.cpu().numpy(), dg_ref.cpu().numpy())
    for buf, rows in ((xmx, xp), (dymx, dy)):
        q, sc = _mx_act_host(buf, R, d)
        rq, rs = mxo.mx_quantize(rows.float().cpu().numpy().astype(np.float64), axis=1)
        np.testing.assert_array_equal(q, rq)
        np.testing.assert_array_equal(sc, rs)


def _mx_tok_host(buf, R, E, d):
    """(codes [d, Rp], scale bytes [Rp/32, d]) of a token-axis MX buffer, scales ungrouped."""
    q, sc = B.mx_tok_split(buf, R, E, d)
    rp = q.shape[1]
    sc = sc.cpu().numpy().reshape(rp // 128, d, 4).transpose(0, 2, 1).reshape(rp // 32, d)
    return q.cpu().numpy(), sc


def _check_tok_layout(q, sc, rows, offsets, blk):
    """Token-axis codes and scales against the oracle's segment quantiser of the bf16 expert rows: expert e's
    blocks at positions [32 blk[e], 32 blk[e+1]), each block's tail and every position past the last block zero."""
    rq, rs = mxo.mx_quantize(rows.astype(np.float64), axis=0, seg_offsets=offsets)
    b = 0
    for e in range(len(offsets) - 1):
        lo, hi = offsets[e], offsets[e + 1]
        assert blk[e] == b
        for j in range(-(-(hi - lo) // 32)):
            r0, r1 = lo + 32 * j, min(lo + 32 * j + 32, hi)
            np.testing.assert_array_equal(q[:, 32 * b: 32 * b + (r1 - r0)], rq[r0:r1].T)
            assert np.all(q[:, 32 * b + (r1 - r0): 32 * (b + 1)] == 0)
            np.testing.assert_array_equal(sc[b], rs[b])
            b += 1
    assert b == len(rs) == blk[-1]
    assert np.all(q[:, 32 * b:] == 0) and np.all(sc[b:] == 0)


# (T, d, E, k, hot): hot routes most tokens to expert 0 and leaves experts empty
TOK_CASES = [(333, 256, 8, 2, False), (1000, 2048, 128, 4, False), (77, 4096, 16, 8, False), (5, 128, 4, 1, False),
             (700, 384, 32, 4, True), (64, 128, 1, 1, False)]


@pytest.mark.parametrize("T,d,E,k,hot", TOK_CASES)
def test_dispatch_and_combine_bwd_mx_tok_bit_exact(gpu, T, d, E, k, hot):
    """The token-axis MX calls: the bf16 rows they can write equal the plain dispatch and combine backward's,
    dgates equals the combine backward's, and both MX layouts equal the oracle's quantiser applied to those rows
    (rows layout along d; token-axis layout down each expert segment, zero-padded)."""
    gu.say(f"case permute MX tok T={T} d={d} E={E} k={k} hot={hot}")
    r = np.random.default_rng(11 + T + d + E)
    lg = r.standard_normal((T, E)).astype(np.float32)
    if hot:
        lg[:, 0] += 3.0
        lg[:, E // 2:] -= 30.0        # half the experts never chosen
    logits = torch.from_numpy(lg).cuda()
    route = B.moe_route_topk(logits, k)
    scale = np.exp2(r.integers(-20, 20, (T, 1))).astype(np.float32)
    x = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32) * scale).to(torch.bfloat16).cuda()
    y = torch.randn((T * k, d), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    dout = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32) * scale).to(torch.bfloat16).cuda()
    xp_ref = B.moe_dispatch(x, route["perm_dst"], k)
    dy_ref, dg_ref = B.moe_combine_bwd(dout, y, route["gates"], route["perm_dst"])
    xp, xmx, xmxt = B.moe_dispatch_mx_tok(x, route, k, E, write_rows=True)
    dy, dg, dymx, dymxt = B.moe_combine_bwd_mx_tok(dout, y, route["gates"], route, E, write_rows=True)
    # without the bf16 rows: the same MX bytes
    _, xmx2, xmxt2 = B.moe_dispatch_mx_tok(x, route, k, E)
    _, dg2, dymx2, dymxt2 = B.moe_combine_bwd_mx_tok(dout, y, route["gates"], route, E)
    torch.cuda.synchronize()
    R = T * k
    np.testing.assert_array_equal(gu.host(xp), gu.host(xp_ref))
    np.testing.assert_array_equal(gu.host(dy), gu.host(dy_ref))
    np.testing.assert_array_equal(dg.cpu().numpy(), dg_ref.cpu().numpy())
    np.testing.assert_array_equal(dg2.cpu().numpy(), dg_ref.cpu().numpy())
    for a, b in ((xmx, xmx2), (dymx, dymx2)):   # codes and scales (not the alignment gap between them)
        for va, vb in zip(B.mx_act_split(a, R, d), B.mx_act_split(b, R, d)):
            assert torch.equal(va, vb)
    for a, b in ((xmxt, xmxt2), (dymxt, dymxt2)):
        for va, vb in zip(B.mx_tok_split(a, R, E, d), B.mx_tok_split(b, R, E, d)):
            assert torch.equal(va, vb)
    offsets = route["offsets"].cpu().numpy()
    blk = route["mx_blk_offsets"].cpu().numpy()
    for mx, mxt, rows in ((xmx, xmxt, xp), (dymx, dymxt, dy)):
        rows = rows.float().cpu().numpy()
        q, sc = _mx_act_host(mx, R, d)
        rq, rs = mxo.mx_quantize(rows.astype(np.float64), axis=1)
        np.testing.assert_array_equal(q, rq)
        np.testing.assert_array_equal(sc, rs)
        _check_tok_layout(*_mx_tok_host(mxt, R, E, d), rows, offsets, blk)


# (T, d, E, accumulate): E <= 8 and E <= 16 take the LDS-staged kernels (d not a
# multiple of 512 leaves a partly filled feature group), E = 24 the generic ones
ROUTER_CASES = [(700, 256, 8, True), (1000, 520, 6, False), (333, 1024, 16, True), (300, 264, 24, True),
                (1, 64, 3, False), (4099, 2048, 8, True)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", ROUTER_CASES, ids=lambda c: f"T{c[0]}-d{c[1]}-E{c[2]}-acc{int(c[3])}")
def test_router_logits_and_backward(gpu, dtype, case):
    T, d, E, acc = case
    print(f"router T={T} d={d} E={E} accumulate={acc} {dtype}", flush=True)
    r = np.random.default_rng(5 + T + d + E)
    x = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(dtype)
    w = torch.from_numpy((r.standard_normal((d, E)) * 0.02).astype(np.float32)).to(dtype)
    dl = torch.from_numpy(r.standard_normal((T, E)).astype(np.float32))
    dx0 = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(dtype)
    xd, wd_, dld = x.cuda(), w.cuda(), dl.cuda()
    lg = B.moe_router_logits(xd, wd_)
    dx = dx0.cuda()
    dw = B.moe_router_logits_bwd(xd, wd_, dld, dx, accumulate_dx=acc)
    torch.cuda.synchronize()
    xf, wf = x.float().numpy(), w.float().numpy()
    err = gu.rel_err(gu.host(lg), mo.router_logits(xf, wf))
    print(f"  logits rel err {err:.2e}", flush=True)
    assert err <= 1e-5
    rdx, rdw = mo.router_logits_backward(xf, wf, dl.numpy())
    tol = 1e-5 if dtype == torch.float32 else 1e-2
    want_dx = (dx0.float().numpy() + rdx) if acc else rdx
    assert gu.rel_err(gu.host(dx), want_dx) <= tol
    assert gu.rel_err(gu.host(dw), rdw) <= tol


def _mx_input(shape, seed, dtype):
    r = np.random.default_rng(seed)
    v = (r.standard_normal(shape) * np.exp2(r.integers(-30, 30, shape[:-1] + (1,)))).astype(np.float32)
    flat = v.reshape(-1)
    flat[::97] = 0.0
    flat[1::101] = -0.0
    flat[2::53] *= 2.0 ** -100          # tiny values next to large ones in a block
    if dtype == torch.float32:
        flat[3::211] = 1.0e-40          # fp32 subnormals
    t = torch.from_numpy(v).to(dtype)
    return t, t.float().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mx_quantize_rows_bit_exact(gpu, dtype):
    t, v = _mx_input((257, 512), 1, dtype)
    q, s = B.mx_quantize(t.cuda(), axis=1)
    torch.cuda.synchronize()
    rq, rs = mxo.mx_quantize(v, axis=1)
    np.testing.assert_array_equal(q[0].cpu().numpy(), rq)
    np.testing.assert_array_equal(s[0].cpu().numpy(), rs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mx_quantize_cols_batched_bit_exact(gpu, dtype):
    t, v = _mx_input((3, 96, 264), 2, dtype)
    q, s = B.mx_quantize(t.cuda(), axis=0)
    torch.cuda.synchronize()
    for b in range(3):
        rq, rs = mxo.mx_quantize(v[b], axis=0)
        np.testing.assert_array_equal(q[b].cpu().numpy(), rq.T)       # stored transposed
        np.testing.assert_array_equal(s[b].cpu().numpy(), rs.T)


def _e4m3_rounding_cases(seed=11):
    """fp32 values below 512 in magnitude around every E4M3 rounding decision:
    each grid value and each midpoint between neighbours (ties to even), the
    saturation range above 448, the subnormal floor 2^-10, three fp32 ulps to
    either side of all of those, both signs; plus random fp32 patterns."""
    g = mxo.e4m3_decode(np.arange(0x7F))
    pts = np.concatenate([g, (g[:-1] + g[1:]) / 2, [456.0, 464.0, 480.0, 500.0, 2.0 ** -10, 1.5 * 2.0 ** -10]])
    u = pts.astype(np.float32).view(np.uint32).astype(np.int64)
    near = (u[:, None] + np.arange(-3, 4)[None, :]).reshape(-1)
    near = near[(near >= 0) & (near < 0x44000000)]
    rnd = np.random.default_rng(seed).integers(0, 0x44000000, 1 << 20)
    bits = np.concatenate([near, rnd]).astype(np.uint32)
    sign = np.random.default_rng(seed + 1).integers(0, 2, bits.size).astype(np.uint32) << 31
    both = np.concatenate([bits, bits | np.uint32(0x80000000), bits ^ sign])
    return both.view(np.float32)


@pytest.mark.parametrize("axis", [1, 0])
def test_mx_quantize_rounding_boundaries(gpu, axis):
    """Blocks [256, 31 cases]: the block exponent is 0, so every case is encoded
    unscaled; codes and scales bit-exact against the oracle."""
    vals = _e4m3_rounding_cases()
    nblk = -(-vals.size // 31 // 8) * 8  # the column layout wants a multiple of 8 columns
    blocks = np.zeros((nblk, 32), np.float32)
    blocks[:, 0] = 256.0
    blocks.reshape(-1)[np.flatnonzero(np.arange(nblk * 32) % 32)[:vals.size]] = vals
    m = blocks if axis == 1 else np.ascontiguousarray(blocks.T)
    q, s = B.mx_quantize(torch.from_numpy(m).cuda(), axis=axis)
    torch.cuda.synchronize()
    rq, rs = mxo.mx_quantize(m.astype(np.float64), axis=axis)
    assert np.all(rs == 127)
    if axis == 0:
        rq, rs = rq.T, rs.T  # stored transposed
    np.testing.assert_array_equal(q[0].cpu().numpy(), rq)
    np.testing.assert_array_equal(s[0].cpu().numpy(), rs)


def test_mx_quantize_segments_bit_exact(gpu):
    t, v = _mx_input((500, 136), 3, torch.bfloat16)
    seg = np.array([0, 0, 45, 45, 77, 300, 301, 500], np.int32)
    nseg = len(seg) - 1
    rp = 32 * (-(-500 // 32) + nseg)
    # outputs pre-filled with 0xFF so that unwritten bytes show
    q0 = torch.full((136, rp), 0xFF, dtype=torch.uint8, device="cuda")
    s0 = torch.full((136, rp // 32), 0xFF, dtype=torch.uint8, device="cuda")
    q, s = B.mx_quantize(t.cuda(), axis=0, seg_offsets=torch.from_numpy(seg).cuda(), nseg=nseg, q=q0, scales=s0)
    torch.cuda.synchronize()
    rq, rs = mxo.mx_quantize(v, axis=0, seg_offsets=seg)
    q, s = q.cpu().numpy(), s.cpu().numpy()
    b = 0
    for i in range(nseg):
        lo, hi = seg[i], seg[i + 1]
        nb = (hi - lo + 31) // 32
        for j in range(nb):
            r0, r1 = lo + 32 * j, min(lo + 32 * j + 32, hi)
            np.testing.assert_array_equal(q[:, 32 * b: 32 * b + (r1 - r0)], rq[r0:r1].T)
            assert np.all(q[:, 32 * b + (r1 - r0): 32 * (b + 1)] == 0)   # zero padding
            np.testing.assert_array_equal(s[:, b], rs[b])
            b += 1
    assert b == len(rs)
    assert np.all(q[:, 32 * b:] == 0) and np.all(s[:, b:] == 0)   # padding past the last segment


def _wcache_regions(E, d, f):
    """Byte ranges of the weight cache as its header documents them: six regions
    (w_gate, w_up, w_down forward, then the same three backward), each the E4M3
    codes followed by the scale bytes, every part starting on a 256-byte boundary."""
    up = lambda n: -(-n // 256) * 256
    n, off, out = E * d * f, 0, []
    for _ in range(6):
        out.append((off, off + n, off + up(n), off + up(n) + n // 32))
        off += up(n) + up(n // 32)
    return out, off


def _wcache_check(cache, reg, wts, E, forward):
    """One region against the oracle: forward codes are each expert's weight
    quantised down its rows and stored transposed, scales grouped per expert
    ([K/128][M][4] bytes, M = output rows, K = the blocked axis); backward codes
    keep the weight's shape, blocks along its last axis, scales grouped over all
    experts' rows ([K/128][E*M][4])."""
    q0, q1, s0, s1 = reg
    m_rows = wts.shape[2] if forward else wts.shape[1]
    k_len = wts.shape[1] if forward else wts.shape[2]
    codes = cache[q0:q1].reshape(E, m_rows, k_len)
    sc = cache[s0:s1]
    nb = k_len // 32
    b = np.arange(nb)
    for e in range(E):
        rq, rs = mxo.mx_quantize(wts[e], axis=0 if forward else 1)
        if forward:
            np.testing.assert_array_equal(codes[e], rq.T)
            m = np.arange(m_rows)[:, None]
            idx = e * m_rows * nb + ((b[None, :] // 4) * m_rows + m) * 4 + b[None, :] % 4
            np.testing.assert_array_equal(sc[idx], rs.T)          # rs [nb, M]
        else:
            np.testing.assert_array_equal(codes[e], rq)
            m = np.arange(m_rows)[:, None]
            idx = ((b[None, :] // 4) * E * m_rows + e * m_rows + m) * 4 + b[None, :] % 4
            np.testing.assert_array_equal(sc[idx], rs)            # rs [M, nb]


@pytest.mark.parametrize("E,d,f", [(3, 256, 384), (2, 128, 128), (1, 512, 256)])
def test_mx_weight_cache_bit_exact(gpu, E, d, f):
    """Both orientations of every weight in the cache (one read of each weight
    feeds both) against the oracle's MX encoding, bit for bit, in the layout the
    header documents; rows of very different magnitude share column blocks."""
    gu.say(f"case mx weight cache E={E} d={d} f={f}")
    wg, vg = _mx_input((E, d, f), 21, torch.bfloat16)
    wu, vu = _mx_input((E, d, f), 22, torch.bfloat16)
    wd, vd = _mx_input((E, f, d), 23, torch.bfloat16)
    vg[0, :32, :32] = 0.0                                         # an all-zero block in both orientations
    wg[0, :32, :32] = 0.0
    regions, total = _wcache_regions(E, d, f)
    assert B.lib().moe_mx_weight_cache_bytes(E, d, f) == total
    cache = torch.full((total,), 0xFF, dtype=torch.uint8, device="cuda")
    B.moe_mx_weight_cache_build(wg.cuda(), wu.cuda(), wd.cuda(), cache=cache)
    torch.cuda.synchronize()
    c = cache.cpu().numpy()
    for i, (v, fwd) in enumerate([(vg, True), (vu, True), (vd, True), (vg, False), (vu, False), (vd, False)]):
        _wcache_check(c, regions[i], v, E, fwd)
