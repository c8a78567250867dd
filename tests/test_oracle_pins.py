"""Pins that tie the CPU oracle to something other than itself (CPU only).

Each check compares the oracle with an independent statement of the same
mathematics: pure-Python brute force on tiny inputs, a dense all-experts
evaluation with no permutation, library routines for special cases that reduce
to a textbook operation (scipy's softmax and logistic function), central finite
differences for every gradient, and the E4M3 / MX format definitions (hand
vectors in tests/golden, exhaustive code round trip, brute-force nearest-even).
``test_oracle_mutations.py`` plants mistakes in the oracle and checks that these
helpers catch them.
"""
import itertools
import os

import numpy as np
import pytest
import scipy.special

from oracle import moe_oracle as mo
from oracle import mx_oracle as mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# small random problems
# ---------------------------------------------------------------------------

def tiny_problem(seed, T, d, E, k, f, router=True):
    r = np.random.default_rng(seed)
    p = {
        "x": r.standard_normal((T, d)),
        "w_gate": r.standard_normal((E, d, f)) * 0.3,
        "w_up": r.standard_normal((E, d, f)) * 0.3,
        "w_down": r.standard_normal((E, f, d)) * 0.3,
        "dout": r.standard_normal((T, d)),
        "k": k,
    }
    if router:
        p["w_router"] = r.standard_normal((d, E)) * 0.5
    else:
        p["logits"] = r.standard_normal((T, E)).astype(np.float32)
    return p


def adversarial_logits(T, E, seed=0):
    """Rows full of ties: integer values, all-equal rows, +-0.0 mixes."""
    r = np.random.default_rng(seed)
    rows = []
    rows.append(np.zeros(E, np.float32))                       # all equal
    rows.append(np.full(E, 3.5, np.float32))
    z = np.zeros(E, np.float32)
    z[::2] = -0.0
    rows.append(z)                                             # +-0.0 mix
    rows.append(np.where(np.arange(E) % 3 == 0, -0.0, 0.0).astype(np.float32))
    one_hot = np.full(E, -1.0, np.float32)
    one_hot[E - 1] = 5.0
    rows.append(one_hot)
    while len(rows) < T:
        rows.append(r.integers(-2, 3, E).astype(np.float32))  # many exact ties
    return np.stack(rows[:T])


# ---------------------------------------------------------------------------
# O1 top-k selection: brute force per token
# ---------------------------------------------------------------------------

def brute_topk(logits, k):
    out = []
    for row in np.asarray(logits, np.float32):
        vals = [float(v) for v in row]
        # NaN ranks below every number, NaNs among themselves by index
        order = sorted(range(len(vals)), key=lambda e: (vals[e] != vals[e], 0.0 if vals[e] != vals[e] else -vals[e], e))
        out.append(order[:k])
    return np.array(out, dtype=np.int32)


def check_topk(topk_fn):
    r = np.random.default_rng(1)
    for E, k in [(8, 2), (8, 4), (16, 4), (5, 5), (1, 1), (32, 8)]:
        cases = [r.standard_normal((64, E)).astype(np.float32), adversarial_logits(64, E, seed=E)]
        for lg in cases:
            np.testing.assert_array_equal(topk_fn(lg, k), brute_topk(lg, k))


def test_topk_matches_bruteforce():
    check_topk(mo.topk_select)


def test_topk_nan_ranks_below_every_number():
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    lg = np.array([[nan, -inf, 0.5, nan, -3.0],
                   [nan, nan, nan, nan, nan],
                   [1.0, nan, -inf, nan, 2.0]], np.float32)
    np.testing.assert_array_equal(mo.topk_select(lg, 4), [[2, 4, 1, 0], [0, 1, 2, 3], [4, 0, 2, 1]])
    r = np.random.default_rng(5)
    for E, k in [(8, 4), (16, 8), (5, 5)]:
        lg = r.standard_normal((200, E)).astype(np.float32)
        lg[r.random((200, E)) < 0.3] = np.nan
        lg[r.random((200, E)) < 0.05] = -np.inf
        np.testing.assert_array_equal(mo.topk_select(lg, k), brute_topk(lg, k))


def test_topk_signed_zero_tie_goes_to_lower_index():
    lg = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    np.testing.assert_array_equal(mo.topk_select(lg, 2), [[0, 1]])
    lg = np.array([[0.0, -0.0, -1.0, 0.0]], np.float32)
    np.testing.assert_array_equal(mo.topk_select(lg, 3), [[0, 1, 3]])


# ---------------------------------------------------------------------------
# O2 gates
# ---------------------------------------------------------------------------

def check_gates(gates_fn, topk_fn=mo.topk_select):
    r = np.random.default_rng(2)
    lg = r.standard_normal((128, 16)).astype(np.float32) * 3
    for k in (1, 2, 4, 16):
        idx = topk_fn(lg, k)
        g = gates_fn(lg, idx)
        assert np.all(np.abs(g.sum(axis=1) - 1.0) < 1e-14)
        assert np.all(np.diff(g, axis=1) <= 0.0)
        if k == 1:
            assert np.all(g == 1.0)
        if k == 16:
            # k = E: the gates are the textbook softmax over all experts, in slot order
            ref = scipy.special.softmax(lg.astype(np.float64), axis=1)
            np.testing.assert_allclose(g, np.take_along_axis(ref, idx.astype(np.int64), axis=1),
                                       rtol=1e-13, atol=0)
        # general k: softmax over all E, restricted to the chosen set, renormalised
        full = scipy.special.softmax(lg.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
        np.testing.assert_allclose(g, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)


def test_gates_properties():
    check_gates(mo.topk_gates)


# ---------------------------------------------------------------------------
# O3/O4 metadata and permutation
# ---------------------------------------------------------------------------

def brute_metadata(idx, E):
    T, k = idx.shape
    pairs = sorted((int(idx[t, j]), t, t * k + j) for t in range(T) for j in range(k))
    perm_src = np.array([p[2] for p in pairs], np.int32)
    counts = np.array([sum(1 for p in pairs if p[0] == e) for e in range(E)], np.int32)
    return perm_src, counts


def check_metadata(meta_fn):
    r = np.random.default_rng(3)
    for T, E, k in [(50, 8, 2), (64, 4, 4), (33, 1, 1), (40, 16, 3)]:
        lg = r.standard_normal((T, E)).astype(np.float32)
        idx = mo.topk_select(lg, k)
        m = meta_fn(idx, E)
        R = T * k
        ps, counts = brute_metadata(idx, E)
        np.testing.assert_array_equal(m["perm_src"], ps)
        np.testing.assert_array_equal(m["counts"], counts)
        assert m["counts"].sum() == R
        assert m["offsets"][0] == 0 and m["offsets"][-1] == R
        assert np.all(np.diff(m["offsets"]) >= 0)
        np.testing.assert_array_equal(np.diff(m["offsets"]), m["counts"])
        # bijection: perm_dst o perm_src = id
        np.testing.assert_array_equal(m["perm_dst"][m["perm_src"]], np.arange(R))
        np.testing.assert_array_equal(np.sort(m["perm_src"]), np.arange(R))
        # within each segment: the expert matches and tokens strictly increase
        for e in range(E):
            seg = m["perm_src"][m["offsets"][e]:m["offsets"][e + 1]]
            assert np.all(idx.reshape(-1)[seg] == e)
            assert np.all(np.diff(seg // k) > 0)
        blocks = (m["counts"] + 31) // 32
        np.testing.assert_array_equal(np.diff(m["mx_blk_offsets"]), blocks)
        if E == 1 and k == 1:
            np.testing.assert_array_equal(m["perm_src"], np.arange(R))
        if k == E:
            assert np.all(m["counts"] == T)


def test_metadata_bruteforce_and_invariants():
    check_metadata(mo.routing_metadata)


# ---------------------------------------------------------------------------
# O5-O7 forward: dense all-experts evaluation with a top-k mask, no permutation
# ---------------------------------------------------------------------------

def textbook_swiglu(x, wg, wu, wd):
    hg = x @ wg
    return (hg * scipy.special.expit(hg) * (x @ wu)) @ wd


def dense_moe(p):
    x = p["x"]
    E = p["w_gate"].shape[0]
    lg = x @ p["w_router"] if "w_router" in p else p["logits"].astype(np.float64)
    T = x.shape[0]
    out = np.zeros_like(x)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(np.float32(lg[t, e])), e))[:p["k"]]
        z = np.exp(lg[t, order] - lg[t, order].max())
        gate = z / z.sum()
        for e in range(E):
            if e in order:
                m = gate[order.index(e)]
                out[t] += m * textbook_swiglu(x[t:t + 1], p["w_gate"][e], p["w_up"][e], p["w_down"][e])[0]
    return out


def oracle_out(p, oracle=mo):
    res = oracle.layer_forward_backward(p["x"], p["w_gate"], p["w_up"], p["w_down"], p["dout"], p["k"],
                                        logits=p.get("logits"), w_router=p.get("w_router"))
    return res


def check_forward(layer_fn):
    for seed, (T, d, E, k, f, router) in enumerate([(37, 16, 5, 2, 24, True), (20, 8, 4, 4, 12, False),
                                                    (16, 8, 1, 1, 8, True), (25, 12, 6, 3, 10, False)]):
        p = tiny_problem(seed, T, d, E, k, f, router)
        got = layer_fn(p)["out"]
        ref = dense_moe(p)
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_routing_stats_hand_example_and_special_cases():
    # four tokens, top-2 of five experts, counted by hand: expert 0 gets 4 rows, 1 gets 2, 2 and 3 one
    # each, 4 none
    idx = np.array([[0, 1], [0, 2], [0, 1], [3, 0]])
    counts = mo.routing_metadata(idx, 5)["counts"]
    assert counts.tolist() == [4, 2, 1, 1, 0]
    assert mo.routing_stats(counts).tolist() == [4, 0, 1, 8]
    # one expert takes every row; k = E spreads every token over all experts
    assert mo.routing_stats([12]).tolist() == [12, 12, 0, 12]
    full = mo.routing_metadata(np.tile(np.arange(6), (7, 1)), 6)["counts"]
    assert mo.routing_stats(full).tolist() == [7, 7, 0, 42]


def test_forward_matches_dense_bruteforce():
    check_forward(oracle_out)


def test_single_expert_is_dense_swiglu_ffn():
    p = tiny_problem(11, 30, 16, 1, 1, 20, router=True)
    got = oracle_out(p)["out"]
    ref = textbook_swiglu(p["x"], p["w_gate"][0], p["w_up"][0], p["w_down"][0])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_k_equals_E_is_soft_moe():
    p = tiny_problem(12, 20, 8, 4, 4, 12, router=False)
    got = oracle_out(p)["out"]
    w = scipy.special.softmax(p["logits"].astype(np.float64), axis=1)
    ref = sum(w[:, e:e + 1] * textbook_swiglu(p["x"], p["w_gate"][e], p["w_up"][e], p["w_down"][e])
              for e in range(4))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# O8 backward: central finite differences of L = sum(out * dout)
# ---------------------------------------------------------------------------

def loss_and_route(p, layer_fn):
    res = layer_fn(p)
    return float(np.sum(res["out"] * p["dout"])), res["topk_idx"]


def check_backward(layer_fn, n_entries=25, seed=5):
    p = tiny_problem(seed, 24, 8, 4, 2, 12, router=True)
    res = layer_fn(p)
    grads = {"x": res["dx"], "w_router": res["dw_router"], "w_gate": res["dw_gate"],
             "w_up": res["dw_up"], "w_down": res["dw_down"]}
    r = np.random.default_rng(seed)
    for name, g_an in grads.items():
        theta = p[name]
        scale = np.max(np.abs(g_an))
        assert scale > 0
        checked = 0
        for _ in range(4 * n_entries):
            if checked == n_entries:
                break
            pos = tuple(int(r.integers(0, s)) for s in theta.shape)
            h = 1e-6 * max(1.0, abs(theta[pos]))
            orig = theta[pos]
            theta[pos] = orig + h
            lp, ip = loss_and_route(p, layer_fn)
            theta[pos] = orig - h
            lm, im = loss_and_route(p, layer_fn)
            theta[pos] = orig
            if not np.array_equal(ip, im):
                continue  # the chosen set changed inside [theta-h, theta+h]: redraw
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g_an[pos]) <= 1e-6 * scale, (name, pos, fd, g_an[pos])
            checked += 1
        assert checked == n_entries


def test_backward_finite_differences():
    check_backward(oracle_out)


def test_dlogits_invariants():
    p = tiny_problem(6, 40, 8, 6, 3, 10, router=False)
    res = oracle_out(p)
    dl = res["dlogits"]
    idx = res["topk_idx"].astype(np.int64)
    sel = np.take_along_axis(dl, idx, axis=1)
    assert np.all(np.abs(sel.sum(axis=1)) <= 1e-14 * max(1.0, np.abs(sel).max()))
    mask = np.ones_like(dl, bool)
    np.put_along_axis(mask, idx, False, axis=1)
    assert np.all(dl[mask] == 0.0)
    p1 = tiny_problem(7, 16, 8, 1, 1, 8, router=False)
    assert np.all(oracle_out(p1)["dlogits"] == 0.0)


def test_combine_backward_dgates_matches_fd():
    # dgates by finite differences of L through the combine alone (gates as free inputs)
    r = np.random.default_rng(8)
    T, k, d = 10, 3, 6
    Y = r.standard_normal((T * k, d))
    g = r.random((T, k))
    dout = r.standard_normal((T, d))
    perm_dst = r.permutation(T * k).astype(np.int32)
    _, dg = mo.combine_backward(dout, Y, g, perm_dst, k)
    for t, j in itertools.product(range(T), range(k)):
        h = 1e-6
        gp = g.copy(); gp[t, j] += h
        gm = g.copy(); gm[t, j] -= h
        fd = (np.sum(mo.combine(Y, gp, perm_dst, k) * dout) - np.sum(mo.combine(Y, gm, perm_dst, k) * dout)) / (2 * h)
        assert abs(fd - dg[t, j]) < 1e-7


# ---------------------------------------------------------------------------
# O9 MXFP8: format definition pins
# ---------------------------------------------------------------------------

FINITE_CODES = [c for c in range(256) if (c & 0x7F) != 0x7F]


def e4m3_value_by_definition(c):
    s = -1.0 if c & 0x80 else 1.0
    E, m = (c >> 3) & 15, c & 7
    return s * (m * 2.0 ** -9 if E == 0 else 2.0 ** (E - 7) * (1 + m / 8))


def test_e4m3_decode_definition():
    for c in FINITE_CODES:
        assert mx.e4m3_decode(np.array([c]))[0] == e4m3_value_by_definition(c)
    assert np.isnan(mx.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert mx.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert mx.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert mx.e4m3_decode(np.array([0x38]))[0] == 1.0


def check_encode(encode_fn):
    # exhaustive round trip over every finite code (both zeros included)
    vals = np.array([e4m3_value_by_definition(c) for c in FINITE_CODES])
    vals[FINITE_CODES.index(0x80)] = -0.0
    np.testing.assert_array_equal(encode_fn(vals), np.array(FINITE_CODES, np.uint8))
    # brute force nearest, ties to even code, saturation above 448
    grid = np.array([e4m3_value_by_definition(c) for c in range(0x7F)])  # codes 0..126, ascending
    r = np.random.default_rng(9)
    ys = np.concatenate([
        r.standard_normal(4000) * np.exp2(r.integers(-12, 10, 4000)),
        (grid[:-1] + grid[1:]) / 2,                  # exact midpoints
        -(grid[:-1] + grid[1:]) / 2,
        [449.0, 464.0, 480.0, 1e6, -1e6, 2.0 ** -11, -2.0 ** -11],
    ])
    got = encode_fn(ys)
    for y, c in zip(ys, got):
        a = abs(y)
        if a >= 448:
            want = 0x7E
        else:
            dist = np.abs(grid - a)
            best = np.flatnonzero(dist == dist.min())
            want = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        if np.signbit(y):
            want |= 0x80
        assert c == want, (y, c, want)


def test_e4m3_encode_bruteforce():
    check_encode(mx.e4m3_encode)


def parse_value(tok):
    neg = tok.startswith("-")
    t = tok[1:] if neg else tok
    if "*" in t:
        a, b = t.split("*")
        v = float(a) * parse_value(b)
    elif t.startswith("2^"):
        v = 2.0 ** int(t[2:])
    else:
        v = float(t)
    return -v if neg else v


def load_hand_vectors():
    blocks = []
    with open(os.path.join(GOLDEN, "e4m3_mx_hand_vectors.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("block "):
                continue
            head, rest = line[len("block "):].split(":", 1)
            lhs, rhs = rest.split("->")
            elems = []
            for item in lhs.split():
                v, n = item.rsplit("x", 1)
                elems += [parse_value(v)] * int(n)
            assert len(elems) == 32
            sc_part, codes_part = rhs.split(";")
            scale = int(sc_part.split()[1], 16)
            expect = {}
            for item in codes_part.split():
                v, c = item.split("=")
                expect[parse_value(v)] = int(c, 16)
            blocks.append((head.strip(), np.array(elems), scale, expect))
    return blocks


def test_mx_hand_vectors():
    blocks = load_hand_vectors()
    assert len(blocks) >= 5
    for name, elems, scale, expect in blocks:
        q, s = mx.mx_quantize(elems[None, :], axis=1)
        assert s[0, 0] == scale, name
        for v, c in expect.items():
            i = int(np.flatnonzero(elems == v)[0])
            assert q[0, i] == c, (name, v, q[0, i], c)


def test_mx_scale_invariant_and_error_bound():
    r = np.random.default_rng(10)
    v = r.standard_normal((64, 256)) * np.exp2(r.integers(-20, 20, (64, 1)))
    q, s = mx.mx_quantize(v, axis=1)
    e = s.astype(np.int64) - 127
    amax = np.abs(v).reshape(64, 8, 32).max(axis=2)
    assert np.all(np.exp2(e + 8.0) <= amax) and np.all(amax < np.exp2(e + 9.0))
    deq = mx.mx_dequantize(q, s, axis=1)
    # half a grid step: 2^-4 relative for normals, 2^(e-10) absolute for subnormals;
    # scaled magnitudes in (448, 512) saturate to exactly 448 * 2^e
    se = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=1)
    sat = np.abs(v) / se > 448.0
    assert sat.any()
    step = np.maximum(np.abs(v) * 2.0 ** -4, se * 2.0 ** -10)
    assert np.all(np.abs(deq - v)[~sat] <= step[~sat])
    np.testing.assert_array_equal(deq[sat], np.sign(v[sat]) * 448.0 * se[sat])


def test_mx_axis0_segments_restart_and_pad():
    r = np.random.default_rng(11)
    rows, cols = 100, 64
    v = r.standard_normal((rows, cols))
    seg = [0, 0, 45, 45, 77, 100]
    q, s = mx.mx_quantize(v, axis=0, seg_offsets=seg)
    nblk = sum((seg[i + 1] - seg[i] + 31) // 32 for i in range(len(seg) - 1))
    assert s.shape == (nblk, cols)
    b = 0
    for i in range(len(seg) - 1):
        lo, hi = seg[i], seg[i + 1]
        for r0 in range(lo, hi, 32):
            r1 = min(r0 + 32, hi)
            blk = np.zeros((32, cols))
            blk[:r1 - r0] = v[r0:r1]
            qb, sb = mx.mx_quantize(blk.T, axis=1)  # same block along the other axis
            np.testing.assert_array_equal(s[b], sb[:, 0])
            np.testing.assert_array_equal(q[r0:r1], qb.T[:r1 - r0])
            b += 1
    atol = np.exp2(s.astype(np.float64).max() - 127 - 10)
    np.testing.assert_allclose(mx.mx_dequantize(q, s, axis=0, seg_offsets=seg), v, rtol=0.125, atol=atol)


# ---------------------------------------------------------------------------
# MXFP8 layer oracle: structure pins
# ---------------------------------------------------------------------------

def _mx_problem(seed=13, T=40, d=64, E=4, k=2, f=96):
    p = tiny_problem(seed, T, d, E, k, f, router=False)
    return p


def test_mx_layer_with_identity_encoding_is_the_plain_oracle(monkeypatch):
    from oracle import moe_mx_oracle as mxl
    p = _mx_problem()
    monkeypatch.setattr(mxl, "q_along", lambda v, axis, seg=None: np.asarray(v, np.float64))
    monkeypatch.setattr(mxl, "round_to_bf16", lambda v: np.asarray(v, np.float64))
    got = mxl.mx_layer_forward_backward(p["x"], p["w_gate"], p["w_up"], p["w_down"], p["dout"], p["k"],
                                        logits=p["logits"])
    ref = oracle_out(p)
    for key in ("out", "dgates", "dx", "dw_gate", "dw_up", "dw_down", "dlogits", "perm_src"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-12, err_msg=key)


def mx_quantisation_calls(layer_fn, p):
    """(shape, axis, segmented) of every MX encoding the layer oracle applies."""
    from oracle import moe_mx_oracle as mxl
    calls = []
    orig = mxl.q_along

    def rec(v, axis, seg=None):
        calls.append((tuple(np.shape(v)), axis, seg is not None))
        return orig(v, axis, seg)
    mxl.q_along = rec
    try:
        layer_fn(p)
    finally:
        mxl.q_along = orig
    return calls


def check_mx_axes(layer_fn):
    """Every GEMM operand is encoded along that GEMM's contraction axis (module
    table), in the order the steps run: forward, input gradients, weight gradients."""
    p = _mx_problem(T=80, d=64, E=2, k=1, f=96)
    idx = mo.topk_select(p["logits"], 1)
    n = np.bincount(idx.ravel(), minlength=2)
    assert n.min() > 0
    R, d, f = 80, 64, 96
    want = [((R, d), 1, False)]                                       # X along d (G1)
    for e in range(2):
        want += [((d, f), 0, False), ((d, f), 0, False)]              # Wg_e, Wu_e along d (G1)
    want += [((R, f), 1, False)]                                      # A along f (G2)
    want += [((f, d), 0, False)] * 2                                  # Wd_e along f (G2)
    want += [((R, d), 1, False)]                                      # dY along d (G3)
    want += [((f, d), 1, False)] * 2                                  # Wd_e along d (G3)
    want += [((R, f), 1, False), ((R, f), 1, False)]                  # dHg, dHu along f (G5)
    for e in range(2):
        ne = int(n[e])
        want += [((d, f), 1, False), ((d, f), 1, False)]              # Wg_e, Wu_e along f (G5)
        want += [((ne, d), 0, True), ((ne, f), 0, True), ((ne, d), 0, True),   # X_e, A_e, dY_e along tokens
                 ((ne, f), 0, True), ((ne, f), 0, True)]              # dHg_e, dHu_e along tokens (G4, G6)
    got = mx_quantisation_calls(layer_fn, p)
    assert got == want, (got, want)


def _mx_layer(p):
    from oracle import moe_mx_oracle as mxl
    return mxl.mx_layer_forward_backward(p["x"], p["w_gate"], p["w_up"], p["w_down"], p["dout"], p["k"],
                                         logits=p["logits"])


def test_mx_layer_quantises_along_contraction_axes():
    check_mx_axes(_mx_layer)


def test_mx_layer_error_is_the_encoding_error():
    # the MX layer differs from the plain oracle by an amount of the order of the
    # E4M3 rounding (a few percent), never by O(1)
    p = _mx_problem(T=200, d=128, E=4, k=2, f=128)
    got = _mx_layer(p)
    ref = oracle_out(p)
    for key in ("out", "dx", "dw_gate", "dw_down"):
        e = np.abs(got[key] - ref[key]).max() / np.abs(ref[key]).max()
        assert 1e-4 < e < 0.2, (key, e)


def test_round_to_bf16_matches_torch_conversion():
    import torch
    from oracle import moe_mx_oracle as mxl
    r = np.random.default_rng(21)
    v = np.concatenate([r.standard_normal(200000) * np.exp2(r.integers(-40, 40, 200000)),
                        [1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 2.0 ** -130, 3.0 * 2.0 ** -133]])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).double().numpy()
    got = mxl.round_to_bf16(v32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# MXFP8 layer oracle: the backward's recompute of the gate/up products
# ---------------------------------------------------------------------------

def _mx_segments(p):
    idx = mo.topk_select(p["logits"], p["k"])
    meta = mo.routing_metadata(idx, p["w_gate"].shape[0])
    X = mo.dispatch(np.asarray(p["x"], np.float64), meta["perm_src"], p["k"])
    dy, _ = mo.combine_backward(p["dout"], np.zeros_like(X), mo.topk_gates(p["logits"], idx), meta["perm_dst"],
                                p["k"])
    return X, dy, meta["offsets"]


def check_mx_recompute(mxl_mod):
    """The MX backward without saved forward tensors (fwd=None) recomputes Hg, Hu
    with G1 and must give the bits of the backward fed by the forward's own saved
    Hg, Hu, A; the recompute (mx_expert_ffn_forward_gate_up) must equal the
    forward's products before their bf16 store: rounding it gives the forward's
    stored h_gate, h_up exactly, and with the bf16 store made the identity the
    forward returns it unchanged.  An empty expert in the middle is included."""
    p = _mx_problem(seed=29, T=60, d=64, E=5, k=2, f=96)
    # one expert never chosen: its logit pushed below every other
    p["logits"] = p["logits"].copy()
    p["logits"][:, 2] = -1e30
    X, dy, off = _mx_segments(p)
    assert off[3] == off[2]
    wg, wu, wd = p["w_gate"], p["w_up"], p["w_down"]
    fwd = mxl_mod.mx_expert_ffn_forward(X, off, wg, wu, wd)
    hg, hu = mxl_mod.mx_expert_ffn_forward_gate_up(X, off, wg, wu)
    np.testing.assert_array_equal(mxl_mod.round_to_bf16(hg), fwd["h_gate"])
    np.testing.assert_array_equal(mxl_mod.round_to_bf16(hu), fwd["h_up"])
    orig = mxl_mod.round_to_bf16
    mxl_mod.round_to_bf16 = lambda v: np.asarray(v, np.float64)
    try:
        raw = mxl_mod.mx_expert_ffn_forward(X, off, wg, wu, wd)
    finally:
        mxl_mod.round_to_bf16 = orig
    np.testing.assert_array_equal(hg, raw["h_gate"])
    np.testing.assert_array_equal(hu, raw["h_up"])
    a = mxl_mod.mx_expert_ffn_backward(dy, X, off, wg, wu, wd, fwd=fwd)
    b = mxl_mod.mx_expert_ffn_backward(dy, X, off, wg, wu, wd, fwd=None)
    for key in ("dx_perm", "dw_gate", "dw_up", "dw_down"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_mx_backward_recompute_equals_saved_forward():
    from oracle import moe_mx_oracle as mxl
    check_mx_recompute(mxl)


def check_mx_recompute_axes(mxl_mod):
    """The recompute encodes X along d and each active expert's Wg, Wu along d,
    as the forward's G1 does (module table), and nothing else."""
    p = _mx_problem(T=80, d=64, E=2, k=1, f=96)
    X, _, off = _mx_segments(p)
    calls = []
    orig = mxl_mod.q_along

    def rec(v, axis, seg=None):
        calls.append((tuple(np.shape(v)), axis, seg is not None))
        return orig(v, axis, seg)
    mxl_mod.q_along = rec
    try:
        mxl_mod.mx_expert_ffn_forward_gate_up(X, off, p["w_gate"], p["w_up"])
    finally:
        mxl_mod.q_along = orig
    want = [((80, 64), 1, False)] + [((64, 96), 0, False)] * 4
    assert calls == want, (calls, want)


def test_mx_recompute_quantises_along_contraction_axes():
    from oracle import moe_mx_oracle as mxl
    check_mx_recompute_axes(mxl)
