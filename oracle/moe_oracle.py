"""CPU oracle for one GPU's share of an MoE layer, forward and backward (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` use it.  It shares no code with the HIP library and imports nothing
from the package.

Sources.  The method is the MoE training path described in the Ai2 announcement
"Introducing Olmo-core 3: open, scalable training infrastructure for large MoE
models" (read here in a Bulgarian translation), and the Georgian news summary of
the same announcement:

* section "Scaling and optimizing MoE training": tokens are routed to a few
  experts, routed rows are written directly into the experts' input buffers
  (row-wise expert parallelism), the routing metadata stays on the GPU, and the
  many small expert products are run as one grouped GEMM; MXFP8 is offered as a
  lower-precision format where it pays;
* introduction: four experts are chosen per token from a pool of 8 or 128.

The pages give no formula.  Where they are silent this module takes the plain
readings below (each one is also listed with its reason in the design notes):

* router: softmax over all experts, then top-k, then the k gates renormalised to
  sum to one.  Selection is done on the fp32 logits under the total order
  (logit descending, expert index ascending); the renormalised gates equal a
  softmax over the k selected logits because the full denominator cancels;
* expert FFN: SwiGLU without biases, ``A = silu(X Wg) * (X Wu)``, ``Y = A Wd``,
  weights stored as ``x @ W`` operands: Wg, Wu are [E, d, f], Wd is [E, f, d];
* dropless and unpadded: every routed row is computed;
* the gate multiplies the expert output in the combine, so the expert output
  buffer is unweighted;
* backward is the exact gradient of ``L = sum(out * dout)``; no gradient flows
  to unselected logits;
* MXFP8 (the pages give no detail): the public OCP Microscaling (MX) v1.0
  format, E4M3 elements with one E8M0 power-of-two scale per 32 consecutive
  elements along the contraction axis, scale exponent floor(log2(amax)) - 8,
  round-to-nearest-even, saturation to +-448.

Every floating-point result is computed in fp64 from the exact input values and
left in fp64; the tests round nothing on this side.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
brute force on tiny inputs, closed forms, library routines for special cases,
finite differences and format invariants.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Router: logits, top-k selection, renormalised gates, routing metadata.
# ----------------------------------------------------------------------------


def router_logits(x, w_r):
    """Router logits ``l = x @ W_r`` in fp64.

    Olmo-core 3 announcement, "Scaling and optimizing MoE training": tokens are
    routed to experts; the router is the plain linear map of the token
    activation onto one score per expert (no bias, no noise).
    x: [T, d], w_r: [d, E] -> [T, E] fp64.
    """
    return np.asarray(x, np.float64) @ np.asarray(w_r, np.float64)


def topk_select(logits, k):
    """Indices of the k chosen experts per token, in slot order.

    Olmo-core 3 announcement, introduction: a fixed number of experts (four in
    the 8->128 benchmark) is chosen per token.  Slot j holds the j-th expert
    under the total order (fp32 logit descending, expert index ascending).
    Values compare as fp32 numbers, so -0.0 and +0.0 tie and the lower index
    wins.  A NaN logit ranks below every number (-inf included) and NaNs among
    themselves by index, so the choice is defined for any input (the pages say
    nothing of non-finite scores; this is the reading taken).
    logits: [T, E] (compared as fp32) -> [T, k] int32.
    """
    l32 = np.asarray(logits, dtype=np.float32)
    if l32.ndim != 2 or not 1 <= k <= l32.shape[1]:
        raise ValueError("need logits [T, E] and 1 <= k <= E")
    # Negation is exact in fp32; a stable sort keeps ascending expert index
    # among equal values (and treats -0.0 == +0.0 as equal); numpy's sort puts
    # NaN after every number, in index order among NaNs.
    order = np.argsort(-l32, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_gates(logits, topk_idx):
    """Renormalised gates: softmax over all experts restricted to the chosen k.

    g[t, j] = exp(l[t, S_j] - l[t, S_0]) / sum_i exp(l[t, S_i] - l[t, S_0]).
    Equal to softmax over all E followed by renormalisation over the chosen set,
    since the full softmax denominator cancels.  The logits are used at the
    precision given (fp32 logits are upcast exactly).  Returns fp64 [T, k].
    """
    l64 = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(l64, np.asarray(topk_idx, np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def routing_metadata(topk_idx, num_experts):
    """Device-resident routing metadata, as a plain definition.

    Olmo-core 3 announcement, "Scaling and optimizing MoE training": routed rows
    go straight into the experts' input buffers and the routing metadata stays on
    the GPU.  The expert input buffer is expert-major: rows of expert e occupy
    [offsets[e], offsets[e+1]) and, inside a segment, appear in token order.

    Returns a dict of int32 arrays:
      counts[E]            rows routed to each expert
      offsets[E+1]         exclusive prefix sum of counts, offsets[E] = T*k
      perm_src[R]          buffer row r -> flat slot t*k+j it came from
      perm_dst[R]          flat slot t*k+j -> buffer row
      mx_blk_offsets[E+1]  prefix sum of ceil(counts/32): 32-row blocks per
                           expert segment for token-axis MX quantisation
    """
    idx = np.asarray(topk_idx, np.int64)
    T, k = idx.shape
    R = T * k
    flat_expert = idx.reshape(R)
    flat_token = np.arange(R, dtype=np.int64) // k
    counts = np.bincount(flat_expert, minlength=num_experts)
    if counts.shape[0] != num_experts:
        raise ValueError("expert index out of range")
    offsets = np.concatenate([[0], np.cumsum(counts)])
    # Sort the R (token, slot) pairs by the key (expert, token); np.lexsort
    # sorts by the last key first.  The key is unique (a token picks an expert
    # at most once), so the order is fully determined.
    perm_src = np.lexsort((flat_token, flat_expert))
    perm_dst = np.empty(R, dtype=np.int64)
    perm_dst[perm_src] = np.arange(R)
    blocks = (counts + 31) // 32
    mx_blk_offsets = np.concatenate([[0], np.cumsum(blocks)])
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "perm_src": perm_src.astype(np.int32),
        "perm_dst": perm_dst.astype(np.int32),
        "mx_blk_offsets": mx_blk_offsets.astype(np.int32),
    }


# ----------------------------------------------------------------------------
# Dispatch, expert FFN, combine (forward).
# ----------------------------------------------------------------------------


def routing_stats(counts):
    """Load statistics of one routing (Olmo-core 3 announcement, "Scaling to the
    trillion-parameter range": a balance metric can be gamed, so the observable
    per-expert load is what gets reported): [largest expert's rows, smallest
    expert's rows, number of experts with no rows, total rows]."""
    c = np.asarray(counts, np.int64)
    return np.array([c.max(), c.min(), int(np.sum(c == 0)), c.sum()], np.int64)


def dispatch(x, perm_src, k):
    """Row-wise dispatch: x_perm[r] = x[perm_src[r] // k] (an exact copy).

    Olmo-core 3 announcement, "Scaling and optimizing MoE training": routed data
    is placed directly in the experts' input buffers.
    """
    x = np.asarray(x)
    return x[np.asarray(perm_src, np.int64) // k].copy()


def silu(z):
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def expert_ffn_forward(x_perm, offsets, w_gate, w_up, w_down):
    """Grouped SwiGLU expert FFN over the expert-major buffer, in fp64.

    Olmo-core 3 announcement, "Scaling and optimizing MoE training": the many
    small per-expert products are one grouped GEMM.  Written here as the plain
    per-expert loop it is equivalent to.  For the rows of expert e:
      Hg = X_e Wg[e], Hu = X_e Wu[e], A = silu(Hg) * Hu, Y_e = A Wd[e].
    Returns dict h_gate, h_up, a_act [R, f] and y_perm [R, d] (fp64).
    """
    X = np.asarray(x_perm, np.float64)
    E, d, f = np.shape(w_gate)
    R = X.shape[0]
    hg = np.zeros((R, f))
    hu = np.zeros((R, f))
    a = np.zeros((R, f))
    y = np.zeros((R, d))
    for e in range(E):
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        if s.start == s.stop:
            continue
        # each expert's weights are converted to fp64 only when it has rows
        Wg, Wu, Wd = (np.asarray(w[e], np.float64) for w in (w_gate, w_up, w_down))
        hg[s] = X[s] @ Wg
        hu[s] = X[s] @ Wu
        a[s] = silu(hg[s]) * hu[s]
        y[s] = a[s] @ Wd
    return {"h_gate": hg, "h_up": hu, "a_act": a, "y_perm": y}


def combine(y_perm, gates, perm_dst, k):
    """Weighted un-permute: out[t] = sum_j g[t, j] * Y[perm_dst[t*k + j]].

    Summed in slot order j = 0..k-1, in fp64.
    """
    Y = np.asarray(y_perm, np.float64)
    g = np.asarray(gates, np.float64)
    T = g.shape[0]
    rows = np.asarray(perm_dst, np.int64).reshape(T, k)
    out = np.zeros((T, Y.shape[1]))
    for j in range(k):
        out += g[:, j:j + 1] * Y[rows[:, j]]
    return out


# ----------------------------------------------------------------------------
# Backward of L = sum(out * dout).
# ----------------------------------------------------------------------------


def combine_backward(dout, y_perm, gates, perm_dst, k):
    """dY[perm_dst[t*k+j]] = g[t,j] * dout[t];  dgates[t,j] = <dout[t], Y[row]>."""
    dO = np.asarray(dout, np.float64)
    Y = np.asarray(y_perm, np.float64)
    g = np.asarray(gates, np.float64)
    T = g.shape[0]
    rows = np.asarray(perm_dst, np.int64).reshape(T, k)
    dy = np.zeros_like(Y)
    dg = np.zeros((T, k))
    for j in range(k):
        dy[rows[:, j]] = g[:, j:j + 1] * dO
        dg[:, j] = np.einsum("td,td->t", dO, Y[rows[:, j]])
    return dy, dg


def expert_ffn_backward(dy_perm, x_perm, offsets, w_gate, w_up, w_down, want_dw=True):
    """Exact backward of the SwiGLU expert FFN, per expert segment (fp64).

    With s = sigmoid(Hg):
      dA = dY Wd^T,  dHu = dA * silu(Hg),  dHg = dA * Hu * s * (1 + Hg (1 - s)),
      dX = dHg Wg^T + dHu Wu^T,
      dWd = A^T dY,  dWg = X^T dHg,  dWu = X^T dHu   (zero for empty experts).
    The forward intermediates are recomputed here from X in fp64.  With
    want_dw=False the weight gradients are skipped (returned as None).
    """
    dY = np.asarray(dy_perm, np.float64)
    X = np.asarray(x_perm, np.float64)
    E, d, f = np.shape(w_gate)
    R = X.shape[0]
    dx = np.zeros((R, d))
    dwg = np.zeros((E, d, f)) if want_dw else None
    dwu = np.zeros((E, d, f)) if want_dw else None
    dwd = np.zeros((E, f, d)) if want_dw else None
    for e in range(E):
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        if s.start == s.stop:
            continue
        Wg, Wu, Wd = (np.asarray(w[e], np.float64) for w in (w_gate, w_up, w_down))
        hg = X[s] @ Wg
        hu = X[s] @ Wu
        sg = sigmoid(hg)
        a = hg * sg * hu
        da = dY[s] @ Wd.T
        dhu = da * hg * sg
        dhg = da * hu * sg * (1.0 + hg * (1.0 - sg))
        dx[s] = dhg @ Wg.T + dhu @ Wu.T
        if want_dw:
            dwd[e] = a.T @ dY[s]
            dwg[e] = X[s].T @ dhg
            dwu[e] = X[s].T @ dhu
    return {"dx_perm": dx, "dw_gate": dwg, "dw_up": dwu, "dw_down": dwd}


def dispatch_backward(dx_perm, perm_dst, k):
    """dx[t] = sum_j dX[perm_dst[t*k + j]], summed in slot order."""
    dX = np.asarray(dx_perm, np.float64)
    R = dX.shape[0]
    T = R // k
    rows = np.asarray(perm_dst, np.int64).reshape(T, k)
    dx = np.zeros((T, dX.shape[1]))
    for j in range(k):
        dx += dX[rows[:, j]]
    return dx


def topk_gates_backward(gates, dgates, topk_idx, num_experts):
    """Gradient of the renormalised gates w.r.t. the logits.

    dlogits[t, S_j] = g_j * (dg_j - sum_i g_i dg_i); zero for unselected experts
    (the renormalised gates do not depend on them).  Returns fp64 [T, E].
    """
    g = np.asarray(gates, np.float64)
    dg = np.asarray(dgates, np.float64)
    idx = np.asarray(topk_idx, np.int64)
    T = g.shape[0]
    inner = (g * dg).sum(axis=1, keepdims=True)
    dl = np.zeros((T, num_experts))
    np.put_along_axis(dl, idx, g * (dg - inner), axis=1)
    return dl


def router_logits_backward(x, w_r, dlogits):
    """Backward of l = x W_r: dx = dl W_r^T, dW_r = x^T dl (fp64)."""
    X = np.asarray(x, np.float64)
    W = np.asarray(w_r, np.float64)
    dl = np.asarray(dlogits, np.float64)
    return dl @ W.T, X.T @ dl


# ----------------------------------------------------------------------------
# Whole layer.
# ----------------------------------------------------------------------------


def layer_forward_backward(x, w_gate, w_up, w_down, dout, k, *, logits=None, w_router=None, want_dw=True):
    """One MoE layer forward and backward, composed from the steps above.

    Either ``w_router`` is given (logits = x W_r, router gradient included) or
    ``logits`` is given directly (fp32 synthetic logits; no router weight).  If
    both are given, routing uses the given fp32 ``logits`` (so that both sides
    route from the same bytes) while the router gradient still uses w_router.
    Returns a dict with every intermediate and gradient, fp64 except integers.
    want_dw=False skips the expert weight gradients (per-token checks).
    """
    x = np.asarray(x, np.float64)
    E = np.asarray(w_gate).shape[0]
    res = {}
    if logits is None:
        # Gates from the fp64 logits (differentiable in every input); the
        # selection still compares the values rounded to fp32.
        lg = router_logits(x, w_router)
        res["logits"] = lg
    else:
        lg = np.asarray(logits, np.float32)
        if w_router is not None:
            res["logits"] = router_logits(x, w_router)
    idx = topk_select(lg, k)
    g = topk_gates(lg, idx)
    meta = routing_metadata(idx, E)
    res.update(meta)
    res["topk_idx"] = idx
    res["gates"] = g
    x_perm = dispatch(x, meta["perm_src"], k)
    res["x_perm"] = x_perm
    fwd = expert_ffn_forward(x_perm, meta["offsets"], w_gate, w_up, w_down)
    res.update(fwd)
    res["out"] = combine(fwd["y_perm"], g, meta["perm_dst"], k)
    dy, dg = combine_backward(dout, fwd["y_perm"], g, meta["perm_dst"], k)
    res["dy_perm"] = dy
    res["dgates"] = dg
    bwd = expert_ffn_backward(dy, x_perm, meta["offsets"], w_gate, w_up, w_down, want_dw=want_dw)
    res.update(bwd)
    dx = dispatch_backward(bwd["dx_perm"], meta["perm_dst"], k)
    dl = topk_gates_backward(g, dg, idx, E)
    res["dlogits"] = dl
    if w_router is not None:
        dx_r, dw_r = router_logits_backward(x, w_router, dl)
        dx = dx + dx_r
        res["dw_router"] = dw_r
    res["dx"] = dx
    return res
