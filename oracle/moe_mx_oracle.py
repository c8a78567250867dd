"""CPU oracle of the MoE layer with MXFP8 expert GEMMs (fp64 apart from the encoding).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline); never imported by
the product path; shares no code with the HIP library.

Source.  Olmo-core 3 announcement, "Scaling and optimizing MoE training":
MXFP8 replaces BF16 in the parts of training where it helps most, and most of
the gain came from the feed-forward (expert) computation.  Reading taken: every
one of the six expert GEMMs (forward, input-gradient and weight-gradient) takes
both operands in MXFP8, each quantised along that GEMM's contraction axis with
the OCP MX encoding of ``mx_oracle``; products and everything outside the
GEMMs stay in fp64 (routing, gates, SwiGLU, combine, dispatch).  Operands and
their contraction axes:

  G1  Hg = Q_d(X) Q_d(Wg_e),  Hu = Q_d(X) Q_d(Wu_e)       (contract over d)
  G2  Y  = Q_f(A) Q_f(Wd_e)                                (over f)
  G3  dA = Q_d(dY) Q_d(Wd_e)^T                             (over d)
  G5  dX = Q_f(dHg) Q_f(Wg_e)^T + Q_f(dHu) Q_f(Wu_e)^T     (over f)
  G4  dWd_e = Q_t(A_e)^T Q_t(dY_e)                         (over the expert's tokens)
  G6  dWg_e = Q_t(X_e)^T Q_t(dHg_e), dWu_e = Q_t(X_e)^T Q_t(dHu_e)

Q_t blocks run along the tokens of one expert segment (blocks restart at the
segment start, last block zero-padded).  Each Q is quantise-then-dequantise of
mx_oracle, i.e. the value the MX GEMM multiplies.

Stored tensors.  The MXFP8 path keeps every tensor that passes between its
steps in bf16 (Hg, Hu, A after G1; Y after G2; dY after the combine backward;
dHg, dHu after G3), and its quantiser encodes those bf16 values.  An E4M3 code
is an integer decision, so this oracle takes it from the same precision: each
of those tensors is rounded to bf16 (round to nearest even, ``round_to_bf16``)
where it is stored, and all arithmetic between stores is fp64.

Pins (tests/test_oracle_pins.py): with the encoding and the bf16 stores
replaced by the identity this function equals moe_oracle.layer_forward_backward;
the operand/axis of every quantisation is checked against the table above by
recording the calls; round_to_bf16 is checked against torch's fp32->bf16
conversion.
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as mo
from . import mx_oracle as mxo


def round_to_bf16(v):
    """fp64 -> nearest bf16 value (8 significant bits, ties to even), as fp64."""
    v = np.asarray(v, np.float64)
    _, ex = np.frexp(v)
    # spacing of bf16 values around v: 2**(floor(log2|v|) - 7); subnormal spacing 2**-133
    quantum = np.ldexp(1.0, np.maximum(ex - 1, -126) - 7)
    return np.round(v / quantum) * quantum


def q_along(v, axis, seg=None):
    """Value of v after MX encoding along ``axis`` (0: down the rows, 1: along a row)."""
    q, s = mxo.mx_quantize(v, axis=axis, seg_offsets=seg)
    return mxo.mx_dequantize(q, s, axis=axis, seg_offsets=seg)


def _expert_weights(w_gate, w_up, w_down, e):
    return tuple(np.asarray(w[e], np.float64) for w in (w_gate, w_up, w_down))


def mx_expert_ffn_forward(x_perm, offsets, w_gate, w_up, w_down):
    """G1 and G2 with MXFP8 operands over the expert-major buffer (fp64 otherwise).

    Returns h_gate, h_up, a_act [R, f] and y_perm [R, d].
    """
    X = np.asarray(x_perm, np.float64)
    E, d, f = np.shape(w_gate)
    R = X.shape[0]
    hg, hu, y = np.zeros((R, f)), np.zeros((R, f)), np.zeros((R, d))
    experts = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    Xq = q_along(X, 1)
    for e in experts:
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        wg, wu, _ = _expert_weights(w_gate, w_up, w_down, e)
        hg[s] = Xq[s] @ q_along(wg, 0)
        hu[s] = Xq[s] @ q_along(wu, 0)
    a = round_to_bf16(mo.silu(hg) * hu)
    Aq = q_along(a, 1)
    for e in experts:
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        y[s] = Aq[s] @ q_along(np.asarray(w_down[e], np.float64), 0)
    return {"h_gate": round_to_bf16(hg), "h_up": round_to_bf16(hu), "a_act": a, "y_perm": round_to_bf16(y)}


def mx_expert_ffn_backward(dy_perm, x_perm, offsets, w_gate, w_up, w_down, want_dw=True, fwd=None):
    """G3, G5, G4, G6 with MXFP8 operands.  The forward intermediates Hg, Hu come
    from ``fwd`` (the result of mx_expert_ffn_forward) or are recomputed (MX G1)."""
    dY = round_to_bf16(dy_perm)
    X = np.asarray(x_perm, np.float64)
    E, d, f = np.shape(w_gate)
    R = X.shape[0]
    if fwd is None:
        hg, hu = mx_expert_ffn_forward_gate_up(X, offsets, w_gate, w_up)
        a = round_to_bf16(mo.silu(hg) * hu)
        hg, hu = round_to_bf16(hg), round_to_bf16(hu)
    else:
        hg, hu, a = fwd["h_gate"], fwd["h_up"], fwd["a_act"]
    experts = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    dyq = q_along(dY, 1)
    dhg, dhu = np.zeros((R, f)), np.zeros((R, f))
    for e in experts:
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        da = dyq[s] @ q_along(np.asarray(w_down[e], np.float64), 1).T
        sg = mo.sigmoid(hg[s])
        dhu[s] = da * hg[s] * sg
        dhg[s] = da * hu[s] * sg * (1.0 + hg[s] * (1.0 - sg))
    dhg, dhu = round_to_bf16(dhg), round_to_bf16(dhu)
    dhgq, dhuq = q_along(dhg, 1), q_along(dhu, 1)
    dX = np.zeros((R, d))
    out = {"dw_gate": None, "dw_up": None, "dw_down": None}
    if want_dw:
        out = {"dw_gate": np.zeros((E, d, f)), "dw_up": np.zeros((E, d, f)), "dw_down": np.zeros((E, f, d))}
    for e in experts:
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        wg, wu, _ = _expert_weights(w_gate, w_up, w_down, e)
        dX[s] = dhgq[s] @ q_along(wg, 1).T + dhuq[s] @ q_along(wu, 1).T
        if want_dw:
            seg = [0, s.stop - s.start]
            xt = q_along(X[s], 0, seg)
            out["dw_down"][e] = q_along(a[s], 0, seg).T @ q_along(dY[s], 0, seg)
            out["dw_gate"][e] = xt.T @ q_along(dhg[s], 0, seg)
            out["dw_up"][e] = xt.T @ q_along(dhu[s], 0, seg)
    out["dx_perm"] = dX
    return out


def mx_expert_ffn_forward_gate_up(X, offsets, w_gate, w_up):
    """G1 alone (Hg, Hu), as the backward recomputes it."""
    E, d, f = np.shape(w_gate)
    R = X.shape[0]
    hg, hu = np.zeros((R, f)), np.zeros((R, f))
    Xq = q_along(X, 1)
    for e in range(E):
        if offsets[e + 1] <= offsets[e]:
            continue
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        hg[s] = Xq[s] @ q_along(np.asarray(w_gate[e], np.float64), 0)
        hu[s] = Xq[s] @ q_along(np.asarray(w_up[e], np.float64), 0)
    return hg, hu


def mx_layer_forward_backward(x, w_gate, w_up, w_down, dout, k, *, logits, want_dw=True):
    """MoE layer forward + backward with the six expert GEMMs in MXFP8 (see module doc).

    Routing from the given fp32 ``logits``.  Returns the keys of
    moe_oracle.layer_forward_backward: routing integers and gates, y_perm, out,
    dgates, dx_perm, dx, dlogits, and dw_gate, dw_up, dw_down (want_dw).
    """
    lg = np.asarray(logits, np.float32)
    E = np.shape(w_gate)[0]
    idx = mo.topk_select(lg, k)
    g = mo.topk_gates(lg, idx)
    meta = mo.routing_metadata(idx, E)
    X = mo.dispatch(np.asarray(x, np.float64), meta["perm_src"], k)
    fwd = mx_expert_ffn_forward(X, meta["offsets"], w_gate, w_up, w_down)
    out = mo.combine(fwd["y_perm"], g, meta["perm_dst"], k)
    dy, dg = mo.combine_backward(dout, fwd["y_perm"], g, meta["perm_dst"], k)
    bwd = mx_expert_ffn_backward(dy, X, meta["offsets"], w_gate, w_up, w_down, want_dw=want_dw, fwd=fwd)
    res = dict(meta)
    res.update(topk_idx=idx, gates=g, x_perm=X, y_perm=fwd["y_perm"], out=out, dgates=dg, dx_perm=bwd["dx_perm"],
               dx=mo.dispatch_backward(bwd["dx_perm"], meta["perm_dst"], k),
               dlogits=mo.topk_gates_backward(g, dg, idx, E))
    if want_dw:
        res.update(dw_gate=bwd["dw_gate"], dw_up=bwd["dw_up"], dw_down=bwd["dw_down"])
    return res
