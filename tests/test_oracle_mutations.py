"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins fail.

Each mutation swaps one oracle function for a subtly wrong version: a dropped
term, a wrong sign or index, a transposed or swapped operand, a wrong tie rule.
The pin helpers of test_oracle_pins must reject every one of them.
"""
import numpy as np
import pytest

from oracle import moe_oracle as mo
from oracle import mx_oracle as mx

import test_oracle_pins as pins


def _fails(check, *args):
    with pytest.raises((AssertionError, ValueError, IndexError)):
        check(*args)


def test_silu_replaced_by_sigmoid(monkeypatch):
    monkeypatch.setattr(mo, "silu", lambda z: mo.sigmoid(z))
    _fails(pins.check_forward, pins.oracle_out)


def test_gate_and_up_swapped(monkeypatch):
    orig = mo.expert_ffn_forward
    monkeypatch.setattr(mo, "expert_ffn_forward",
                        lambda x, o, wg, wu, wd: orig(x, o, wu, wg, wd))
    _fails(pins.check_forward, pins.oracle_out)


def test_combine_uses_wrong_slot_order(monkeypatch):
    orig = mo.combine
    monkeypatch.setattr(mo, "combine", lambda y, g, pd, k: orig(y, g[:, ::-1], pd, k))
    _fails(pins.check_forward, pins.oracle_out)


def test_dhg_missing_term(monkeypatch):
    def bad(dy_perm, x_perm, offsets, wg, wu, wd, want_dw=True):
        X, dY = np.asarray(x_perm, float), np.asarray(dy_perm, float)
        out = {"dx_perm": np.zeros_like(X), "dw_gate": np.zeros_like(wg), "dw_up": np.zeros_like(wu),
               "dw_down": np.zeros_like(wd)}
        for e in range(wg.shape[0]):
            s = slice(int(offsets[e]), int(offsets[e + 1]))
            hg, hu = X[s] @ wg[e], X[s] @ wu[e]
            sg = mo.sigmoid(hg)
            da = dY[s] @ wd[e].T
            dhu = da * hg * sg
            dhg = da * hu * sg  # the (1 + hg (1 - sg)) factor dropped
            out["dx_perm"][s] = dhg @ wg[e].T + dhu @ wu[e].T
            out["dw_down"][e] = (hg * sg * hu).T @ dY[s]
            out["dw_gate"][e] = X[s].T @ dhg
            out["dw_up"][e] = X[s].T @ dhu
        return out
    monkeypatch.setattr(mo, "expert_ffn_backward", bad)
    _fails(pins.check_backward, pins.oracle_out)


def test_wgrad_operands_swapped(monkeypatch):
    orig = mo.expert_ffn_backward

    def bad(*a, **kw):
        r = orig(*a, **kw)
        r["dw_gate"], r["dw_up"] = r["dw_up"], r["dw_gate"]
        return r
    monkeypatch.setattr(mo, "expert_ffn_backward", bad)
    _fails(pins.check_backward, pins.oracle_out)


def test_router_bwd_sign_flipped(monkeypatch):
    orig = mo.topk_gates_backward
    monkeypatch.setattr(mo, "topk_gates_backward", lambda g, dg, i, E: -orig(g, dg, i, E))
    _fails(pins.check_backward, pins.oracle_out)


def test_router_weight_grad_transposed_input(monkeypatch):
    monkeypatch.setattr(mo, "router_logits_backward",
                        lambda x, w, dl: (dl @ np.asarray(w).T, np.asarray(x).T @ dl[::-1]))
    _fails(pins.check_backward, pins.oracle_out)


def test_dispatch_bwd_uses_wrong_index(monkeypatch):
    orig = mo.dispatch_backward
    monkeypatch.setattr(mo, "dispatch_backward",
                        lambda dX, pd, k: orig(dX, np.roll(pd, 1), k))
    _fails(pins.check_backward, pins.oracle_out)


def test_topk_tie_to_higher_index():
    def bad(logits, k):
        l32 = np.asarray(logits, np.float32)
        E = l32.shape[1]
        rev = np.argsort(-l32[:, ::-1], axis=1, kind="stable")
        return (E - 1 - rev[:, :k]).astype(np.int32)
    _fails(pins.check_topk, bad)


def test_gates_not_renormalised():
    def bad(logits, idx):
        l64 = np.asarray(logits, np.float64)
        full = np.exp(l64 - l64.max(axis=1, keepdims=True))
        full /= full.sum(axis=1, keepdims=True)
        return np.take_along_axis(full, np.asarray(idx, np.int64), axis=1)
    _fails(pins.check_gates, bad)


def test_metadata_token_major_order():
    def bad(idx, E):
        m = mo.routing_metadata(idx, E)
        R = idx.size
        m["perm_src"] = np.arange(R, dtype=np.int32)  # token-major instead of expert-major
        m["perm_dst"] = np.arange(R, dtype=np.int32)
        return m
    _fails(pins.check_metadata, bad)


def test_metadata_offsets_inclusive():
    def bad(idx, E):
        m = mo.routing_metadata(idx, E)
        m["offsets"] = np.concatenate([np.cumsum(m["counts"]), [idx.size]]).astype(np.int32)
        return m
    _fails(pins.check_metadata, bad)


def test_e4m3_round_half_up():
    def bad(y):
        y = np.asarray(y, np.float64)
        a = np.abs(y)
        _, ex = np.frexp(a)
        p = np.maximum(ex - 1, -6)
        q = np.ldexp(1.0, p - 3)
        r = np.minimum(np.floor(a / q + 0.5) * q, 448.0)
        return mx.e4m3_encode(np.where(np.signbit(y), -r, r))
    _fails(pins.check_encode, bad)


def test_e4m3_no_saturation():
    def bad(y):
        y = np.asarray(y, np.float64)
        c = mx.e4m3_encode(y).astype(np.int64)
        return np.where(np.abs(y) > 464, c | 0x7F, c).astype(np.uint8)  # NaN instead of 448
    _fails(pins.check_encode, bad)


def test_mx_weight_quantised_along_wrong_axis():
    from oracle import moe_mx_oracle as mxl

    def layer_with_bad_axes(p):
        inner = mxl.q_along

        def bad(v, axis, seg=None):
            # weights (the two 64/96-sized operands) encoded along the wrong axis
            if seg is None and set(np.shape(v)) == {64, 96}:
                axis = 1 - axis
            return inner(v, axis, seg)
        mxl.q_along = bad
        try:
            return pins._mx_layer(p)
        finally:
            mxl.q_along = inner
    _fails(pins.check_mx_axes, layer_with_bad_axes)


def test_mx_recompute_weight_along_wrong_axis(monkeypatch):
    """The backward's recompute of Hg, Hu with Wg encoded along f instead of d."""
    from oracle import moe_mx_oracle as mxl

    def bad(X, offsets, w_gate, w_up):
        E, d, f = np.shape(w_gate)
        hg, hu = np.zeros((X.shape[0], f)), np.zeros((X.shape[0], f))
        Xq = mxl.q_along(X, 1)
        for e in range(E):
            s = slice(int(offsets[e]), int(offsets[e + 1]))
            hg[s] = Xq[s] @ mxl.q_along(np.asarray(w_gate[e], np.float64), 1)
            hu[s] = Xq[s] @ mxl.q_along(np.asarray(w_up[e], np.float64), 0)
        return hg, hu
    monkeypatch.setattr(mxl, "mx_expert_ffn_forward_gate_up", bad)
    _fails(pins.check_mx_recompute, mxl)
    _fails(pins.check_mx_recompute_axes, mxl)


def test_mx_recompute_activation_along_wrong_axis(monkeypatch):
    """The recompute with X encoded down the tokens instead of along d."""
    from oracle import moe_mx_oracle as mxl
    orig = mxl.mx_expert_ffn_forward_gate_up

    def bad(X, offsets, w_gate, w_up):
        inner = mxl.q_along

        def wrong(v, axis, seg=None):
            if np.shape(v) == np.shape(X):
                axis = 1 - axis
            return inner(v, axis, seg)
        mxl.q_along = wrong
        try:
            return orig(X, offsets, w_gate, w_up)
        finally:
            mxl.q_along = inner
    monkeypatch.setattr(mxl, "mx_expert_ffn_forward_gate_up", bad)
    _fails(pins.check_mx_recompute, mxl)


def test_mx_recompute_skips_silu(monkeypatch):
    """The fwd=None branch building A without the SiLU (A = Hg * Hu)."""
    from oracle import moe_mx_oracle as mxl
    orig_bwd = mxl.mx_expert_ffn_backward

    def bad(dy_perm, x_perm, offsets, w_gate, w_up, w_down, want_dw=True, fwd=None):
        if fwd is None:
            hg, hu = mxl.mx_expert_ffn_forward_gate_up(np.asarray(x_perm, np.float64), offsets, w_gate, w_up)
            fwd = {"h_gate": mxl.round_to_bf16(hg), "h_up": mxl.round_to_bf16(hu),
                   "a_act": mxl.round_to_bf16(hg * hu)}
        return orig_bwd(dy_perm, x_perm, offsets, w_gate, w_up, w_down, want_dw=want_dw, fwd=fwd)
    monkeypatch.setattr(mxl, "mx_expert_ffn_backward", bad)
    _fails(pins.check_mx_recompute, mxl)
