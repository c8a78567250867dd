"""Thin Python binding of libmoe's C ABI (argument marshalling only).

Each function here has the name of the C entry point it calls, takes torch
tensors (device memory) and the current torch stream, and passes their raw
pointers through ctypes.  Every step of the computation runs in libmoe's HIP
kernels; nothing here computes.  If the library is not built the first call
raises, there is no fallback path.

torch is imported before the library is loaded so that libmoe binds to the HIP
runtime already in the process (torch ships one with the same soname).
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
_PREC = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8}

_c_void_p, _i64, _i32, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int

_SIGS = {
    "moe_abi_version": (_int, []),
    "moe_status_str": (ctypes.c_char_p, [_int]),
    "moe_router_logits": (_int, [_c_void_p, _c_void_p, _int, _i64, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_router_logits_bwd_workspace": (_sz, [_i64, _i32, _i32]),
    "moe_router_logits_bwd": (_int, [_c_void_p, _c_void_p, _int, _c_void_p, _i64, _i32, _i32, _c_void_p, _int,
                                     _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_route_topk_workspace": (_sz, [_i64, _i32, _i32]),
    "moe_route_topk": (_int, [_c_void_p, _i64, _i32, _i32] + [_c_void_p] * 8 + [_sz, _c_void_p]),
    "moe_route_topk_noalloc": (_int, [_c_void_p, _i64, _i32, _i32] + [_c_void_p] * 8),
    "moe_route_topk_bwd": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_dispatch": (_int, [_c_void_p, _int, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "moe_dispatch_bwd": (_int, [_c_void_p, _int, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "moe_combine": (_int, [_c_void_p, _int, _c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_combine_bwd": (_int, [_c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p,
                               _c_void_p, _c_void_p]),
    "moe_grouped_ffn_workspace": (_sz, [_i64, _i32, _i32, _i32, _int, _int]),
    "moe_grouped_ffn_fwd": (_int, [_i64, _i32, _i32, _i32, _int] + [_c_void_p] * 11 + [_c_void_p, _sz, _c_void_p]),
    "moe_grouped_ffn_bwd": (_int, [_i64, _i32, _i32, _i32, _int] + [_c_void_p] * 18 + [_c_void_p, _sz, _c_void_p]),
    "moe_mx_act_bytes": (_sz, [_i64, _i32]),
    "moe_mx_tok_rows": (_i64, [_i64, _i32]),
    "moe_mx_tok_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_dispatch_mx_tok": (_int, [_c_void_p, _i64, _i32, _i32, _i32] + [_c_void_p] * 7),
    "moe_combine_bwd_mx_tok": (_int, [_c_void_p] * 7 + [_i64, _i32, _i32, _i32] + [_c_void_p] * 5),
    "moe_dispatch_mx": (_int, [_c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "moe_combine_bwd_mx": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p,
                                  _c_void_p, _c_void_p, _c_void_p]),
    "moe_mx_weight_cache_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_route_stats": (_int, [_c_void_p, _i32, _c_void_p, _c_void_p]),
    "moe_mx_weight_cache_build": (_int, [_c_void_p] * 3 + [_i32, _i32, _i32, _c_void_p, _sz, _c_void_p]),
    "mx_quantize": (_int, [_c_void_p, _int, _i64, _i64, _i64, _i32, _c_void_p, _i32, _c_void_p, _c_void_p,
                           _c_void_p]),
    "moe_timing_enable": (_int, [_int]),
    "moe_timing_report": (_int, [ctypes.c_char_p, _sz]),
}

_lib = None


class MoeError(RuntimeError):
    pass


def lib():
    """Load libmoe.so (once) and declare its C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def _check(status: int, what: str):
    if status != 0:
        msg = lib().moe_status_str(status).decode()
        raise MoeError(f"{what} failed: {msg} (status {status})")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise MoeError(f"unsupported dtype {t.dtype}")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- router

def moe_router_logits(x, w_r, out=None):
    T, d = x.shape
    E = w_r.shape[1]
    out = torch.empty((T, E), dtype=torch.float32, device=x.device) if out is None else out
    _check(lib().moe_router_logits(_p(x), _p(w_r), _dtype_code(x), T, d, E, _p(out), _stream()), "moe_router_logits")
    return out


def moe_router_logits_bwd(x, w_r, dlogits, dx, accumulate_dx=True, dw_r=None, ws=None):
    T, d = x.shape
    E = w_r.shape[1]
    dw_r = torch.empty_like(w_r) if dw_r is None else dw_r
    need = lib().moe_router_logits_bwd_workspace(T, d, E)
    ws = _ws(need, x.device) if ws is None else ws
    _check(lib().moe_router_logits_bwd(_p(x), _p(w_r), _dtype_code(x), _p(dlogits), T, d, E, _p(dx),
                                       int(bool(accumulate_dx)), _p(dw_r), _p(ws), ws.numel(), _stream()),
           "moe_router_logits_bwd")
    return dw_r


def moe_route_topk(logits, k, out=None, ws=None):
    """Returns dict topk_idx, gates, counts, offsets, perm_src, perm_dst, mx_blk_offsets."""
    T, E = logits.shape
    dev = logits.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {
            "topk_idx": torch.empty((T, k), **i32),
            "gates": torch.empty((T, k), dtype=torch.float32, device=dev),
            "counts": torch.empty(E, **i32),
            "offsets": torch.empty(E + 1, **i32),
            "perm_src": torch.empty(T * k, **i32),
            "perm_dst": torch.empty(T * k, **i32),
            "mx_blk_offsets": torch.empty(E + 1, **i32),
        }
    need = lib().moe_route_topk_workspace(T, E, k)
    ws = _ws(need, dev) if ws is None else ws
    _check(lib().moe_route_topk(_p(logits), T, E, k, _p(out["topk_idx"]), _p(out["gates"]), _p(out["counts"]),
                                _p(out["offsets"]), _p(out["perm_src"]), _p(out["perm_dst"]),
                                _p(out.get("mx_blk_offsets")), _p(ws), ws.numel(), _stream()), "moe_route_topk")
    return out


def moe_route_topk_noalloc(logits, k, out):
    """moe_route_topk on the library's static scratch (no workspace); `out` as moe_route_topk returns it."""
    T, E = logits.shape
    _check(lib().moe_route_topk_noalloc(_p(logits), T, E, k, _p(out["topk_idx"]), _p(out["gates"]),
                                        _p(out["counts"]), _p(out["offsets"]), _p(out["perm_src"]),
                                        _p(out["perm_dst"]), _p(out.get("mx_blk_offsets")), _stream()),
           "moe_route_topk_noalloc")
    return out


def moe_route_topk_bwd(gates, dgates, topk_idx, E, out=None):
    T, k = gates.shape
    out = torch.empty((T, E), dtype=torch.float32, device=gates.device) if out is None else out
    _check(lib().moe_route_topk_bwd(_p(gates), _p(dgates), _p(topk_idx), T, E, k, _p(out), _stream()),
           "moe_route_topk_bwd")
    return out


# --------------------------------------------------------------------------- dispatch / combine

def moe_dispatch(x, perm_dst, k, out=None):
    T, d = x.shape
    out = torch.empty((T * k, d), dtype=x.dtype, device=x.device) if out is None else out
    _check(lib().moe_dispatch(_p(x), _dtype_code(x), T, d, k, _p(perm_dst), _p(out), _stream()), "moe_dispatch")
    return out


def moe_mx_act_buffer(rows, cols, device):
    """Caller buffer for moe_dispatch_mx / moe_combine_bwd_mx: E4M3 codes [rows, cols], then grouped scales."""
    n = lib().moe_mx_act_bytes(rows, cols)
    if n == 0:
        raise MoeError(f"moe_mx_act_bytes({rows}, {cols}): unsupported size")
    return _ws(n, device)


def mx_act_split(buf, rows, cols):
    """(codes uint8 [rows, cols], grouped scale bytes uint8 [rows * cols / 32]) views of an MX activation buffer."""
    off = -(-rows * cols // 256) * 256
    return buf[:rows * cols].view(rows, cols), buf[off:off + rows * cols // 32]


def moe_dispatch_mx(x, perm_dst, k, out=None, mx=None):
    """moe_dispatch that also writes the MX rows layout of x_perm (bf16, d % 128 == 0); returns (x_perm, mx)."""
    T, d = x.shape
    out = torch.empty((T * k, d), dtype=x.dtype, device=x.device) if out is None else out
    mx = moe_mx_act_buffer(T * k, d, x.device) if mx is None else mx
    _check(lib().moe_dispatch_mx(_p(x), T, d, k, _p(perm_dst), _p(out), _p(mx), _stream()), "moe_dispatch_mx")
    return out, mx


def moe_mx_tok_buffer(rows, E, cols, device):
    """Caller buffer for the token-axis MX layout: E4M3 codes [cols, moe_mx_tok_rows(rows, E)], then grouped scales."""
    n = lib().moe_mx_tok_bytes(rows, E, cols)
    if n == 0:
        raise MoeError(f"moe_mx_tok_bytes({rows}, {E}, {cols}): unsupported size")
    return _ws(n, device)


def mx_tok_split(buf, rows, E, cols):
    """(codes uint8 [cols, Rp], grouped scale bytes uint8 [Rp / 32 * cols]) views of a token-axis MX buffer."""
    rp = lib().moe_mx_tok_rows(rows, E)
    off = -(-rp * cols // 256) * 256
    return buf[:rp * cols].view(cols, rp), buf[off:off + rp // 32 * cols]


def moe_dispatch_mx_tok(x, route, k, E, out=None, mx=None, mxt=None, write_rows=False):
    """Both MX layouts of the expert rows of x (rows and token-axis), from the routing `route` (perm_src,
    offsets, mx_blk_offsets); the bf16 rows too when write_rows or `out` is given.  Returns (x_perm or None, mx,
    mxt)."""
    T, d = x.shape
    R = T * k
    if out is None and write_rows:
        out = torch.empty((R, d), dtype=x.dtype, device=x.device)
    mx = moe_mx_act_buffer(R, d, x.device) if mx is None else mx
    mxt = moe_mx_tok_buffer(R, E, d, x.device) if mxt is None else mxt
    _check(lib().moe_dispatch_mx_tok(_p(x), T, d, k, E, _p(route["perm_src"]), _p(route["offsets"]),
                                     _p(route["mx_blk_offsets"]), _p(out), _p(mx), _p(mxt), _stream()),
           "moe_dispatch_mx_tok")
    return out, mx, mxt


def moe_dispatch_bwd(dx_perm, perm_dst, k, out=None):
    R, d = dx_perm.shape
    T = R // k
    out = torch.empty((T, d), dtype=dx_perm.dtype, device=dx_perm.device) if out is None else out
    _check(lib().moe_dispatch_bwd(_p(dx_perm), _dtype_code(dx_perm), T, d, k, _p(perm_dst), _p(out), _stream()),
           "moe_dispatch_bwd")
    return out


def moe_combine(y_perm, gates, perm_dst, out=None):
    T, k = gates.shape
    d = y_perm.shape[1]
    out = torch.empty((T, d), dtype=y_perm.dtype, device=y_perm.device) if out is None else out
    _check(lib().moe_combine(_p(y_perm), _dtype_code(y_perm), _p(gates), _p(perm_dst), T, d, k, _p(out), _stream()),
           "moe_combine")
    return out


def moe_combine_bwd(dout, y_perm, gates, perm_dst, dy_perm=None, dgates=None):
    T, k = gates.shape
    d = dout.shape[1]
    dy_perm = torch.empty_like(y_perm) if dy_perm is None else dy_perm
    dgates = torch.empty((T, k), dtype=torch.float32, device=dout.device) if dgates is None else dgates
    _check(lib().moe_combine_bwd(_p(dout), _p(y_perm), _dtype_code(dout), _p(gates), _p(perm_dst), T, d, k,
                                 _p(dy_perm), _p(dgates), _stream()), "moe_combine_bwd")
    return dy_perm, dgates


def moe_combine_bwd_mx(dout, y_perm, gates, perm_dst, dy_perm=None, dgates=None, mx=None):
    """moe_combine_bwd that also writes the MX rows layout of dy_perm; returns (dy_perm, dgates, mx)."""
    T, k = gates.shape
    d = dout.shape[1]
    dy_perm = torch.empty_like(y_perm) if dy_perm is None else dy_perm
    dgates = torch.empty((T, k), dtype=torch.float32, device=dout.device) if dgates is None else dgates
    mx = moe_mx_act_buffer(T * k, d, dout.device) if mx is None else mx
    _check(lib().moe_combine_bwd_mx(_p(dout), _p(y_perm), _p(gates), _p(perm_dst), T, d, k, _p(dy_perm), _p(dgates),
                                    _p(mx), _stream()), "moe_combine_bwd_mx")
    return dy_perm, dgates, mx


def moe_combine_bwd_mx_tok(dout, y_perm, gates, route, E, dy_perm=None, dgates=None, mx=None, mxt=None,
                           write_rows=False):
    """dgates, and dY = gate x dout in both MX layouts (rows and token-axis); the bf16 rows too when write_rows
    or `dy_perm` is given.  Returns (dy_perm or None, dgates, mx, mxt)."""
    T, k = gates.shape
    d = dout.shape[1]
    R = T * k
    if dy_perm is None and write_rows:
        dy_perm = torch.empty_like(y_perm)
    dgates = torch.empty((T, k), dtype=torch.float32, device=dout.device) if dgates is None else dgates
    mx = moe_mx_act_buffer(R, d, dout.device) if mx is None else mx
    mxt = moe_mx_tok_buffer(R, E, d, dout.device) if mxt is None else mxt
    _check(lib().moe_combine_bwd_mx_tok(_p(dout), _p(y_perm), _p(gates), _p(route["perm_dst"]), _p(route["perm_src"]),
                                        _p(route["offsets"]), _p(route["mx_blk_offsets"]), T, d, k, E, _p(dy_perm),
                                        _p(dgates), _p(mx), _p(mxt), _stream()), "moe_combine_bwd_mx_tok")
    return dy_perm, dgates, mx, mxt


def moe_route_stats(counts, out=None):
    """counts [E] int32 (device) -> int32 [4] on the device: max rows, min rows, empty experts, total rows."""
    E = counts.shape[0]
    out = torch.empty(4, dtype=torch.int32, device=counts.device) if out is None else out
    _check(lib().moe_route_stats(_p(counts), E, _p(out), _stream()), "moe_route_stats")
    return out


# --------------------------------------------------------------------------- grouped FFN

def moe_grouped_ffn_workspace(R, E, d, f, prec, is_bwd):
    return lib().moe_grouped_ffn_workspace(R, E, d, f, _PREC[prec], int(is_bwd))


def moe_grouped_ffn_fwd(x_perm, offsets, w_gate, w_up, w_down, prec, out=None, ws=None, mx_wcache=None, x_mx=None,
                        rows=None):
    """x_perm may be None with prec "mxfp8" and x_mx given; then `rows` (R) is required."""
    E, d, f = w_gate.shape
    R = x_perm.shape[0] if x_perm is not None else int(rows)
    dev = w_gate.device
    if out is None:
        out = {name: torch.empty((R, f), dtype=w_gate.dtype, device=dev) for name in ("h_gate", "h_up", "a_act")}
        out["y_perm"] = torch.empty((R, d), dtype=w_gate.dtype, device=dev)
    ws = _ws(moe_grouped_ffn_workspace(R, E, d, f, prec, 0), dev) if ws is None else ws
    _check(lib().moe_grouped_ffn_fwd(R, E, d, f, _PREC[prec], _p(offsets), _p(x_perm), _p(w_gate), _p(w_up),
                                     _p(w_down), _p(mx_wcache), _p(x_mx), _p(out["h_gate"]), _p(out["h_up"]),
                                     _p(out["a_act"]), _p(out["y_perm"]), _p(ws), ws.numel(), _stream()),
           "moe_grouped_ffn_fwd")
    return out


def moe_grouped_ffn_bwd(dy_perm, x_perm, h_gate, h_up, a_act, offsets, mx_blk_offsets, w_gate, w_up, w_down, prec,
                        out=None, ws=None, mx_wcache=None, dy_mx=None, x_mxt=None, dy_mxt=None):
    """With prec "mxfp8", x_perm may be None when x_mxt is given, dy_perm when dy_mx and dy_mxt are."""
    E, d, f = w_gate.shape
    R = h_gate.shape[0]
    dev = h_gate.device
    if out is None:
        out = {"dx_perm": torch.empty((R, d), dtype=h_gate.dtype, device=dev), "dw_gate": torch.empty_like(w_gate),
               "dw_up": torch.empty_like(w_up), "dw_down": torch.empty_like(w_down)}
    ws = _ws(moe_grouped_ffn_workspace(R, E, d, f, prec, 1), dev) if ws is None else ws
    _check(lib().moe_grouped_ffn_bwd(R, E, d, f, _PREC[prec], _p(offsets), _p(mx_blk_offsets), _p(dy_perm),
                                     _p(x_perm), _p(h_gate), _p(h_up), _p(a_act), _p(w_gate), _p(w_up), _p(w_down),
                                     _p(mx_wcache), _p(dy_mx), _p(x_mxt), _p(dy_mxt), _p(out["dx_perm"]),
                                     _p(out["dw_gate"]), _p(out["dw_up"]),
                                     _p(out["dw_down"]), _p(ws), ws.numel(), _stream()), "moe_grouped_ffn_bwd")
    return out


def moe_mx_weight_cache_build(w_gate, w_up, w_down, cache=None):
    """Pre-quantised MXFP8 weights (both orientations); returns the uint8 cache tensor."""
    E, d, f = w_gate.shape
    n = lib().moe_mx_weight_cache_bytes(E, d, f)
    cache = _ws(n, w_gate.device) if cache is None else cache
    _check(lib().moe_mx_weight_cache_build(_p(w_gate), _p(w_up), _p(w_down), E, d, f, _p(cache), cache.numel(),
                                           _stream()), "moe_mx_weight_cache_build")
    return cache


# --------------------------------------------------------------------------- MX quantiser

def mx_quantize(src, axis, seg_offsets=None, nseg=0, q=None, scales=None):
    """src [rows, cols] or [batch, rows, cols]; layouts as documented in include/moe.h."""
    s3 = src if src.dim() == 3 else src.unsqueeze(0)
    B, rows, cols = s3.shape
    dev = src.device
    if q is None:
        if axis == 1:
            q = torch.empty((B, rows, cols), dtype=torch.uint8, device=dev)
            scales = torch.empty((B, rows, cols // 32), dtype=torch.uint8, device=dev)
        elif seg_offsets is None:
            q = torch.empty((B, cols, rows), dtype=torch.uint8, device=dev)
            scales = torch.empty((B, cols, rows // 32), dtype=torch.uint8, device=dev)
        else:
            rp = 32 * (-(-rows // 32) + nseg)
            q = torch.empty((cols, rp), dtype=torch.uint8, device=dev)
            scales = torch.empty((cols, rp // 32), dtype=torch.uint8, device=dev)
    _check(lib().mx_quantize(_p(s3), _dtype_code(src), B, rows, cols, axis, _p(seg_offsets), nseg, _p(q), _p(scales),
                             _stream()), "mx_quantize")
    return q, scales


# --------------------------------------------------------------------------- diagnostics

def moe_timing_enable(on: bool = True):
    _check(lib().moe_timing_enable(int(bool(on))), "moe_timing_enable")


def moe_timing_report() -> dict:
    """{kernel name: (launches, total ms)} of the launches since the last enable/report."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(lib().moe_timing_report(buf, len(buf)), "moe_timing_report")
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        out[name] = (int(n), float(ms))
    return out
