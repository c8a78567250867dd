"""One MoE layer step (forward + backward) as a sequence of libmoe ABI calls.

Olmo-core 3 announcement, "Scaling and optimizing MoE training": route, place
the routed rows straight into the experts' buffers, run the expert FFN as a
grouped GEMM, combine; the routing metadata never leaves the GPU, so the host
enqueues the whole step without a single synchronisation.

This module only allocates device buffers (once, up front) and calls the
binding in order; every step runs in libmoe's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .workloads import Workload


def to_device(inp: dict, device="cuda") -> dict:
    """Host inputs (fp32 numpy arrays exactly representable in storage type) -> device tensors."""
    dt = torch.bfloat16 if inp["storage"] == "bf16" else torch.float32
    out = {}
    for key, val in inp.items():
        if not isinstance(val, np.ndarray):
            continue
        t = torch.from_numpy(np.ascontiguousarray(val))
        out[key] = t.to(device=device, dtype=torch.float32 if key == "logits" else dt)
    return out


class LayerStep:
    """Preallocated buffers and workspaces for one layer step of workload ``w``.

    MXFP8 expert weights, three ways:
      default               the forward and the backward quantise the layouts they use (no cache);
      mx_weights_per_step   every step first quantises the weights into both layouts from one read
                            (moe_mx_weight_cache_build), and its forward and backward use them: the weights
                            change once per optimiser step, so this is the whole per-step conversion;
      mx_weight_cache       quantised once here and reused by every step (valid while the weights do not change).
    MXFP8 activations (mx_movement), bit-identical results every way:
      "tok" (default)       the dispatch and the combine backward write X and dY straight into both MX layouts the
                            FFN uses, rows (along d) and token-axis (along each expert's tokens, for the weight
                            gradients), from the routing permutation (moe_dispatch_mx_tok / moe_combine_bwd_mx_tok);
                            the bf16 expert rows x_perm / dy_perm are then not needed and not written, unless
                            keep_rows asks for them;
      "rows"                they write the bf16 rows and their rows layout (moe_dispatch_mx / moe_combine_bwd_mx),
                            the FFN quantises the token-axis layouts;
      "none"                plain dispatch and combine backward; the FFN quantises everything.
    """

    def __init__(self, w: Workload, dev_inputs: dict, mx_weight_cache: bool = False,
                 mx_weights_per_step: bool = False, mx_movement: str = "tok", keep_rows: bool = False):
        self.w = w
        self.inp = dev_inputs
        self.mx_wcache = None
        self.mx_per_step = bool(mx_weights_per_step) and w.prec == "mxfp8"
        assert mx_movement in ("tok", "rows", "none"), mx_movement
        self.mx_movement = mx_movement if w.prec == "mxfp8" else "none"
        self.mx_fused = self.mx_movement != "none"
        tok = self.mx_movement == "tok"
        x = dev_inputs["x"]
        dev = x.device
        T, d, E, k, f, R = w.T, w.d, w.E, w.k, w.f, w.R
        dt = x.dtype
        i32 = dict(dtype=torch.int32, device=dev)
        self.linear_router = "w_router" in dev_inputs
        self.logits = (torch.empty((T, E), dtype=torch.float32, device=dev) if self.linear_router
                       else dev_inputs["logits"])
        self.route = {
            "topk_idx": torch.empty((T, k), **i32),
            "gates": torch.empty((T, k), dtype=torch.float32, device=dev),
            "counts": torch.empty(E, **i32),
            "offsets": torch.empty(E + 1, **i32),
            "perm_src": torch.empty(R, **i32),
            "perm_dst": torch.empty(R, **i32),
            "mx_blk_offsets": torch.empty(E + 1, **i32),
        }
        self.route_ws = B._ws(B.lib().moe_route_topk_workspace(T, E, k), dev)
        rows = not tok or keep_rows  # the bf16 expert rows x_perm, dy_perm are written
        self.x_perm = torch.empty((R, d), dtype=dt, device=dev) if rows else None
        self.x_mx = B.moe_mx_act_buffer(R, d, dev) if self.mx_fused else None
        self.dy_mx = B.moe_mx_act_buffer(R, d, dev) if self.mx_fused else None
        self.x_mxt = B.moe_mx_tok_buffer(R, E, d, dev) if tok else None
        self.dy_mxt = B.moe_mx_tok_buffer(R, E, d, dev) if tok else None
        self.ffn = {n: torch.empty((R, f), dtype=dt, device=dev) for n in ("h_gate", "h_up", "a_act")}
        self.ffn["y_perm"] = torch.empty((R, d), dtype=dt, device=dev)
        self.ffn_ws_f = B._ws(B.moe_grouped_ffn_workspace(R, E, d, f, w.prec, 0), dev)
        self.ffn_ws_b = B._ws(B.moe_grouped_ffn_workspace(R, E, d, f, w.prec, 1), dev)
        self.out = torch.empty((T, d), dtype=dt, device=dev)
        self.dy_perm = torch.empty((R, d), dtype=dt, device=dev) if rows else None
        self.dgates = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.grads = {
            "dx_perm": torch.empty((R, d), dtype=dt, device=dev),
            "dw_gate": torch.empty_like(dev_inputs["w_gate"]),
            "dw_up": torch.empty_like(dev_inputs["w_up"]),
            "dw_down": torch.empty_like(dev_inputs["w_down"]),
        }
        self.dx = torch.empty((T, d), dtype=dt, device=dev)
        self.dlogits = torch.empty((T, E), dtype=torch.float32, device=dev)
        if self.linear_router:
            self.dw_router = torch.empty_like(dev_inputs["w_router"])
            self.router_ws = B._ws(B.lib().moe_router_logits_bwd_workspace(T, d, E), dev)
        if (mx_weight_cache or self.mx_per_step) and w.prec == "mxfp8":
            self.build_weight_cache()

    def build_weight_cache(self):
        """Quantise the expert weights (both orientations) into the cache the forward and backward read."""
        inp = self.inp
        self.mx_wcache = B.moe_mx_weight_cache_build(inp["w_gate"], inp["w_up"], inp["w_down"], cache=self.mx_wcache)
        return self.mx_wcache

    # ------------------------------------------------------------------ steps
    def forward(self):
        w, inp = self.w, self.inp
        if self.linear_router:
            B.moe_router_logits(inp["x"], inp["w_router"], out=self.logits)
        B.moe_route_topk(self.logits, w.k, out=self.route, ws=self.route_ws)
        if self.mx_movement == "tok":
            B.moe_dispatch_mx_tok(inp["x"], self.route, w.k, w.E, out=self.x_perm, mx=self.x_mx, mxt=self.x_mxt)
        elif self.mx_movement == "rows":
            B.moe_dispatch_mx(inp["x"], self.route["perm_dst"], w.k, out=self.x_perm, mx=self.x_mx)
        else:
            B.moe_dispatch(inp["x"], self.route["perm_dst"], w.k, out=self.x_perm)
        B.moe_grouped_ffn_fwd(self.x_perm, self.route["offsets"], inp["w_gate"], inp["w_up"], inp["w_down"], w.prec,
                              out=self.ffn, ws=self.ffn_ws_f, mx_wcache=self.mx_wcache, x_mx=self.x_mx, rows=w.R)
        B.moe_combine(self.ffn["y_perm"], self.route["gates"], self.route["perm_dst"], out=self.out)
        return self.out

    def backward(self, dout=None):
        w, inp = self.w, self.inp
        dout = inp["dout"] if dout is None else dout
        if self.mx_movement == "tok":
            B.moe_combine_bwd_mx_tok(dout, self.ffn["y_perm"], self.route["gates"], self.route, w.E,
                                     dy_perm=self.dy_perm, dgates=self.dgates, mx=self.dy_mx, mxt=self.dy_mxt)
        elif self.mx_movement == "rows":
            B.moe_combine_bwd_mx(dout, self.ffn["y_perm"], self.route["gates"], self.route["perm_dst"],
                                 dy_perm=self.dy_perm, dgates=self.dgates, mx=self.dy_mx)
        else:
            B.moe_combine_bwd(dout, self.ffn["y_perm"], self.route["gates"], self.route["perm_dst"],
                              dy_perm=self.dy_perm, dgates=self.dgates)
        B.moe_grouped_ffn_bwd(self.dy_perm, self.x_perm, self.ffn["h_gate"], self.ffn["h_up"], self.ffn["a_act"],
                              self.route["offsets"], self.route["mx_blk_offsets"], inp["w_gate"], inp["w_up"],
                              inp["w_down"], w.prec, out=self.grads, ws=self.ffn_ws_b, mx_wcache=self.mx_wcache,
                              dy_mx=self.dy_mx, x_mxt=self.x_mxt, dy_mxt=self.dy_mxt)
        B.moe_dispatch_bwd(self.grads["dx_perm"], self.route["perm_dst"], w.k, out=self.dx)
        B.moe_route_topk_bwd(self.route["gates"], self.dgates, self.route["topk_idx"], w.E, out=self.dlogits)
        if self.linear_router:
            B.moe_router_logits_bwd(inp["x"], inp["w_router"], self.dlogits, self.dx, accumulate_dx=True,
                                    dw_r=self.dw_router, ws=self.router_ws)
        return self.dx

    def step(self):
        if self.mx_per_step:
            self.build_weight_cache()
        self.forward()
        self.backward()
