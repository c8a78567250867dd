"""Seeded synthetic inputs for the MoE layer workloads (no method arithmetic here).

The Olmo-core 3 announcement benchmarks its MoE stack with random routing and an
even expert load ("Scaling to the trillion-parameter range", "Scaling and
optimizing MoE training") and warns that kernel time depends on the values, not
only the shapes, so every comparison must reuse identical inputs.  This module
makes those inputs, identically for the HIP library and for the CPU oracle.

Recipe: numpy ``default_rng(SeedSequence([seed, workload_id, tensor_id]))``
(per-expert weight slices add the expert index as a fourth word), standard
normal fp32 draws times sigma (1 for activations, logits and upstream gradients,
0.02 for weights; sigma is the standard deviation), then round-to-nearest-even
to bf16 where the workload is bf16.  Tensor ids: x 0, W_r 1, Wg 2, Wu 3, Wd 4,
logits 5, dout 6, Zipf ranks 7.

Workloads (T tokens, d model width, E experts, k chosen per token, f expert
hidden width):
  1 tiny-fp32     T=256,   d=64,   E=8,   k=2, f=128,  fp32, logits = x W_r
  2 bf16-e8       T=8192,  d=2048, E=8,   k=4, f=1024, bf16, logits = x W_r
  3 bf16-e128     T=16384, d=2048, E=128, k=4, f=1024, bf16, logits ~ N(0,1)
  4 bf16-e128-zipf  as 3, logits ~ N(0,1) + 3*ln(1/rank_e), ranks a seeded
                  permutation of 1..E (a few hot experts, many empty)
  5 mxfp8-e128    T=16384, d=4096, E=128, k=4, f=1536, bf16 masters with
                  MXFP8 expert GEMMs, logits ~ N(0,1)
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses

import numpy as np

DEFAULT_SEED = 17

TID_X, TID_WR, TID_WG, TID_WU, TID_WD, TID_LOGITS, TID_DOUT, TID_RANKS = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    prec: str          # "f32" | "bf16" | "mxfp8" (mxfp8: bf16 masters, MX GEMMs)
    router: str        # "linear" (logits = x W_r) | "normal" | "zipf"

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def storage(self) -> str:
        """Element type of activations and weights in memory."""
        return "f32" if self.prec == "f32" else "bf16"

    def describe(self) -> dict:
        return {"T": self.T, "d": self.d, "E": self.E, "k": self.k, "f": self.f,
                "prec": self.prec, "router": self.router}


WORKLOADS = {
    1: Workload(1, "tiny-fp32", 256, 64, 8, 2, 128, "f32", "linear"),
    2: Workload(2, "bf16-e8", 8192, 2048, 8, 4, 1024, "bf16", "linear"),
    3: Workload(3, "bf16-e128", 16384, 2048, 128, 4, 1024, "bf16", "normal"),
    4: Workload(4, "bf16-e128-zipf", 16384, 2048, 128, 4, 1024, "bf16", "zipf"),
    5: Workload(5, "mxfp8-e128", 16384, 4096, 128, 4, 1536, "mxfp8", "normal"),
}


def scaled(w: Workload, **changes) -> Workload:
    """Same distributions at other sizes (parity cases smaller than the full workload)."""
    return dataclasses.replace(w, **changes)


def rng(seed: int, wid: int, tid: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, wid, tid, *extra]))


def normal(shape, sigma: float, seed: int, wid: int, tid: int) -> np.ndarray:
    """Standard normal fp32 draws times sigma."""
    return rng(seed, wid, tid).standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def expert_normal(E: int, shape, sigma: float, seed: int, wid: int, tid: int) -> np.ndarray:
    """[E, *shape] fp32; expert e drawn from its own stream (threads in parallel)."""
    out = np.empty((E, *shape), np.float32)

    def fill(e):
        r = rng(seed, wid, tid, e)
        r.standard_normal(shape, dtype=np.float32, out=out[e])
        out[e] *= np.float32(sigma)

    with _cf.ThreadPoolExecutor(max_workers=min(16, max(1, E))) as ex:
        list(ex.map(fill, range(E)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_bias(E: int, seed: int, wid: int) -> np.ndarray:
    """Per-expert logit bias 3*ln(1/rank_e), ranks a seeded permutation of 1..E."""
    ranks = rng(seed, wid, TID_RANKS).permutation(E) + 1
    return (3.0 * np.log(1.0 / ranks)).astype(np.float32)


def make_inputs(w: Workload, seed: int = DEFAULT_SEED) -> dict:
    """All host inputs of one layer step as numpy arrays.

    Float tensors are returned as fp32 values exactly representable in the
    workload's storage type; ``storage`` says which.  Keys: x [T,d], w_gate,
    w_up [E,d,f], w_down [E,f,d], dout [T,d], and w_router [d,E] for the linear
    router or logits [T,E] (fp32) otherwise.
    """
    bf = w.storage == "bf16"

    def cast(a):
        return bf16_bits_to_f32(f32_to_bf16_bits(a)) if bf else a

    inp = {
        "x": cast(normal((w.T, w.d), 1.0, seed, w.wid, TID_X)),
        "w_gate": cast(expert_normal(w.E, (w.d, w.f), 0.02, seed, w.wid, TID_WG)),
        "w_up": cast(expert_normal(w.E, (w.d, w.f), 0.02, seed, w.wid, TID_WU)),
        "w_down": cast(expert_normal(w.E, (w.f, w.d), 0.02, seed, w.wid, TID_WD)),
        "dout": cast(normal((w.T, w.d), 1.0, seed, w.wid, TID_DOUT)),
    }
    if w.router == "linear":
        inp["w_router"] = cast(normal((w.d, w.E), 0.02, seed, w.wid, TID_WR))
    else:
        logits = normal((w.T, w.E), 1.0, seed, w.wid, TID_LOGITS)
        if w.router == "zipf":
            logits = logits + zipf_bias(w.E, seed, w.wid)[None, :]
        inp["logits"] = logits.astype(np.float32)
    inp["storage"] = w.storage
    return inp
