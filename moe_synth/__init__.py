"""Seeded synthetic inputs for the MoE expert layer.

This module is shared by the CPU oracle, the GPU tests and the benchmark.  It
holds workload shapes and random draws only: none of the layer's arithmetic
(no routing, no rounding rules of the method, no GEMMs).

Recipe (one recipe for every workload):
  * x, dY ~ N(0, 1); router and expert weights ~ N(0, 0.02^2), the
    initialisation the OLMoE page gives for experts and router
    (OLMoE walkthrough, "expert layer" section: normal init with
    initializer_range 0.02).
  * Every tensor is drawn in float32 from its own numpy PCG64 stream,
    seeded by (seed, tensor id, chunk id), in chunks so that large tensors
    can be drawn by several threads and still be identical for any thread
    count.
  * bf16 workloads take the float32 draw and round it to bf16 with torch's
    round-to-nearest-even conversion (a library call, not the method).
  * Pre-routed workloads (one GPU's share of a large MoE) draw each row's
    local expert from a truncated Zipf(s) law over the non-empty experts
    (rank order fixed by a seeded permutation) and its combine weight from
    U(0, 1).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "draw_normal",
           "zipf_routing", "to_bf16_bits", "bf16_bits_to_f32"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""
    name: str
    T: int          # tokens (received rows for pre-routed workloads)
    d: int          # d_model
    E: int          # experts
    f: int          # d_ff per expert
    k: int          # top_k
    dtype: str      # storage/arithmetic type of the tensors: "fp32" | "bf16"
    prec: str       # GEMM precision: "fp32" | "bf16" | "mxfp8"
    routing: str    # "router" (softmax top-k on x.Wr) | "zipf" (pre-routed rows)
    zipf_s: float = 1.1
    empty_experts: Tuple[int, ...] = ()
    note: str = ""
    passes: str = "fwd+bwd"   # "fwd": inference-shaped, forward only
    mx_wgrad: bool = False    # MXFP8 weight gradients as well (prec "mxfp8")

    @property
    def R(self) -> int:
        return self.T * self.k

    def flops(self) -> float:
        """Algorithmic FLOPs of one forward+backward pass.

        Expert GEMMs: forward 3 GEMMs of 2*R*d*f, backward 6 (dgrad + wgrad),
        i.e. 18*R*d*f.  Router: x.Wr forward plus dWr and dx backward,
        6*T*d*E (absent for pre-routed rows)."""
        g = 18.0 * self.R * self.d * self.f
        if self.routing == "router":
            g += 6.0 * self.T * self.d * self.E
        return g

    def expert_flops(self) -> float:
        return 18.0 * self.R * self.d * self.f

    def fwd_flops(self) -> float:
        """Forward only: 6*R*d*f in the experts plus 2*T*d*E in the router."""
        g = 6.0 * self.R * self.d * self.f
        if self.routing == "router":
            g += 2.0 * self.T * self.d * self.E
        return g


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", T=256, d=64, E=8, f=128, k=2, dtype="fp32",
                          prec="fp32", routing="router",
                          note="tiny fp32 layer, parity-size"),
    "olmoe_bf16": Workload("olmoe_bf16", T=8192, d=2048, E=64, f=1024, k=8,
                           dtype="bf16", prec="bf16", routing="router",
                           note="OLMoE-shaped layer (4x2048 tokens)"),
    "escan_e8_bf16": Workload("escan_e8_bf16", T=16384, d=4096, E=8, f=1536, k=4,
                              dtype="bf16", prec="bf16", routing="router"),
    "escan_e32_bf16": Workload("escan_e32_bf16", T=16384, d=4096, E=32, f=1536, k=4,
                               dtype="bf16", prec="bf16", routing="router"),
    "escan_e128_bf16": Workload("escan_e128_bf16", T=16384, d=4096, E=128, f=1536, k=4,
                                dtype="bf16", prec="bf16", routing="router"),
    "share1t_bf16": Workload("share1t_bf16", T=65536, d=7168, E=24, f=2048, k=1,
                             dtype="bf16", prec="bf16", routing="zipf", zipf_s=1.1,
                             empty_experts=(0, 11, 23),
                             note="one GPU's share of a trillion-scale MoE: "
                                  "65536 received rows, 24 resident experts"),
    "olmoe_mxfp8": Workload("olmoe_mxfp8", T=8192, d=2048, E=64, f=1024, k=8,
                            dtype="bf16", prec="mxfp8", routing="router"),
    "tiny_mxfp8": Workload("tiny_mxfp8", T=256, d=64, E=8, f=128, k=2,
                           dtype="bf16", prec="mxfp8", routing="router"),
    "olmoe_mxfp8_wgrad": Workload("olmoe_mxfp8_wgrad", T=8192, d=2048, E=64, f=1024, k=8,
                                  dtype="bf16", prec="mxfp8", routing="router", mx_wgrad=True,
                                  note="every expert GEMM in MXFP8, weight gradients too"),
}
# Inference-shaped small batches of the OLMoE layer (token-by-token generation
# and short prompts): forward only.
for _t in (1, 8, 64):
    WORKLOADS[f"olmoe_decode_t{_t}"] = Workload(
        f"olmoe_decode_t{_t}", T=_t, d=2048, E=64, f=1024, k=8, dtype="bf16", prec="bf16",
        routing="router", passes="fwd", note=f"OLMoE layer forward on {_t} token(s)")
del _t


def workload(base: str, **overrides) -> Workload:
    """A named workload, optionally with some fields replaced (smaller T, ...)."""
    w = WORKLOADS[base]
    if overrides:
        w = dataclasses.replace(w, **overrides)
    return w


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------
_TENSOR_IDS = {"x": 1, "Wr": 2, "Wg": 3, "Wu": 4, "Wd": 5, "dY": 6,
               "route_perm": 7, "route_rank": 8, "route_w": 9}
_CHUNK = 1 << 22  # elements per independently seeded chunk


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def draw_normal(seed: int, tensor: str, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draw of the given shape; identical for any thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    tid = _TENSOR_IDS[tensor]
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, c])))
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (torch's RNE conversion) and return the raw
    16-bit patterns as uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def zipf_routing(seed: int, rows: int, E: int, s: float, empty: Tuple[int, ...]):
    """Pre-routed rows: expert index per row (k = 1) and a U(0,1) combine weight.

    The non-empty experts get Zipf ranks 1..n through a seeded permutation; each
    row draws its rank i.i.d. with P(rank = r) proportional to r^-s."""
    live = np.array([e for e in range(E) if e not in set(empty)], dtype=np.int64)
    n = live.size
    rng_p = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSOR_IDS["route_perm"]])))
    order = live[rng_p.permutation(n)]            # order[r-1] = expert of rank r
    pr = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    pr /= pr.sum()
    rng_r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSOR_IDS["route_rank"]])))
    ranks = rng_r.choice(n, size=rows, p=pr)
    idx = order[ranks].astype(np.int32).reshape(rows, 1)
    rng_w = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSOR_IDS["route_w"]])))
    w = rng_w.uniform(0.0, 1.0, size=rows).astype(np.float32)
    # U(0,1) is open at 0: redraw exact zeros (probability ~2^-53) as the smallest weight
    w[w == 0.0] = np.float32(np.finfo(np.float32).tiny)
    return idx, w.reshape(rows, 1)


def make_inputs(wl: Workload, seed: int = 0, with_dY: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one forward+backward pass as float32 numpy arrays.

    For bf16 workloads every array holds bf16-representable values, and the
    raw bf16 bit patterns are returned under '<name>_bits'.  Pre-routed
    workloads also return 'topk_idx' (int32 [T,1]) and 'topk_w' (fp32 [T,1])."""
    T, d, E, f = wl.T, wl.d, wl.E, wl.f
    out: Dict[str, np.ndarray] = {}
    shapes = {"x": ((T, d), 1.0), "Wg": ((E, d, f), 0.02), "Wu": ((E, d, f), 0.02),
              "Wd": ((E, f, d), 0.02)}
    if wl.routing == "router":
        shapes["Wr"] = ((d, E), 0.02)
    if with_dY:
        shapes["dY"] = ((T, d), 1.0)
    for name, (shape, std) in shapes.items():
        a = draw_normal(seed, name, shape, std)
        if wl.dtype == "bf16":
            bits = to_bf16_bits(a)
            out[name + "_bits"] = bits
            a = bf16_bits_to_f32(bits)
        out[name] = a
    if wl.routing == "zipf":
        idx, w = zipf_routing(seed, T, E, wl.zipf_s, wl.empty_experts)
        out["topk_idx"] = idx
        out["topk_w"] = w
    return out
