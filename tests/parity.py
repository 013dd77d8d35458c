"""Helpers of the GPU parity tests: upload seeded inputs, run the layer
through the C ABI, run the oracle on the same inputs, compare."""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

from moe_synth import Workload, make_inputs
from oracle import moe_oracle as O

TOL = {"fp32": 1e-4, "bf16": 2e-2, "mxfp8": 6e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(inp: Dict[str, np.ndarray], name: str, dtype: torch.dtype) -> torch.Tensor:
    from routing_grouped_gemm_amd import upload
    if dtype == torch.bfloat16:
        return upload(inp[name + "_bits"], torch.bfloat16)
    return upload(np.ascontiguousarray(inp[name], dtype=np.float32))


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.detach().cpu().numpy()


def relerr(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Normwise relative error ||gpu - ref|| / ||ref|| (0 when both are 0)."""
    gpu = np.asarray(gpu, np.float64); ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    nd = np.linalg.norm(gpu - ref)
    if nr == 0.0:
        return 0.0 if nd == 0.0 else float("inf")
    return float(nd / nr)


# Local gates beside the normwise bound, so that an error confined to a few
# rows or elements (one wrong 16-byte store piece, a broken ragged tail) cannot
# hide in a large tensor's norm:
#   * worst row: ||gpu_r - ref_r|| / max(||ref_r||, ROW_FLOOR * rms_r ||ref_r||)
#     over the rows r of the last axis, at most ROW_C * tol;
#   * worst element: max |gpu - ref| / RMS(ref), at most ELEM_C * tol.
# Legitimate differences are one storage-rounding step on values a few RMS
# large (bf16: 2^-8 of ~6 RMS = 0.02 RMS) and float32 summation order; a
# misplaced element or piece is off by about its own size (~RMS).
ROW_C, ELEM_C, ROW_FLOOR = 5.0, 10.0, 0.25


def local_errors(gpu: np.ndarray, ref: np.ndarray):
    """(normwise, worst row, worst element / RMS) of gpu against ref."""
    g = np.asarray(gpu, np.float64); r = np.asarray(ref, np.float64)
    if g.shape != r.shape:
        raise AssertionError(f"shape {g.shape} != {r.shape}")
    norm = relerr(g, r)
    if r.size == 0:
        return norm, 0.0, 0.0
    g2 = g.reshape(-1, r.shape[-1]) if r.ndim > 1 else g.reshape(1, -1)
    r2 = r.reshape(-1, r.shape[-1]) if r.ndim > 1 else r.reshape(1, -1)
    rn = np.linalg.norm(r2, axis=1)
    dn = np.linalg.norm(g2 - r2, axis=1)
    rms_row = float(np.sqrt(np.mean(rn ** 2)))
    den = np.maximum(rn, ROW_FLOOR * rms_row)
    with np.errstate(divide="ignore", invalid="ignore"):
        row = np.where(den > 0, dn / np.where(den > 0, den, 1.0), np.where(dn > 0, np.inf, 0.0))
    rms = float(np.sqrt(np.mean(r ** 2)))
    md = float(np.max(np.abs(g - r)))
    elem = (md / rms) if rms > 0 else (0.0 if md == 0.0 else float("inf"))
    return norm, float(np.max(row)), elem


def gate(name: str, gpu, ref, tol: float, errs: Optional[dict] = None):
    """Returns (and records in errs) the three errors; the caller asserts
    with check_gates."""
    e = local_errors(gpu, ref)
    if errs is not None:
        errs[name] = e
    return e


def check_gates(label: str, errs: dict, tol: float) -> None:
    say(f"  {label}: " + " ".join(f"{n}={e[0]:.2e}/{e[1]:.1e}/{e[2]:.1e}" for n, e in errs.items())
        + "  (normwise/worst row/worst element over RMS)")
    bad = {n: e for n, e in errs.items()
           if not (e[0] <= tol and e[1] <= ROW_C * tol and e[2] <= ELEM_C * tol)}
    assert not bad, (f"{label}: over tolerance (normwise {tol}, row {ROW_C * tol}, "
                     f"element {ELEM_C * tol} RMS): {bad}")


def run_gpu(wl: Workload, inp: Dict[str, np.ndarray], logits: Optional[np.ndarray] = None,
            renorm: bool = False, aux_coef: float = 0.0, wgrad_f32: bool = False,
            wgrad_init=None, mx_wgrad: bool = False):
    """Forward + backward of the layer on the GPU; returns every buffer as numpy.
    wgrad_init: a value, or a dict of arrays by name ("dWg", "dWu", "dWd"),
    to fill the weight-gradient buffers with before accumulating into them."""
    import routing_grouped_gemm_amd as rgg
    dt = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
    router = wl.routing == "router"
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, dt, wl.prec, router=router,
                            renorm=renorm, aux_coef=aux_coef, wgrad_f32=wgrad_f32,
                            mx_wgrad=mx_wgrad)
    x = dev_tensor(inp, "x", dt)
    Wg, Wu, Wd = (dev_tensor(inp, n, dt) for n in ("Wg", "Wu", "Wd"))
    Wr = dev_tensor(inp, "Wr", dt) if router else None
    dY = dev_tensor(inp, "dY", dt)
    kw = {}
    if router and logits is not None:
        kw["logits"] = rgg.upload(np.ascontiguousarray(logits, np.float32))
    if not router:
        kw["topk_idx"] = rgg.upload(inp["topk_idx"])
        kw["topk_w"] = rgg.upload(inp["topk_w"])
    layer.forward(x, Wr, Wg, Wu, Wd, **kw)
    if isinstance(wgrad_init, dict):
        for n in ("dWg", "dWu", "dWd"):
            t = getattr(layer, n)
            t.copy_(torch.as_tensor(np.ascontiguousarray(wgrad_init[n], np.float32)).to(t.dtype))
    elif wgrad_init is not None:
        for t in (layer.dWg, layer.dWu, layer.dWd):
            t.fill_(wgrad_init)
    layer.backward(dY, accumulate_wgrad=wgrad_init is not None)
    torch.cuda.synchronize()
    names = ["topk_idx", "topk_w", "counts", "offsets", "dest_row", "src_token", "Hg", "Hu",
             "A", "Ys", "y", "dYs", "dw", "dH", "dXs", "dx", "dWg", "dWu", "dWd", "Xs"]
    if wl.prec == "mxfp8":
        names += ["Xq", "Xq_scale", "dYs_q", "dYs_q_scale"]
    if router:
        names += ["logits", "dlogits", "dWr"]
    if router and aux_coef:
        names += ["aux_loss", "aux_dp"]
    out = {n: to_np(getattr(layer, n)) for n in names}
    if wl.prec == "mxfp8":
        # activation scales as [R][d/32] (row, block); the raw shape is checked too
        R = wl.T * wl.k
        for n in ("Xq_scale", "dYs_q_scale"):
            raw = getattr(layer, n)
            assert tuple(raw.shape) == rgg.mx_scale_shape(R, wl.d), (n, tuple(raw.shape))
            out[n] = to_np(rgg.mx_scale_rows(raw, R, wl.d))
    f = wl.f
    out["dHg"], out["dHu"] = out["dH"][:, :f], out["dH"][:, f:]
    return out


def run_oracle(wl: Workload, inp: Dict[str, np.ndarray], logits: Optional[np.ndarray] = None,
               renorm: bool = False, aux_coef: float = 0.0, wgrad_f32: bool = False,
               mx_wgrad: bool = False):
    prec = wl.prec
    if wl.routing == "router":
        return O.layer(inp["x"], inp["Wr"], inp["Wg"], inp["Wu"], inp["Wd"], wl.k, inp["dY"], prec,
                       logits=logits, renorm=renorm, aux_coef=aux_coef, wgrad_f32=wgrad_f32,
                       mx_wgrad=mx_wgrad)
    return O.layer(inp["x"], None, inp["Wg"], inp["Wu"], inp["Wd"], wl.k, inp["dY"], prec,
                   topk_idx=inp["topk_idx"], topk_w=inp["topk_w"], wgrad_f32=wgrad_f32,
                   mx_wgrad=mx_wgrad)


EXACT = ("topk_idx", "counts", "offsets", "dest_row", "src_token")
FLOATS = ("Xs", "Hg", "Hu", "A", "Ys", "y", "dYs", "dw", "dHg", "dHu", "dXs", "dx", "dWg",
          "dWu", "dWd", "dlogits", "dWr")


def compare(wl: Workload, gpu, ref, tol: Optional[float] = None, skip=()):
    """Bit-exact integer metadata; per float tensor the normwise relative
    error within tol, and the worst row and worst element within the local
    gates (ROW_C, ELEM_C)."""
    tol = TOL[wl.prec] if tol is None else tol
    errs = {}
    for n in EXACT:
        if n in gpu and n in ref and n not in skip:
            np.testing.assert_array_equal(gpu[n], np.asarray(ref[n]), err_msg=f"{wl.name}: {n}")
    if "topk_w" in gpu and "topk_w" in ref:
        ew = relerr(gpu["topk_w"], ref["topk_w"])
        assert ew <= 1e-5, (wl.name, "topk_w", ew)
    for n in FLOATS:
        if n in gpu and n in ref and n not in skip:
            gate(n, gpu[n], ref[n], tol, errs)
    check_gates(wl.name, errs, tol)
    return {n: e[0] for n, e in errs.items()}
