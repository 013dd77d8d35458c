"""Python binding of libmoe_hip.so, the MI355X MoE expert-layer library.

Argument marshalling only: every function here takes torch tensors that live
on the GPU, checks nothing the C library does not check itself, passes their
data pointers, sizes and torch's current HIP stream to the C entry point of
the same name (declared in include/moe.h), and raises RuntimeError on a
non-zero status.  All computation happens in the library's HIP kernels; there
is no CPU or PyTorch fallback, and importing the binding fails loudly when
the library has not been built.

ExpertLayer owns the buffers of one layer (forward and backward) and calls
the entry points in the order of the layer: route -> dispatch ->
grouped_ffn_fwd -> combine, then combine_bwd -> grouped_ffn_bwd ->
dispatch_bwd -> route_bwd.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "lib", "moe_route", "moe_dispatch", "moe_dispatch_noalloc", "moe_grouped_ffn_fwd", "moe_combine",
    "moe_combine_bwd", "moe_grouped_ffn_bwd", "moe_dispatch_bwd", "moe_route_bwd",
    "moe_route_aux", "moe_check_routing", "moe_workspace_size", "moe_status_string",
    "ExpertLayer", "LIB_PATH",
    "MOE_ROUTE_LOGITS_IN", "MOE_ROUTE_RENORM", "MOE_ACCUMULATE", "MOE_WGRAD_F32", "MOE_MX_KEEP_WEIGHTS",
    "KernelTimer", "upload", "mx_scale_pitch", "mx_scale_shape", "mx_scale_rows", "probe_clock",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_hip.so")

MOE_F32, MOE_BF16 = 0, 1
PREC = {"fp32": 0, "bf16": 1, "mxfp8": 2}
MOE_ROUTE_LOGITS_IN = 0x1
MOE_ACCUMULATE = 0x2
MOE_ROUTE_RENORM = 0x4
MOE_WGRAD_F32 = 0x8
MOE_WGRAD_MX = 0x10
MOE_MX_KEEP_WEIGHTS = 0x20
OPS = {"route": 0, "dispatch": 1, "ffn_fwd": 2, "combine": 3, "combine_bwd": 4,
       "ffn_bwd": 5, "dispatch_bwd": 6, "route_bwd": 7, "route_aux": 8,
       "ffn_bwd_mxw": 9, "ffn_fwd_keep": 10}

_P, _I, _U, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
_SIGS = {
    "moe_route": [_P, _P, _I, _I, _I, _I, _I, _U, _P, _P, _P, _P, _S, _P],
    "moe_dispatch": [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P],
    "moe_dispatch_noalloc": [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_grouped_ffn_fwd": [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _I, _I, _U, _P, _P, _P,
                            _P, _P, _S, _P],
    "moe_combine": [_P, _P, _P, _I, _I, _I, _I, _P, _P],
    "moe_combine_bwd": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P],
    "moe_grouped_ffn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _I,
                            _I, _U, _P, _P, _P, _P, _P, _P, _S, _P],
    "moe_dispatch_bwd": [_P, _P, _I, _I, _I, _I, _U, _P, _P],
    "moe_route_bwd": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _U, _P, _P, _P, _P, _S, _P],
    "moe_route_aux": [_P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P, _S, _P],
    "moe_workspace_size": [_I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
    "moe_check_routing": [_P, _I, _I, _I, _P, _P],
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m routing_grouped_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_set_kernel_events.argtypes = [_P, _P, _I, _P]
        L.moe_set_kernel_events.restype = ctypes.c_int
        L.moe_set_kernel_filter.argtypes = [ctypes.c_char_p]
        L.moe_set_kernel_filter.restype = ctypes.c_int
        L.moe_probe_clock.argtypes = [_P, _I, _I, _P]
        L.moe_probe_clock.restype = ctypes.c_int
        L.moe_last_launch_error.argtypes = []
        L.moe_last_launch_error.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def upload(a, dtype: Optional[torch.dtype] = None, device="cuda") -> torch.Tensor:
    """Copy a host numpy array to the GPU through a freshly allocated pinned
    buffer.  Large copies straight from pageable memory make the runtime pin
    the user's pages in place, which some hosts refuse; staging through
    allocated pinned memory avoids that.  dtype=torch.bfloat16 takes an
    array of raw bf16 bit patterns (uint16/int16)."""
    import numpy as np
    a = np.ascontiguousarray(a)
    if dtype == torch.bfloat16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    out = t.pin_memory().to(device)
    return out.view(torch.bfloat16) if dtype == torch.bfloat16 else out


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, name: str) -> None:
    if status != 0:
        detail = ""
        if status == -7:
            detail = f", HIP error {lib().moe_last_launch_error().decode()}"
        raise RuntimeError(f"{name}: {moe_status_string(status)} (status {status}{detail})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def _ws(ws: Optional[torch.Tensor]):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def moe_workspace_size(op: str, T: int, d: int, E: int, f: int, k: int, dtype: torch.dtype,
                       prec: str) -> int:
    out = ctypes.c_size_t(0)
    dt = MOE_F32 if dtype == torch.float32 else MOE_BF16
    _check(lib().moe_workspace_size(OPS[op], T, d, E, f, k, dt, PREC[prec], ctypes.byref(out)),
           "moe_workspace_size")
    return out.value


def moe_route(x, Wr, k, logits, topk_idx, topk_w, logits_in=False, renorm=False, ws=None,
              stream=None):
    T, E = logits.shape
    d = x.shape[1] if x is not None else 64
    dt = _dtype(x) if x is not None else MOE_BF16
    flags = (MOE_ROUTE_LOGITS_IN if logits_in else 0) | (MOE_ROUTE_RENORM if renorm else 0)
    wp, wb = _ws(ws)
    _check(lib().moe_route(_ptr(x), _ptr(Wr), T, d, E, k, dt, flags, _ptr(logits),
                           _ptr(topk_idx), _ptr(topk_w), wp, wb, _stream(stream)), "moe_route")


def moe_dispatch(x, topk_idx, E, counts, offsets, dest_row, src_token, Xs, ws, Xq=None,
                 Xq_scale=None, prec="bf16", stream=None):
    T, d = x.shape
    k = topk_idx.shape[1]
    wp, wb = _ws(ws)
    _check(lib().moe_dispatch(_ptr(x), _ptr(topk_idx), T, d, E, k, _dtype(x), PREC[prec],
                              _ptr(counts), _ptr(offsets), _ptr(dest_row), _ptr(src_token),
                              _ptr(Xs), _ptr(Xq), _ptr(Xq_scale), wp, wb, _stream(stream)),
           "moe_dispatch")


def moe_dispatch_noalloc(x, topk_idx, E, counts, offsets, dest_row, src_token, Xs, Xq=None,
                         Xq_scale=None, prec="bf16", stream=None):
    T, d = x.shape
    k = topk_idx.shape[1]
    _check(lib().moe_dispatch_noalloc(_ptr(x), _ptr(topk_idx), T, d, E, k, _dtype(x), PREC[prec],
                                      _ptr(counts), _ptr(offsets), _ptr(dest_row),
                                      _ptr(src_token), _ptr(Xs), _ptr(Xq), _ptr(Xq_scale),
                                      _stream(stream)),
           "moe_dispatch_noalloc")


REALTIME_MHZ = 100.0   # rate of the constant-rate counter that s_memrealtime reads


def probe_clock(grid: int = 256, iters: int = 20000, stream=None):
    """Clock under MFMA load and the sustained dense bf16 MFMA rate, from one
    moe_probe_clock launch (after an untimed one that loads the kernel).
    clock_mhz: shader clock cycles per constant-rate tick x 100 MHz;
    event_clock_mhz / realtime_mhz: the same counts over the launch's HIP-event
    time (a check: realtime_mhz near 100 means the event window is the
    kernel's); mfma_tflops: the probe's FLOPs over its constant-rate time."""
    ticks = torch.zeros(4 * grid, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream() if stream is None else stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(st):
        _check(lib().moe_probe_clock(_ptr(ticks), grid, 16, _stream(st)), "moe_probe_clock")
        e0.record()
        _check(lib().moe_probe_clock(_ptr(ticks), grid, iters, _stream(st)), "moe_probe_clock")
        e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    t = ticks.view(grid, 4).cpu().double()
    cyc = float((t[:, 1] - t[:, 0]).mean())
    rt = float((t[:, 3] - t[:, 2]).mean())
    rt_us = rt / REALTIME_MHZ
    flops = 8.0 * 32768 * 4 * iters * grid
    return {"clock_mhz": cyc / rt * REALTIME_MHZ, "event_clock_mhz": cyc / us,
            "realtime_mhz": rt / us, "mfma_tflops": flops / (rt_us * 1e-6) / 1e12,
            "probe_us": rt_us}


def moe_check_routing(topk_idx, E, report, stream=None):
    """Enqueue the device check of pre-routed indices; report (int32 [2], on
    the GPU) receives the out-of-range entry count and the count of tokens
    with a repeated expert."""
    T, k = topk_idx.shape
    _check(lib().moe_check_routing(_ptr(topk_idx), T, E, k, _ptr(report), _stream(stream)),
           "moe_check_routing")


def mx_scale_pitch(R: int) -> int:
    """Row pitch of the MXFP8 activation scales: R rounded up to 16."""
    return (R + 15) // 16 * 16


def mx_scale_shape(R: int, K: int):
    """Shape of the MXFP8 activation scales of R rows of K elements: groups of
    four 32-element blocks, [ceil(K/128)][Rp][4] bytes (Rp = mx_scale_pitch(R));
    block b of row r is element [b // 4][r][b % 4]."""
    return ((K + 127) // 128, mx_scale_pitch(R), 4)


def mx_scale_rows(scale, R: int, K: int):
    """View of an activation scale array as [R][K/32] (row r, block b)."""
    G, Rp, _ = mx_scale_shape(R, K)
    return scale.reshape(G, Rp, 4).permute(1, 0, 2).reshape(Rp, 4 * G)[:R, :K // 32]


def moe_grouped_ffn_fwd(Xs, Xs_scale, offsets, T, k, Wg, Wu, Wd, Hg, Hu, A, Ys, ws=None,
                        prec="bf16", stream=None, keep_weights=False):
    E, d, f = Wg.shape
    wp, wb = _ws(ws)
    flags = MOE_MX_KEEP_WEIGHTS if keep_weights else 0
    _check(lib().moe_grouped_ffn_fwd(_ptr(Xs), _ptr(Xs_scale), _ptr(offsets), T, k, d, f, E,
                                     _ptr(Wg), _ptr(Wu), _ptr(Wd), _dtype(Wg), PREC[prec], flags,
                                     _ptr(Hg), _ptr(Hu), _ptr(A), _ptr(Ys), wp, wb,
                                     _stream(stream)), "moe_grouped_ffn_fwd")


def moe_combine(Ys, topk_w, dest_row, y, stream=None):
    T, d = y.shape
    k = topk_w.shape[1]
    _check(lib().moe_combine(_ptr(Ys), _ptr(topk_w), _ptr(dest_row), T, d, k, _dtype(y), _ptr(y),
                             _stream(stream)), "moe_combine")


def moe_combine_bwd(dY, Ys, topk_w, dest_row, dYs, dtopk_w, dYs_q=None, dYs_q_scale=None,
                    stream=None):
    T, d = dY.shape
    k = topk_w.shape[1]
    _check(lib().moe_combine_bwd(_ptr(dY), _ptr(Ys), _ptr(topk_w), _ptr(dest_row), T, d, k,
                                 _dtype(dY), _ptr(dYs), _ptr(dtopk_w), _ptr(dYs_q),
                                 _ptr(dYs_q_scale), _stream(stream)), "moe_combine_bwd")


def moe_grouped_ffn_bwd(dYs, Xs, Hg, Hu, A, offsets, T, k, Wg, Wu, Wd, dH, dXs,
                        dWg, dWu, dWd, ws=None, prec="bf16", accumulate=False, dYs_q=None,
                        dYs_q_scale=None, stream=None, mx_wgrad=False, keep_weights=False):
    E, d, f = Wg.shape
    wp, wb = _ws(ws)
    # float32 weight gradients of a bf16 layer select float32 accumulation
    flags = (MOE_ACCUMULATE if accumulate else 0) | \
        (MOE_WGRAD_F32 if dWg.dtype == torch.float32 and Wg.dtype == torch.bfloat16 else 0) | \
        (MOE_WGRAD_MX if mx_wgrad else 0) | (MOE_MX_KEEP_WEIGHTS if keep_weights else 0)
    _check(lib().moe_grouped_ffn_bwd(_ptr(dYs), _ptr(dYs_q), _ptr(dYs_q_scale), _ptr(Xs),
                                     _ptr(Hg), _ptr(Hu), _ptr(A),
                                     _ptr(offsets), T, k, d, f, E, _ptr(Wg),
                                     _ptr(Wu), _ptr(Wd), _dtype(Wg), PREC[prec],
                                     flags, _ptr(dH), _ptr(dXs),
                                     _ptr(dWg), _ptr(dWu), _ptr(dWd), wp, wb, _stream(stream)),
           "moe_grouped_ffn_bwd")


def moe_dispatch_bwd(dXs, dest_row, dx, accumulate=False, stream=None):
    T, d = dx.shape
    k = dest_row.shape[1]
    _check(lib().moe_dispatch_bwd(_ptr(dXs), _ptr(dest_row), T, d, k, _dtype(dx),
                                  MOE_ACCUMULATE if accumulate else 0, _ptr(dx), _stream(stream)),
           "moe_dispatch_bwd")


def moe_route_bwd(x, Wr, logits, topk_idx, dtopk_w, dlogits, dWr, dx, ws=None, accumulate=False,
                  renorm=False, aux_dp=None, stream=None):
    T, d = x.shape
    E = Wr.shape[1]
    k = topk_idx.shape[1]
    wp, wb = _ws(ws)
    flags = (MOE_ACCUMULATE if accumulate else 0) | (MOE_ROUTE_RENORM if renorm else 0)
    _check(lib().moe_route_bwd(_ptr(x), _ptr(Wr), _ptr(logits), _ptr(topk_idx), _ptr(dtopk_w),
                               _ptr(aux_dp), T, d, E, k, _dtype(x), flags, _ptr(dlogits),
                               _ptr(dWr), _ptr(dx), wp, wb, _stream(stream)),
           "moe_route_bwd")


def moe_route_aux(logits, counts, k, coef, aux_loss, aux_dp, ws, stream=None):
    T, E = logits.shape
    wp, wb = _ws(ws)
    _check(lib().moe_route_aux(_ptr(logits), _ptr(counts), T, E, k, float(coef), _ptr(aux_loss),
                               _ptr(aux_dp), wp, wb, _stream(stream)), "moe_route_aux")


class KernelTimer:
    """Per-kernel durations through moe_set_kernel_events: a start event, then
    one event after every kernel the library launches on this thread.  With
    only="<label>" (moe_set_kernel_filter), just that kernel is timed, by an
    event right before and one right after each of its launches, and the
    other kernels run with no events between them."""

    def __init__(self, capacity: int = 4096, only: str | None = None):
        self.capacity = capacity
        self.only = only
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        self.start = torch.cuda.Event(enable_timing=True)
        self._names = (ctypes.c_char_p * capacity)()
        self._count = ctypes.c_int(0)
        self._handles = None

    def __enter__(self):
        # torch creates the HIP events lazily, on their first record()
        for e in self.events:
            e.record()
        torch.cuda.synchronize()
        handles = [e.cuda_event for e in self.events]
        if not all(handles):
            raise RuntimeError("KernelTimer: torch did not create the HIP events")
        self._handles = (ctypes.c_void_p * self.capacity)(*handles)
        self.start.record()
        _check(lib().moe_set_kernel_filter(self.only.encode() if self.only else None),
               "moe_set_kernel_filter")
        _check(lib().moe_set_kernel_events(self._handles, self._names, self.capacity,
                                           ctypes.byref(self._count)), "moe_set_kernel_events")
        return self

    def __exit__(self, *exc):
        lib().moe_set_kernel_events(None, None, 0, None)
        lib().moe_set_kernel_filter(None)
        return False

    def durations(self):
        """[(kernel name, milliseconds)] in launch order (after synchronising)."""
        torch.cuda.synchronize()
        if self._count.value < 0:
            raise RuntimeError(f"KernelTimer: hipEventRecord failed (HIP error {-self._count.value})")
        if self.only:
            return [(self._names[i].decode(), self.events[i].elapsed_time(self.events[i + 1]))
                    for i in range(0, self._count.value, 2)]
        out, prev = [], self.start
        for i in range(self._count.value):
            out.append((self._names[i].decode(), prev.elapsed_time(self.events[i])))
            prev = self.events[i]
        return out


class ExpertLayer:
    """Buffers and launch order of one MoE expert layer, forward and backward.

    router=True: top-k softmax router on x.Wr (or on given logits), with the
    top-k weights renormalised to sum to 1 when renorm=True, and the
    load-balancing loss (coefficient aux_coef, into aux_loss) and its
    gradient added to the router backward when aux_coef != 0.
    wgrad_f32=True keeps the expert weight gradients dWg, dWu, dWd in float32
    (float32 accumulation with backward(..., accumulate_wgrad=True)).
    mx_wgrad=True (prec "mxfp8"): the weight-gradient GEMMs run in MXFP8 too.
    router=False: pre-routed rows (topk_idx / topk_w are inputs, no router
    backward).  All buffers are allocated once, on construction."""

    def __init__(self, T: int, d: int, E: int, f: int, k: int, dtype=torch.bfloat16,
                 prec: str = "bf16", router: bool = True, device="cuda", renorm: bool = False,
                 aux_coef: float = 0.0, wgrad_f32: bool = False, mx_wgrad: bool = False):
        lib()
        self.T, self.d, self.E, self.f, self.k = T, d, E, f, k
        self.R = R = T * k
        self.dtype, self.prec, self.router = dtype, prec, router
        self.renorm, self.aux_coef = renorm, float(aux_coef)
        self.mx_wgrad = bool(mx_wgrad)
        dev = torch.device(device)
        z = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)
        i32, f32 = torch.int32, torch.float32
        self.logits = z(T, E, dt=f32)
        self.topk_idx = z(T, k, dt=i32)
        self.topk_w = z(T, k, dt=f32)
        self.counts = z(E, dt=i32)
        self.offsets = z(E + 1, dt=i32)
        self.dest_row = z(T, k, dt=i32)
        self.src_token = z(R, dt=i32)
        self.Xs = z(R, d)
        if prec == "mxfp8":
            self.Xq = z(R, d, dt=torch.uint8)
            self.Xq_scale = z(*mx_scale_shape(R, d), dt=torch.uint8)
            self.dYs_q = z(R, d, dt=torch.uint8)
            self.dYs_q_scale = z(*mx_scale_shape(R, d), dt=torch.uint8)
        else:
            self.Xq = self.Xq_scale = self.dYs_q = self.dYs_q_scale = None
        self.Hg, self.Hu, self.A = z(R, f), z(R, f), z(R, f)
        self.Ys = z(R, d)
        self.y = z(T, d)
        self.dYs = z(R, d)
        self.dw = z(T, k, dt=f32)
        self.dH = z(R, 2 * f)
        self.dXs = z(R, d)
        self.dx = z(T, d)
        wdt = torch.float32 if wgrad_f32 else dtype
        self.dWg, self.dWu, self.dWd = z(E, d, f, dt=wdt), z(E, d, f, dt=wdt), z(E, f, d, dt=wdt)
        self.dlogits = z(T, E, dt=f32)
        self.dWr = z(d, E)
        self.aux_loss = z(1, dt=f32)
        self.aux_dp = z(E, dt=f32)

        def ws(op):
            n = moe_workspace_size(op, T, d, E, f, k, dtype, prec)
            return torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.ws_route = ws("route")
        self.ws_dispatch = ws("dispatch")
        bwd_op = "ffn_bwd_mxw" if self.mx_wgrad else "ffn_bwd"
        if prec == "mxfp8":
            # one workspace for both directions: the forward quantises each
            # weight once and keeps the backward's codes in its part, which
            # the backward reads (MOE_MX_KEEP_WEIGHTS)
            nf = moe_workspace_size("ffn_fwd_keep", T, d, E, f, k, dtype, prec)
            nb = moe_workspace_size(bwd_op, T, d, E, f, k, dtype, prec)
            self.ws_bwd = torch.empty(nf + nb, dtype=torch.uint8, device=dev)
            self.ws_fwd = self.ws_bwd[:nf]
        else:
            self.ws_fwd = ws("ffn_fwd")
            self.ws_bwd = ws(bwd_op)
        self.ws_route_bwd = ws("route_bwd")
        self.ws_route_aux = ws("route_aux")

    def forward(self, x, Wr, Wg, Wu, Wd, topk_idx=None, topk_w=None, logits=None, stream=None):
        self.x, self.Wr, self.Wg, self.Wu, self.Wd = x, Wr, Wg, Wu, Wd
        if self.router:
            if logits is not None:
                self.logits.copy_(logits)
            moe_route(x, Wr, self.k, self.logits, self.topk_idx, self.topk_w,
                      logits_in=logits is not None, renorm=self.renorm, ws=self.ws_route,
                      stream=stream)
        else:
            self.topk_idx.copy_(topk_idx)
            self.topk_w.copy_(topk_w)
        moe_dispatch(x, self.topk_idx, self.E, self.counts, self.offsets, self.dest_row,
                     self.src_token, self.Xs, self.ws_dispatch, self.Xq, self.Xq_scale, self.prec,
                     stream)
        if self.router and self.aux_coef != 0.0:
            moe_route_aux(self.logits, self.counts, self.k, self.aux_coef, self.aux_loss,
                          self.aux_dp, self.ws_route_aux, stream)
        mx = self.prec == "mxfp8"
        moe_grouped_ffn_fwd(self.Xq if mx else self.Xs, self.Xq_scale, self.offsets, self.T,
                            self.k, Wg, Wu, Wd, self.Hg, self.Hu, self.A, self.Ys, self.ws_fwd,
                            self.prec, stream, keep_weights=mx)
        moe_combine(self.Ys, self.topk_w, self.dest_row, self.y, stream)
        return self.y

    def backward(self, dY, stream=None, accumulate_wgrad: bool = False):
        moe_combine_bwd(dY, self.Ys, self.topk_w, self.dest_row, self.dYs, self.dw, self.dYs_q,
                        self.dYs_q_scale, stream)
        moe_grouped_ffn_bwd(self.dYs, self.Xs, self.Hg, self.Hu, self.A, self.offsets, self.T, self.k,
                            self.Wg, self.Wu, self.Wd, self.dH, self.dXs, self.dWg, self.dWu,
                            self.dWd, self.ws_bwd, self.prec, accumulate_wgrad, self.dYs_q,
                            self.dYs_q_scale, stream, mx_wgrad=self.mx_wgrad,
                            keep_weights=self.prec == "mxfp8")
        moe_dispatch_bwd(self.dXs, self.dest_row, self.dx, False, stream)
        if self.router:
            aux = self.aux_dp if self.aux_coef != 0.0 else None
            moe_route_bwd(self.x, self.Wr, self.logits, self.topk_idx, self.dw, self.dlogits,
                          self.dWr, self.dx, self.ws_route_bwd, False, self.renorm, aux, stream)
        return self.dx
