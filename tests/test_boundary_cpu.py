"""The C-ABI library on the host: it loads, exports every entry point that
include/moe.h declares, sizes workspaces, and rejects bad arguments with the
documented status before anything is enqueued (no call here reaches a kernel
launch, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WS, UNSUP, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -8
F32, BF16 = 0, 1
P_F32, P_BF16, P_MX = 0, 1, 2

# Fake device addresses: never dereferenced, because every call below fails
# validation before it could launch anything.
A = 0x10000          # 16-byte aligned
MIS = 0x10008        # misaligned


@pytest.fixture(scope="module")
def L():
    import routing_grouped_gemm_amd as rgg
    if not os.path.exists(rgg.LIB_PATH):
        pytest.fail("libmoe_hip.so is not built (python -m routing_grouped_gemm_amd.build)")
    return rgg.lib()


def declared_entry_points():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(moe_\w+)\(", txt, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_entry_points()
    assert len(names) == 17, names
    for n in names:
        assert hasattr(L, n), n


def test_kernel_event_hook_switches(L):
    # switching the hook on and off needs no device
    cnt = ctypes.c_int(5)
    assert L.moe_set_kernel_events(None, None, 0, ctypes.byref(cnt)) == OK and cnt.value == 0
    ev = (ctypes.c_void_p * 4)()
    assert L.moe_set_kernel_events(ev, None, 0, None) == SHAPE
    assert L.moe_set_kernel_events(ev, None, 4, ctypes.byref(cnt)) == OK and cnt.value == 0
    assert L.moe_set_kernel_events(None, None, 0, None) == OK
    # the name filter is copied; a name of 64 characters or more is refused
    assert L.moe_set_kernel_filter(b"gemm_fwd_gateup_swiglu") == OK
    assert L.moe_set_kernel_filter(b"x" * 63) == OK
    assert L.moe_set_kernel_filter(b"x" * 64) == SHAPE
    assert L.moe_set_kernel_filter(None) == OK


def test_status_strings(L):
    for s in (OK, NULL, SHAPE, DTYPE, ALIGN, WS, UNSUP, -7, SCRATCH):
        assert L.moe_status_string(s)
    assert b"unknown" in L.moe_status_string(12345)
    assert L.moe_last_launch_error() == b"none"


def ws_size(L, op, T, d, E, f, k, dtype, prec):
    out = ctypes.c_size_t(7)
    s = L.moe_workspace_size(op, T, d, E, f, k, dtype, prec, ctypes.byref(out))
    return s, out.value


def test_workspace_sizes(L):
    # dispatch: two int32 tables of E * ceil(T/64), each rounded up to 256 bytes
    s, n = ws_size(L, 1, 8192, 2048, 64, 1024, 8, BF16, P_BF16)
    assert s == OK and n == 2 * 128 * 64 * 4
    s, n = ws_size(L, 1, 100, 64, 3, 64, 1, F32, P_F32)
    assert s == OK and n == 2 * 256
    # route backward: bf16 copy of dlogits (E padded to 64) plus float32 dWr
    # partials of 32 token chunks; none in fp32
    assert ws_size(L, 7, 8192, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 8192 * 64 * 2 + 32 * 2048 * 64 * 4)
    assert ws_size(L, 7, 100, 64, 6, 64, 2, BF16, P_BF16) == (OK, 100 * 64 * 2)  # E % 8: no split
    assert ws_size(L, 7, 256, 64, 8, 128, 2, F32, P_F32) == (OK, 0)
    # small batches: router partial logits (slices of 128 rows of Wr) and the
    # float partial sums of the sliced small-batch expert GEMMs
    assert ws_size(L, 0, 1, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 16 * 1 * 64 * 4)
    assert ws_size(L, 0, 64, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 16 * 64 * 64 * 4)
    assert ws_size(L, 0, 65, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 0)     # general router
    assert ws_size(L, 0, 8, 2048, 6, 1024, 2, BF16, P_BF16) == (OK, 0)      # E % 8 != 0
    assert ws_size(L, 0, 8, 2048, 64, 1024, 8, F32, P_F32) == (OK, 0)
    # T=1, top-8 of 64: 8 experts x 16 column blocks, sliced 4 ways (gate/up
    # and down) into float partials
    assert ws_size(L, 2, 1, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 4 * 8 * 2048 * 4)
    assert ws_size(L, 2, 64, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 0)    # 1024 workgroups
    assert ws_size(L, 2, 8192, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 0)   # general engine
    # load-balancing loss: float32 partial sums of E per 64-token block
    assert ws_size(L, 8, 8192, 2048, 64, 1024, 8, BF16, P_BF16) == (OK, 128 * 64 * 4)
    assert ws_size(L, 8, 100, 64, 3, 64, 1, F32, P_F32) == (OK, 256)
    for op in (0, 2, 3, 4, 5, 6):
        assert ws_size(L, op, 256, 64, 8, 128, 2, BF16, P_BF16) == (OK, 0)
    assert ws_size(L, 1, 0, 64, 8, 128, 2, BF16, P_BF16)[0] == SHAPE
    assert ws_size(L, 1, 8, 64, 8, 128, 2, F32, P_BF16)[0] == DTYPE
    assert ws_size(L, 1, 8, 64, 8, 128, 2, BF16, 7)[0] == DTYPE
    assert ws_size(L, 99, 8, 64, 8, 128, 2, BF16, P_BF16)[0] == SHAPE
    assert L.moe_workspace_size(1, 8, 64, 8, 128, 2, BF16, P_BF16, None) == NULL
    # MXFP8: quantised copies of the three weights (1 byte per element, one
    # scale byte per 32) plus the quantised activations of the second GEMM
    T, d, E, f, k = 8192, 2048, 64, 1024, 8
    R = T * k
    s, n = ws_size(L, 2, T, d, E, f, k, BF16, P_MX)
    assert s == OK and 3 * E * d * f * 33 // 32 + R * f * 33 // 32 <= n <= 3 * E * d * f * 1.1 + R * f * 1.1
    s, n = ws_size(L, 5, T, d, E, f, k, BF16, P_MX)
    assert s == OK and 3 * E * d * f * 33 // 32 + R * 2 * f * 33 // 32 <= n  # weights + dH codes
    assert ws_size(L, 2, T, d, E, f, k, F32, P_MX)[0] == DTYPE
    # MXFP8 weight gradients: the dgrad workspace, then the padded offsets and
    # the token-quantised operands (codes [max(d,f)][Kp], [max(2f,d)][Kp] with
    # Kp = R + 127 E rounded up to 128, one scale byte per 32 codes)
    s, n = ws_size(L, 9, T, d, E, f, k, BF16, P_MX)
    Kp = (R + 127 * E + 127) // 128 * 128
    assert s == OK and n >= ws_size(L, 5, T, d, E, f, k, BF16, P_MX)[1] + 2 * 2048 * Kp * 33 // 32
    assert ws_size(L, 9, T, d, E, f, k, BF16, P_BF16)[0] == DTYPE


def route(L, x=A, Wr=A, T=16, d=64, E=8, k=2, dt=BF16, flags=0, lg=A, idx=A, w=A):
    return L.moe_route(x, Wr, T, d, E, k, dt, flags, lg, idx, w, None, 0, None)


def test_route_validation(L):
    assert route(L, x=None) == NULL
    assert route(L, lg=None) == NULL
    assert route(L, T=0) == SHAPE
    assert route(L, k=0) == SHAPE
    assert route(L, T=1 << 28, k=16, E=16) == SHAPE      # T*k overflows int32
    assert route(L, E=300, k=2) == UNSUP
    assert route(L, E=4, k=5) == UNSUP
    assert route(L, d=96) == UNSUP
    assert route(L, dt=5) == DTYPE
    assert route(L, x=MIS) == ALIGN
    assert route(L, idx=MIS) == ALIGN


def dispatch(L, T=16, d=64, E=8, k=2, dt=BF16, prec=P_BF16, ws=A, wsb=1 << 20, xs=A, xq=A, sc=A,
             x=A):
    return L.moe_dispatch(x, A, T, d, E, k, dt, prec, A, A, A, A, xs, xq, sc, ws, wsb, None)


def test_dispatch_validation(L):
    assert dispatch(L, ws=None) == NULL
    assert dispatch(L, xs=None) == NULL
    assert dispatch(L, dt=F32, prec=P_BF16) == DTYPE
    assert dispatch(L, dt=BF16, prec=P_F32) == DTYPE
    assert dispatch(L, d=100) == UNSUP
    assert dispatch(L, x=MIS) == ALIGN
    assert dispatch(L, wsb=2 * 256 - 1) == WS
    assert dispatch(L, prec=P_MX, xq=None) == NULL      # MXFP8 needs the codes
    assert dispatch(L, prec=P_MX, sc=None) == NULL      # ... and the scales
    assert dispatch(L, prec=P_MX, sc=MIS) == ALIGN
    assert dispatch(L, prec=P_MX, dt=F32) == DTYPE


def ffn_fwd(L, T=16, k=2, d=64, f=64, E=8, dt=BF16, prec=P_BF16, Xs=A, Wg=A):
    return L.moe_grouped_ffn_fwd(Xs, A, A, T, k, d, f, E, Wg, A, A, dt, prec, 0, A, A, A, A,
                                 A, 1 << 20, None)


def test_ffn_fwd_validation(L):
    assert ffn_fwd(L, Xs=None) == NULL
    assert ffn_fwd(L, f=96) == UNSUP
    assert ffn_fwd(L, f=0) == SHAPE
    assert ffn_fwd(L, dt=F32) == DTYPE
    assert ffn_fwd(L, Wg=MIS) == ALIGN
    assert ffn_fwd(L, E=257) == UNSUP


def ffn_bwd(L, Xs=A, dt=BF16, prec=P_BF16, f=64, dH=A, ws=A, dq=A, dqs=A):
    return L.moe_grouped_ffn_bwd(A, dq, dqs, Xs, A, A, A, A, 16, 2, 64, f, 8, A, A, A, dt, prec,
                                 0, dH, A, A, A, A, ws, 1 << 20, None)


def test_ffn_bwd_mx_weight_gradient_flag(L):
    # MOE_WGRAD_MX needs the MXFP8 precision and its larger workspace
    f = L.moe_grouped_ffn_bwd
    args = lambda prec, flags, wsb: (A, A, A, A, A, A, A, A, 16, 2, 64, 64, 8, A, A, A, BF16, prec,
                                     flags, A, A, A, A, A, A, wsb, None)
    assert f(*args(P_BF16, 0x10, 1 << 30)) == DTYPE
    assert f(*args(P_MX, 0x10, 4096)) == WS


def test_ffn_bwd_validation(L):
    assert ffn_bwd(L, Xs=None) == NULL             # the weight gradients read Xs
    assert ffn_bwd(L, Xs=None, prec=P_MX) == NULL
    assert ffn_bwd(L, ws=None, prec=P_MX) == NULL  # MXFP8 quantises into the workspace
    assert ffn_bwd(L, dq=None, prec=P_MX) == NULL  # ... and reads the quantised dYs
    assert ffn_bwd(L, dqs=MIS, prec=P_MX) == ALIGN
    assert ffn_bwd(L, dH=None) == NULL
    assert ffn_bwd(L, f=32) == UNSUP
    assert ffn_bwd(L, dH=MIS) == ALIGN
    assert ffn_bwd(L, dt=F32, prec=P_MX) == DTYPE


def test_combine_and_gather_validation(L):
    assert L.moe_combine(A, A, A, 16, 64, 2, BF16, None, None) == NULL
    assert L.moe_combine(A, A, A, 0, 64, 2, BF16, A, None) == SHAPE
    assert L.moe_combine(A, A, A, 16, 72, 2, BF16, A, None) == UNSUP
    assert L.moe_combine(A, A, A, 16, 64, 2, BF16, MIS, None) == ALIGN
    assert L.moe_combine_bwd(A, A, A, A, 16, 64, 2, 9, A, A, None, None, None) == DTYPE
    assert L.moe_combine_bwd(A, A, A, A, 16, 64, 2, BF16, A, A, A, None, None) == NULL  # codes w/o scales
    assert L.moe_combine_bwd(A, A, A, A, 16, 64, 2, F32, A, A, A, A, None) == DTYPE     # MX codes need bf16
    assert L.moe_combine_bwd(A, A, A, A, 16, 64, 2, BF16, A, A, A, MIS, None) == ALIGN
    assert L.moe_dispatch_bwd(A, A, 16, 64, 0, BF16, 0, A, None) == SHAPE
    assert L.moe_dispatch_bwd(None, A, 16, 64, 2, BF16, 0, A, None) == NULL


def test_route_bwd_validation(L):
    f = L.moe_route_bwd
    assert f(A, A, A, A, A, None, 16, 64, 8, 2, BF16, 0, A, A, A, None, 0, None) == NULL  # bf16 needs ws
    assert f(A, A, A, A, A, None, 16, 64, 8, 2, BF16, 0, A, A, A, A, 16 * 8 * 2 - 1, None) == WS
    assert f(A, A, A, A, A, None, 16, 64, 8, 2, BF16, 0, A, A, MIS, A, 1 << 20, None) == ALIGN
    assert f(A, A, A, A, A, MIS, 16, 64, 8, 2, BF16, 4, A, A, A, A, 1 << 20, None) == ALIGN
    assert f(A, A, A, A, A, None, 16, 64, 8, 9, BF16, 0, A, A, A, A, 1 << 20, None) == UNSUP


def test_route_aux_validation(L):
    f = L.moe_route_aux
    assert f(None, A, 16, 8, 2, 0.01, A, A, A, 256, None) == NULL
    assert f(A, A, 16, 8, 2, 0.01, A, None, A, 256, None) == NULL
    assert f(A, A, 16, 8, 2, 0.01, A, A, None, 256, None) == NULL
    assert f(A, A, 0, 8, 2, 0.01, A, A, A, 256, None) == SHAPE
    assert f(A, A, 16, 8, 9, 0.01, A, A, A, 256, None) == UNSUP
    assert f(A, A, 16, 8, 2, float("nan"), A, A, A, 256, None) == SHAPE
    assert f(A, MIS, 16, 8, 2, 0.01, A, A, A, 256, None) == ALIGN
    assert f(A, A, 200, 8, 2, 0.01, A, A, A, 4 * 8 * 4 - 1, None) == WS


def test_ffn_offset_limits(L):
    """Shapes whose operands would pass the GEMM engines' 32-bit byte offsets
    are refused with MOE_ERR_UNSUPPORTED before anything else; just inside
    the limit the call gets as far as the alignment check (a misaligned
    pointer makes it stop there, so nothing is launched)."""
    fwd = lambda T, k, d, f, Wg=A: L.moe_grouped_ffn_fwd(A, A, A, T, k, d, f, 8, Wg, A, A, BF16,
                                                         P_BF16, 0, A, A, A, A, A, 1 << 20, None)
    # one expert's weights: d * (f + 128) * 2 bytes below 2^32
    assert fwd(16, 2, 65536, 32768) == UNSUP
    assert fwd(16, 2, 32768, 32640, Wg=MIS) == ALIGN

    def bwd(T, k, d, f, flags=0, prec=P_BF16, dH=A):
        return L.moe_grouped_ffn_bwd(A, A, A, A, A, A, A, A, T, k, d, f, 8, A, A, A, BF16, prec,
                                     flags, dH, A, A, A, A, A, 1 << 20, None)
    # bf16 weight gradients: R * max(d, 2f) * 2 bytes below 2^32
    assert bwd(1 << 20, 2, 1024, 512) == UNSUP            # R = 2^21, width 1024
    assert bwd((1 << 20) - 1, 2, 1024, 512, dH=MIS) == ALIGN
    assert bwd(1 << 19, 2, 512, 1024) == UNSUP            # width 2f = 2048
    assert bwd(1 << 16, 1, 7168, 2048, dH=MIS) == ALIGN   # one GPU's share of a 1T MoE
    assert bwd(300000, 1, 7168, 2048) == UNSUP            # ~300k rows at d = 7168
    # MXFP8 weight gradients: 256 * Kp and (Kp / 32) * max(d, 2f) below 2^32
    assert bwd(1 << 23, 2, 64, 64, flags=0x10, prec=P_MX) == UNSUP    # Kp >= 2^24
    assert bwd(1 << 21, 2, 64, 64, flags=0x10, prec=P_MX, dH=MIS) == ALIGN
    assert bwd(1 << 21, 1, 65536, 64, flags=0x10, prec=P_MX) == UNSUP  # scale column
    # MXFP8 activation scales: ceil(max(d, 2f) / 128) * 4 * Rp bytes below 2^30
    fwd_mx = lambda T, k, d, f, Wg=A: L.moe_grouped_ffn_fwd(A, A, A, T, k, d, f, 8, Wg, A, A, BF16,
                                                            P_MX, 0, A, A, A, A, A, 1 << 20, None)
    assert fwd_mx(1 << 20, 8, 4096, 64) == UNSUP                      # 32 * 4 * 2^23 = 2^30
    assert fwd_mx((1 << 20) - 16, 8, 4096, 64, Wg=MIS) == ALIGN       # 2^30 - 2^14
    # (in the backward the weight-gradient limits are the tighter ones)


def test_dispatch_noalloc_validation(L):
    """The no-allocation dispatch checks its arguments like moe_dispatch and
    refuses a problem whose tables exceed its 4 MiB static scratch before it
    touches any device (2 * ceil(T/64) * E * 4 bytes, each table padded to
    256 bytes)."""
    f = L.moe_dispatch_noalloc
    args = lambda T, E, x=A, xs=A, prec=P_BF16: (x, A, T, 64, E, 2, BF16, prec, A, A, A, A, xs,
                                                 A, A, None)
    assert f(*args(16, 8, x=None)) == NULL
    assert f(*args(16, 8, xs=MIS)) == ALIGN
    assert f(*args(16, 300)) == UNSUP
    assert f(*args(1 << 20, 64)) == SCRATCH          # 2 * 16384 * 64 * 4 B = 8 MiB
    assert f(*args(1 << 19, 64 + 1)) == SCRATCH       # just over 4 MiB
    assert f(*args(1 << 18, 256, prec=P_MX)) == SCRATCH   # 8 MiB


def test_mx_keep_weights_flag(L):
    """MOE_MX_KEEP_WEIGHTS exists for the MXFP8 precision only, and both
    directions check that the workspace holds the kept codes."""
    KEEP = 0x20
    fwd = lambda prec, flags, wsb: L.moe_grouped_ffn_fwd(A, A, A, 16, 2, 64, 64, 8, A, A, A, BF16,
                                                         prec, flags, A, A, A, A, A, wsb, None)
    assert fwd(P_BF16, KEEP, 1 << 30) == DTYPE
    need = ws_size(L, 10, 16, 64, 8, 64, 2, BF16, P_MX)[1]
    plain = ws_size(L, 2, 16, 64, 8, 64, 2, BF16, P_MX)[1]
    assert need > plain > 0
    assert fwd(P_MX, KEEP, need - 1) == WS
    assert fwd(P_MX, 0, plain - 1) == WS
    bwd = lambda prec, flags, wsb: L.moe_grouped_ffn_bwd(A, A, A, A, A, A, A, A, 16, 2, 64, 64, 8,
                                                         A, A, A, BF16, prec, flags, A, A, A, A,
                                                         A, A, wsb, None)
    own = ws_size(L, 5, 16, 64, 8, 64, 2, BF16, P_MX)[1]
    assert bwd(P_BF16, KEEP, 1 << 30) == DTYPE
    assert bwd(P_MX, KEEP, need + own - 1) == WS
    out = ctypes.c_size_t(0)
    assert L.moe_workspace_size(10, 16, 64, 8, 64, 2, BF16, P_BF16, ctypes.byref(out)) == DTYPE


def test_check_routing_validation(L):
    f = L.moe_check_routing
    assert f(None, 16, 8, 2, A, None) == NULL
    assert f(A, 16, 8, 2, None, None) == NULL
    assert f(A, 0, 8, 2, A, None) == SHAPE
    assert f(A, 16, 300, 2, A, None) == UNSUP
    assert f(A, 16, 8, 2, MIS, None) == ALIGN


def test_mx_activation_scale_layout():
    """mx_scale_shape / mx_scale_rows follow the byte layout include/moe.h
    documents for the activation scales: block b of row r at byte
    ((b / 4) * Rp + r) * 4 + b % 4 (Rp = R rounded up to 16), including a
    partial last group (d = 576: 18 blocks) and rows past R in the pitch."""
    import torch
    import routing_grouped_gemm_amd as rgg
    for R, K in ((37, 576), (16, 128), (1, 64), (300, 4096)):
        G, Rp, four = rgg.mx_scale_shape(R, K)
        assert (G, Rp, four) == (-(-K // 128), -(-R // 16) * 16, 4)
        flat = torch.full((G * Rp * 4,), 255, dtype=torch.int64)
        for r in range(R):
            for b in range(K // 32):
                flat[((b // 4) * Rp + r) * 4 + b % 4] = (r * 7 + b * 3) % 251
        rows = rgg.mx_scale_rows(flat.reshape(G, Rp, 4), R, K)
        assert tuple(rows.shape) == (R, K // 32)
        want = (torch.arange(R)[:, None] * 7 + torch.arange(K // 32)[None, :] * 3) % 251
        assert torch.equal(rows, want)
