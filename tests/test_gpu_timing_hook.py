"""The per-kernel timing hook on the GPU: an event after every kernel, or,
under a name filter, events right before and after each launch of one
kernel only (moe_set_kernel_events, moe_set_kernel_filter)."""
import pytest
import torch

from tests.parity import say

pytestmark = pytest.mark.gpu

T, D, E, F, K = 512, 2048, 64, 1024, 8   # 4096 routed rows: the 256x256 GEMM engine
GATEUP = "gemm_fwd_gateup_swiglu"


def _layer():
    import routing_grouped_gemm_amd as rgg
    say(f"[case] timing hook: T={T} d={D} E={E} f={F} k={K} bf16")
    g = torch.Generator(device="cpu").manual_seed(5)
    r = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc).to(torch.bfloat16).cuda()
    ops = dict(x=r(T, D), Wr=r(D, E, sc=0.02), Wg=r(E, D, F, sc=0.02), Wu=r(E, D, F, sc=0.02),
               Wd=r(E, F, D, sc=0.02))
    layer = rgg.ExpertLayer(T, D, E, F, K, torch.bfloat16, "bf16", router=True)
    fwd = lambda: layer.forward(ops["x"], ops["Wr"], ops["Wg"], ops["Wu"], ops["Wd"])
    fwd()
    torch.cuda.synchronize()
    return rgg, fwd


def test_every_kernel_then_one_kernel():
    rgg, fwd = _layer()
    full = rgg.KernelTimer(capacity=256)
    with full:
        fwd()
    every = full.durations()
    names = [n for n, _ in every]
    say(f"  every kernel: {names}")
    assert GATEUP in names and len(names) >= 5
    assert all(ms >= 0.0 for _, ms in every)

    # three forwards, only the gate/up GEMM bracketed: one pair of events each
    only = rgg.KernelTimer(capacity=64, only=GATEUP)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with only:
        a.record()
        for _ in range(3):
            fwd()
        b.record()
    runs = only.durations()
    total = a.elapsed_time(b)
    say(f"  {GATEUP} alone: {[round(ms, 4) for _, ms in runs]} ms of {total:.4f} ms")
    assert [n for n, _ in runs] == [GATEUP] * 3
    assert all(0.0 < ms < total for _, ms in runs)
    assert sum(ms for _, ms in runs) < total

    # leaving the filtered timer clears the filter: every kernel is seen again
    again = rgg.KernelTimer(capacity=256)
    with again:
        fwd()
    assert [n for n, _ in again.durations()] == names


def test_filter_on_a_kernel_not_launched_records_nothing():
    rgg, fwd = _layer()
    none = rgg.KernelTimer(capacity=16, only="no_such_kernel")
    with none:
        fwd()
    assert none.durations() == []
