"""Inference-shaped small batches (1, 8 and 64 tokens of the OLMoE layer):
the forward pass against the oracle, and the forward captured once in a HIP
graph and replayed, against eager launches."""
import numpy as np
import pytest
import torch

from moe_synth import make_inputs, workload
from oracle import moe_oracle as O
from tests.parity import EXACT, TOL, dev_tensor, relerr, say, to_np

pytestmark = pytest.mark.gpu

FWD = ("Xs", "Hg", "Hu", "A", "Ys", "y")


def _case(name, seed=0):
    wl = workload(name)
    say(f"[case] {name}: T={wl.T} d={wl.d} E={wl.E} f={wl.f} k={wl.k} seed={seed}")
    inp = make_inputs(wl, seed=seed, with_dY=False)
    return wl, inp


def _layer(wl, inp):
    import routing_grouped_gemm_amd as rgg
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, torch.bfloat16, wl.prec, router=True)
    ops = {n: dev_tensor(inp, n, torch.bfloat16) for n in ("x", "Wr", "Wg", "Wu", "Wd")}
    return layer, ops


@pytest.mark.parametrize("name", ["olmoe_decode_t1", "olmoe_decode_t8", "olmoe_decode_t64"])
def test_small_batch_forward(name):
    import routing_grouped_gemm_amd as rgg
    wl, inp = _case(name)
    logits = O.router_logits(inp["x"], inp["Wr"], wl.prec)
    ref = O.layer(inp["x"], inp["Wr"], inp["Wg"], inp["Wu"], inp["Wd"], wl.k, None, wl.prec,
                  logits=logits)
    layer, o = _layer(wl, inp)
    layer.forward(o["x"], o["Wr"], o["Wg"], o["Wu"], o["Wd"],
                  logits=rgg.upload(np.ascontiguousarray(logits, np.float32)))
    torch.cuda.synchronize()
    for n in EXACT:
        np.testing.assert_array_equal(to_np(getattr(layer, n)), np.asarray(ref[n]), err_msg=n)
    errs = {n: relerr(to_np(getattr(layer, n)), ref[n]) for n in FWD}
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


@pytest.mark.parametrize("name", ["olmoe_decode_t1", "olmoe_decode_t64"])
def test_forward_graph_replays_match_eager(name):
    """One capture, three replays with eager launches and host reads in
    between; every replay's output equals the eager output bit for bit."""
    wl, inp = _case(name, seed=1)
    layer, o = _layer(wl, inp)

    def fwd():
        layer.forward(o["x"], o["Wr"], o["Wg"], o["Wu"], o["Wd"])

    fwd()
    torch.cuda.synchronize()
    want = {n: getattr(layer, n).clone() for n in ("topk_idx", "counts", "offsets", "Ys", "y")}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for rep in range(3):
        layer.y.zero_()
        layer.Ys.zero_()
        g.replay()
        torch.cuda.synchronize()
        for n, t in want.items():
            assert torch.equal(getattr(layer, n), t), (rep, n)
        fwd()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(layer.y, want["y"])


@pytest.mark.parametrize("name,renorm", [("olmoe_decode_t1", False), ("olmoe_decode_t8", True),
                                         ("olmoe_decode_t64", False)])
def test_small_batch_router(name, renorm):
    """The one-kernel small-batch router: logits against the oracle's, top-k
    a valid choice on its own logits (bit-exact where the k-th and (k+1)-th
    logits are apart), weights the (renormalised) softmax probabilities."""
    import routing_grouped_gemm_amd as rgg
    wl, inp = _case(name, seed=2)
    layer, o = _layer(wl, inp)
    layer.renorm = renorm
    layer.forward(o["x"], o["Wr"], o["Wg"], o["Wu"], o["Wd"])
    torch.cuda.synchronize()
    ref_logits = O.router_logits(inp["x"], inp["Wr"], wl.prec)
    lg = to_np(layer.logits)
    err = relerr(lg, ref_logits)
    say(f"  logits relerr {err:.2e}")
    assert err <= 1e-5
    idx = to_np(layer.topk_idx)
    own_idx, own_w, _ = O.route(lg, wl.k, "fp32", renorm)
    np.testing.assert_array_equal(idx, own_idx)
    np.testing.assert_allclose(to_np(layer.topk_w), own_w, rtol=4e-6, atol=0)
    srt = np.sort(ref_logits, axis=1)[:, ::-1]
    safe = (srt[:, wl.k - 1] - srt[:, wl.k]) > 4 * np.max(np.abs(lg - ref_logits))
    np.testing.assert_array_equal(idx[safe], O.topk_select(ref_logits, wl.k)[safe])
