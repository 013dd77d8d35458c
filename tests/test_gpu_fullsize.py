"""Parity at the benchmark sizes, on sampled outputs.

Each benchmark workload runs through the C ABI exactly as the benchmark runs
it (ExpertLayer forward + backward; with a router the oracle's float32
logits are passed in, so that the routing is comparable bit for bit).  The
oracle then evaluates the same definitions only where it is sampled
(oracle.layer_tokens for whole tokens and their rows, oracle.expert_columns
for weight-gradient columns of chosen experts).  Checks:
  * routing metadata (top-k, counts, offsets, dest_row, src_token): bit-exact
    over all tokens; topk_w within 1e-5;
  * every per-row and per-token output at the sampled tokens, and the weight
    gradients at the sampled columns: normwise relative error within the
    precision's bound (bf16 2e-2, MXFP8 6e-2);
  * experts with no rows get exactly zero weight gradients;
  * router weight gradient: dWr equals x^T . dlogits (the layer's own
    dlogits, a property that holds at any size) within the bf16 bound, and
    every dlogits row sums to ~0.
"""
import time

import numpy as np
import pytest
import torch

from moe_synth import make_inputs, workload
from oracle import moe_oracle as O
from tests.parity import TOL, dev_tensor, relerr, say, to_np

pytestmark = pytest.mark.gpu

FULL = ["olmoe_bf16", "escan_e8_bf16", "escan_e32_bf16", "escan_e128_bf16", "share1t_bf16",
        "olmoe_mxfp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    import routing_grouped_gemm_amd as rgg
    t0 = time.time()
    wl = workload(name)
    say(f"[full] {name}: T={wl.T} d={wl.d} E={wl.E} f={wl.f} k={wl.k} {wl.prec}")
    inp = make_inputs(wl, seed=0)
    router = wl.routing == "router"
    if router:
        logits = O.router_logits(inp["x"], inp["Wr"], wl.prec)
        idx, w, _ = O.route(logits, wl.k, wl.prec)
    else:
        logits, idx, w = None, inp["topk_idx"], inp["topk_w"]
    counts, offsets, dest_row, src_token = O.routing_metadata(idx, wl.E)
    say(f"  inputs and routing ready ({time.time() - t0:.0f} s)")

    dt = torch.bfloat16
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, dt, wl.prec, router=router)
    x = dev_tensor(inp, "x", dt)
    Wg, Wu, Wd = (dev_tensor(inp, n, dt) for n in ("Wg", "Wu", "Wd"))
    Wr = dev_tensor(inp, "Wr", dt) if router else None
    dY = dev_tensor(inp, "dY", dt)
    kw = dict(logits=rgg.upload(np.ascontiguousarray(logits, np.float32))) if router else \
        dict(topk_idx=rgg.upload(idx), topk_w=rgg.upload(w))
    layer.forward(x, Wr, Wg, Wu, Wd, **kw)
    layer.backward(dY)
    torch.cuda.synchronize()
    say(f"  layer ran ({time.time() - t0:.0f} s)")

    # routing metadata, bit for bit
    np.testing.assert_array_equal(to_np(layer.topk_idx), idx)
    np.testing.assert_array_equal(to_np(layer.counts), counts)
    np.testing.assert_array_equal(to_np(layer.offsets), offsets)
    np.testing.assert_array_equal(to_np(layer.dest_row), dest_row)
    np.testing.assert_array_equal(to_np(layer.src_token), src_token)
    assert relerr(to_np(layer.topk_w), w) <= 1e-5

    # sampled tokens
    rng = np.random.default_rng(7)
    ntok = 4 if wl.prec == "mxfp8" else 16
    tokens = np.sort(rng.choice(wl.T, ntok, replace=False))
    s = O.layer_tokens(inp["x"], inp.get("Wr"), inp["Wg"], inp["Wu"], inp["Wd"], idx, w,
                       inp["dY"], tokens, wl.prec, logits=logits)
    rows = torch.from_numpy(np.asarray(s["rows"], np.int64).reshape(-1)).cuda()
    tt = torch.from_numpy(tokens).cuda()
    tol = TOL[wl.prec]
    errs = {}
    f = wl.f

    def rowvals(t):
        return to_np(t.index_select(0, rows)).reshape(ntok, wl.k, -1)

    for key in ("Hg", "Hu", "A", "Ys", "dYs", "dXs"):
        errs[key] = relerr(rowvals(getattr(layer, key)), s[key])
    dH = rowvals(layer.dH)
    errs["dHg"] = relerr(dH[..., :f], s["dHg"])
    errs["dHu"] = relerr(dH[..., f:], s["dHu"])
    errs["y"] = relerr(to_np(layer.y.index_select(0, tt)), s["y"])
    errs["dx"] = relerr(to_np(layer.dx.index_select(0, tt)), s["dx"])
    errs["dw"] = relerr(to_np(layer.dw.index_select(0, tt)), s["dw"])
    if router:
        errs["dlogits"] = relerr(to_np(layer.dlogits.index_select(0, tt)), s["dlogits"])
    say(f"  tokens checked ({time.time() - t0:.0f} s)")

    # weight gradients at sampled columns of two non-empty experts
    nonempty = np.flatnonzero(counts > 0)
    experts = [int(nonempty[0]), int(nonempty[len(nonempty) // 2])]
    cols = np.sort(rng.choice(f, 3, replace=False))
    tcols = torch.from_numpy(cols).cuda()
    gw = {k: [] for k in ("dWg", "dWu", "dWd")}
    rw = {k: [] for k in ("dWg", "dWu", "dWd")}
    for e in experts:
        c = O.expert_columns(inp["x"], inp["Wg"], inp["Wu"], inp["Wd"], idx, w, inp["dY"], e, cols,
                             wl.prec)
        gw["dWg"].append(to_np(layer.dWg[e].index_select(1, tcols))); rw["dWg"].append(c["dWg"])
        gw["dWu"].append(to_np(layer.dWu[e].index_select(1, tcols))); rw["dWu"].append(c["dWu"])
        gw["dWd"].append(to_np(layer.dWd[e].index_select(0, tcols))); rw["dWd"].append(c["dWd"])
    for key in gw:
        errs[key] = relerr(np.stack(gw[key]), np.stack(rw[key]))
    for e in np.flatnonzero(counts == 0):
        for t in (layer.dWg, layer.dWu, layer.dWd):
            assert torch.count_nonzero(t[int(e)]).item() == 0, (name, "empty expert", int(e))
    say(f"  weight gradients checked ({time.time() - t0:.0f} s)")

    if router:
        dl = to_np(layer.dlogits)
        assert np.max(np.abs(dl.sum(axis=1))) <= 1e-5 * max(1.0, np.max(np.abs(dl)))
        prop = np.asarray(inp["x"], np.float64).T @ dl
        errs["dWr~x^T.dlogits"] = relerr(to_np(layer.dWr), prop)

    say(f"  {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (name, tol, bad)
