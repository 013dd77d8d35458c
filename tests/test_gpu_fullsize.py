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
    gradients at sampled columns of every expert with rows: normwise relative
    error within the precision's bound (bf16 2e-2, MXFP8 6e-2), and the
    worst row and worst element within the local gates of tests/parity.py;
  * experts with no rows get exactly zero weight gradients;
  * router weight gradient: dWr equals x^T . dlogits (the layer's own
    dlogits, a property that holds at any size) within the bf16 bound, and
    every dlogits row sums to ~0.
A second test runs the GPU router itself (no logits passed in) at the
benchmark's router shapes: logits against the oracle's float32 logits,
top-k bit-exact where the k-th/(k+1)-th gap exceeds the logit error, and the
top-k, weights and metadata bit-exact against the oracle fed the GPU's own
logits.
"""
import time

import numpy as np
import pytest
import torch

from moe_synth import make_inputs, workload
from oracle import moe_oracle as O
from tests.parity import TOL, check_gates, dev_tensor, gate, relerr, say, to_np

pytestmark = pytest.mark.gpu

FULL = ["olmoe_bf16", "escan_e8_bf16", "escan_e32_bf16", "escan_e128_bf16", "share1t_bf16",
        "olmoe_mxfp8", "olmoe_mxfp8_wgrad"]


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
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, dt, wl.prec, router=router,
                            mx_wgrad=wl.mx_wgrad)
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
        gate(key, rowvals(getattr(layer, key)), s[key], tol, errs)
    dH = rowvals(layer.dH)
    gate("dHg", dH[..., :f], s["dHg"], tol, errs)
    gate("dHu", dH[..., f:], s["dHu"], tol, errs)
    gate("y", to_np(layer.y.index_select(0, tt)), s["y"], tol, errs)
    gate("dx", to_np(layer.dx.index_select(0, tt)), s["dx"], tol, errs)
    gate("dw", to_np(layer.dw.index_select(0, tt)), s["dw"], tol, errs)
    if router:
        gate("dlogits", to_np(layer.dlogits.index_select(0, tt)), s["dlogits"], tol, errs)
    say(f"  tokens checked ({time.time() - t0:.0f} s)")

    # weight gradients at sampled columns of every expert with rows
    nonempty = np.flatnonzero(counts > 0)
    cols = np.sort(rng.choice(f, 3, replace=False))
    tcols = torch.from_numpy(cols).cuda()
    gw = {k: [] for k in ("dWg", "dWu", "dWd")}
    rw = {k: [] for k in ("dWg", "dWu", "dWd")}
    for e in nonempty:
        e = int(e)
        c = O.expert_columns(inp["x"], inp["Wg"], inp["Wu"], inp["Wd"], idx, w, inp["dY"], e, cols,
                             wl.prec, mx_wgrad=wl.mx_wgrad)
        # rows of the comparison: one sampled d_ff column (length d) each
        gw["dWg"].append(to_np(layer.dWg[e].index_select(1, tcols)).T); rw["dWg"].append(c["dWg"].T)
        gw["dWu"].append(to_np(layer.dWu[e].index_select(1, tcols)).T); rw["dWu"].append(c["dWu"].T)
        gw["dWd"].append(to_np(layer.dWd[e].index_select(0, tcols))); rw["dWd"].append(c["dWd"])
    for key in gw:
        gate(key, np.stack(gw[key]), np.stack(rw[key]), tol, errs)
    for e in np.flatnonzero(counts == 0):
        for t in (layer.dWg, layer.dWu, layer.dWd):
            assert torch.count_nonzero(t[int(e)]).item() == 0, (name, "empty expert", int(e))
    say(f"  weight gradients of {len(nonempty)} experts checked ({time.time() - t0:.0f} s)")

    if router:
        dl = to_np(layer.dlogits)
        assert np.max(np.abs(dl.sum(axis=1))) <= 1e-5 * max(1.0, np.max(np.abs(dl)))
        prop = np.asarray(inp["x"], np.float64).T @ dl
        gate("dWr~x^T.dlogits", to_np(layer.dWr), prop, tol, errs)

    check_gates(name, errs, tol)


@pytest.mark.parametrize("name", ["olmoe_bf16", "escan_e128_bf16"])
def test_full_size_gpu_router(name):
    """The router GEMM and top-k on the GPU at the benchmark's shapes (8192 x
    2048 x 64 and 16384 x 4096 x 128), in the benchmark's launch path."""
    import routing_grouped_gemm_amd as rgg
    t0 = time.time()
    wl = workload(name)
    say(f"[full-router] {name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k}")
    inp = make_inputs(wl, seed=0)
    ref_logits = O.router_logits(inp["x"], inp["Wr"], wl.prec)
    dt = torch.bfloat16
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, dt, wl.prec, router=True)
    x = dev_tensor(inp, "x", dt)
    Wg, Wu, Wd = (dev_tensor(inp, n, dt) for n in ("Wg", "Wu", "Wd"))
    Wr = dev_tensor(inp, "Wr", dt)
    layer.forward(x, Wr, Wg, Wu, Wd)
    torch.cuda.synchronize()
    say(f"  forward ran ({time.time() - t0:.0f} s)")
    lg = to_np(layer.logits)
    err = relerr(lg, ref_logits)
    rows = np.linalg.norm(lg - ref_logits, axis=1) / np.linalg.norm(ref_logits, axis=1)
    maxerr = float(np.max(np.abs(lg - ref_logits)))
    say(f"  logits normwise {err:.2e}, worst token {rows.max():.2e}, max abs {maxerr:.2e}")
    assert err <= 1e-5 and rows.max() <= 1e-4
    idx = to_np(layer.topk_idx)
    srt = np.sort(ref_logits, axis=1)[:, ::-1]
    safe = (srt[:, wl.k - 1] - srt[:, wl.k]) > 4 * maxerr
    say(f"  {safe.mean() * 100:.2f}% of tokens with a safe k-th gap")
    assert safe.mean() > 0.9
    np.testing.assert_array_equal(idx[safe], O.topk_select(ref_logits, wl.k)[safe])
    # on its own logits the GPU's routing and metadata are the oracle's, bit for bit
    own_idx, own_w, _ = O.route(lg, wl.k, wl.prec)
    np.testing.assert_array_equal(idx, own_idx)
    assert relerr(to_np(layer.topk_w), own_w) <= 1e-5
    counts, offsets, dest_row, src_token = O.routing_metadata(own_idx, wl.E)
    np.testing.assert_array_equal(to_np(layer.counts), counts)
    np.testing.assert_array_equal(to_np(layer.offsets), offsets)
    np.testing.assert_array_equal(to_np(layer.dest_row), dest_row)
    np.testing.assert_array_equal(to_np(layer.src_token), src_token)
    say(f"  routing checked ({time.time() - t0:.0f} s)")
