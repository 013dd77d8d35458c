"""Parity of the HIP layer (through the C ABI) with the CPU oracle.

Routing decisions are compared given the same float32 logits: the layer is
run with the oracle's logits passed in (MOE_ROUTE_LOGITS_IN), so top-k
indices, counts, offsets and the permutation must match bit for bit, and
every float tensor must match within the precision's normwise tolerance
(fp32 1e-4, bf16 2e-2, MXFP8 6e-2).  MXFP8 codes and block scales of the
dispatched rows are compared bit for bit.  The router GEMM itself is checked separately
against the oracle's logits, with top-k compared wherever the k-th and
(k+1)-th logits are separated by more than the logit error.
"""
import numpy as np
import pytest
import torch

from moe_synth import make_inputs, workload
from oracle import moe_oracle as O
from tests.parity import (TOL, check_gates, compare, dev_tensor, gate, relerr, run_gpu, run_oracle,
                          say, to_np)

pytestmark = pytest.mark.gpu

# name -> (base workload, overrides): small enough for the oracle, several
# tiles in every GEMM dimension and ragged expert tails.
SHAPES = {
    "tiny_fp32": ("tiny_fp32", {}),
    "tiny_bf16": ("tiny_fp32", dict(name="tiny_bf16", dtype="bf16", prec="bf16")),
    "mid_bf16_E8": ("olmoe_bf16", dict(name="mid_bf16_E8", T=1000, d=512, E=8, f=384, k=2)),
    "mid_bf16_E64": ("olmoe_bf16", dict(name="mid_bf16_E64", T=512, d=256, E=64, f=128, k=8)),
    "mid_fp32_E16": ("tiny_fp32", dict(name="mid_fp32_E16", T=300, d=128, E=16, f=192, k=3)),
    "share_zipf_bf16": ("share1t_bf16", dict(name="share_zipf_bf16", T=3000, d=256, f=320)),
    "edge_T1_E1": ("olmoe_bf16", dict(name="edge_T1_E1", T=1, d=64, E=1, f=64, k=1)),
    "edge_kE": ("olmoe_bf16", dict(name="edge_kE", T=70, d=128, E=8, f=64, k=8)),
    "edge_E3_fp32": ("tiny_fp32", dict(name="edge_E3_fp32", T=50, d=64, E=3, f=64, k=2)),
    "edge_E6_bf16": ("olmoe_bf16", dict(name="edge_E6_bf16", T=130, d=128, E=6, f=128, k=2)),
    # small batches (the weight-streaming forward engine): contraction slices
    # with a float reduction (d = 256), a half-empty last down column block
    # (d = 192), experts with more than 32 rows and empty experts (Zipf loads)
    "skinny_d256": ("olmoe_bf16", dict(name="skinny_d256", T=40, d=256, E=8, f=320, k=2)),
    "skinny_zipf_d192": ("share1t_bf16", dict(name="skinny_zipf_d192", T=700, d=192, f=256)),
    # rows wider than one 2048-column pass of the row kernels (dispatch,
    # combine and their backwards), the second pass partly filled
    "wide_bf16_d2560": ("olmoe_bf16", dict(name="wide_bf16_d2560", T=200, d=2560, E=8, f=128, k=3)),
    "wide_fp32_d2112": ("tiny_fp32", dict(name="wide_fp32_d2112", T=90, d=2112, E=4, f=64, k=2)),
    # the router's thin-product kernel: 16 blocks of 16 experts with 64-row
    # chunks and a partial last one (E = 256, d = 576); a half-empty last
    # expert block (E = 40) and a chunk of one 64-row piece (d = 320)
    "router_E256": ("olmoe_bf16", dict(name="router_E256", T=300, d=576, E=256, f=64, k=8)),
    "router_E40": ("olmoe_bf16", dict(name="router_E40", T=130, d=320, E=40, f=64, k=4)),
    # eight expert blocks (128-row chunks, two 64-wide dl16 blocks) and six
    # real blocks padded to eight (E = 96)
    "router_E128": ("olmoe_bf16", dict(name="router_E128", T=200, d=384, E=128, f=64, k=4)),
    "router_E96": ("olmoe_bf16", dict(name="router_E96", T=100, d=448, E=96, f=64, k=6)),
    # the 256x256 engine at output widths that end in a partial column tile
    # in every GEMM (d = 320, f = 192: 64- and 128-column remainders), for
    # the bf16-staged plain stores and the SwiGLU epilogues
    "ragged_n_bf16": ("olmoe_bf16", dict(name="ragged_n_bf16", T=600, d=320, E=8, f=192, k=2)),
    # the largest expert count and a wide top-k: 256 experts of ~12 rows
    # (many one-row and empty segments) through the 256x256 engine, and the
    # same width on the small-batch forward engine (R = 1536 rows)
    "max_E256_k16": ("olmoe_bf16", dict(name="max_E256_k16", T=200, d=128, E=256, f=64, k=16)),
    "max_E256_k16_small": ("olmoe_bf16", dict(name="max_E256_k16_small", T=96, d=128, E=256, f=64,
                                              k=16)),
    # both tile orders of an expert in one launch: Zipf loads give the
    # largest expert 8 M-tiles (more than the 5 gate/up and 4 down N-tiles:
    # N-tiles fastest), the next ones 2-4 (M-tiles fastest where that is fewer
    # than the N-tiles), the rest one tile or none
    "order_mix_bf16": ("share1t_bf16", dict(name="order_mix_bf16", T=6000, d=1024, f=640)),
    "order_mix_mxfp8": ("share1t_bf16", dict(name="order_mix_mxfp8", T=6000, d=1024, f=640,
                                             prec="mxfp8")),
    "tiny_mxfp8": ("tiny_mxfp8", {}),
    # d = 576: an odd number of 64-deep K stages; f = 320: a half-filled last gate/up panel
    "mid_mxfp8_E8": ("olmoe_mxfp8", dict(name="mid_mxfp8_E8", T=1000, d=576, E=8, f=320, k=2)),
    "mid_mxfp8_E64": ("olmoe_mxfp8", dict(name="mid_mxfp8_E64", T=512, d=256, E=64, f=128, k=8)),
    "share_zipf_mxfp8": ("share1t_bf16", dict(name="share_zipf_mxfp8", T=3000, d=256, f=320,
                                              prec="mxfp8")),
    "max_E256_k16_mxfp8": ("olmoe_mxfp8", dict(name="max_E256_k16_mxfp8", T=200, d=128, E=256,
                                                f=64, k=16)),
}


def _layer_case(name, seed=0):
    base, ov = SHAPES[name]
    wl = workload(base, **ov)
    say(f"[case] {name}: T={wl.T} d={wl.d} E={wl.E} f={wl.f} k={wl.k} {wl.dtype}/{wl.prec} seed={seed}")
    inp = make_inputs(wl, seed=seed)
    logits = O.router_logits(inp["x"], inp["Wr"], wl.prec) if wl.routing == "router" else None
    return wl, inp, logits


@pytest.mark.parametrize("name", list(SHAPES))
def test_layer_parity(name):
    wl, inp, logits = _layer_case(name)
    ref = run_oracle(wl, inp, logits)
    gpu = run_gpu(wl, inp, logits)
    compare(wl, gpu, ref)
    # the expert segments hold each expert's rows in ascending token order
    offs, src = gpu["offsets"], gpu["src_token"]
    for e in range(wl.E):
        assert np.all(np.diff(src[offs[e]:offs[e + 1]]) > 0)


@pytest.mark.parametrize("name", ["tiny_fp32", "mid_bf16_E8", "mid_bf16_E64", "edge_E6_bf16",
                                  "router_E256", "router_E40", "router_E128", "router_E96",
                                  "wide_bf16_d2560"])
def test_router_logits_and_topk(name):
    """Router GEMM on the GPU against the oracle's logits; top-k bit-exact on
    every token whose k-th/(k+1)-th logit gap exceeds the logit error."""
    wl, inp, ref_logits = _layer_case(name)
    gpu = run_gpu(wl, inp, None)
    err = relerr(gpu["logits"], ref_logits)
    tol = 1e-6 if wl.dtype == "fp32" else 1e-5
    say(f"  logits relerr {err:.2e}")
    assert err <= tol
    ref_idx = O.topk_select(ref_logits, wl.k)
    srt = np.sort(ref_logits, axis=1)[:, ::-1]
    maxerr = np.max(np.abs(gpu["logits"] - ref_logits))
    if wl.k < wl.E:
        safe = (srt[:, wl.k - 1] - srt[:, wl.k]) > 4 * maxerr
    else:
        safe = np.ones(wl.T, bool)
    assert safe.mean() > 0.9
    np.testing.assert_array_equal(gpu["topk_idx"][safe], ref_idx[safe])
    # the GPU's choice is a valid top-k of its own logits everywhere
    own = O.topk_select(gpu["logits"], wl.k)
    np.testing.assert_array_equal(gpu["topk_idx"], own)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (256, 16), (5, 5), (1, 1)])
def test_topk_with_ties(E, k):
    """Integer-valued logits with many ties: slots ordered by (logit desc,
    index asc), bit-exact against the oracle; weights = softmax probs."""
    import routing_grouped_gemm_amd as rgg
    say(f"[case] topk ties E={E} k={k}")
    rng = np.random.Generator(np.random.PCG64(E * 100 + k))
    T = 333
    lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    lg[:7] = 0.0
    logits = rgg.upload(lg)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    rgg.moe_route(None, None, k, logits, idx, w, logits_in=True)
    torch.cuda.synchronize()
    ref_idx, ref_w, _ = O.route(lg, k, "fp32")
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=0)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (256, 16), (5, 5), (1, 1)])
def test_topk_renorm_with_ties(E, k):
    """Top-k renormalisation: the same choice as without it, the chosen
    probabilities divided by their sum (each row sums to 1)."""
    import routing_grouped_gemm_amd as rgg
    say(f"[case] topk renorm E={E} k={k}")
    rng = np.random.Generator(np.random.PCG64(E * 100 + k + 7))
    T = 333
    lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * 0.7
    logits = rgg.upload(lg)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    rgg.moe_route(None, None, k, logits, idx, w, logits_in=True, renorm=True)
    torch.cuda.synchronize()
    ref_idx, ref_w, _ = O.route(lg, k, "fp32", renorm=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=4e-6, atol=0)


# Router variants: renormalised top-k weights and the load-balancing loss,
# through the full layer (router on the fp32 SIMT, bf16 MFMA split-K, bf16
# SIMT (E % 8 != 0) and MXFP8 paths).
VARIANT_SHAPES = ["tiny_fp32", "mid_bf16_E64", "edge_E6_bf16", "mid_mxfp8_E8"]


# aux_coef = 100: large enough that the loss's gradient is a sizeable part of
# dlogits (with 0.01 it is about 1e-4 of it)
@pytest.mark.parametrize("renorm,aux", [(True, 0.0), (False, 0.01), (True, 100.0)])
@pytest.mark.parametrize("name", VARIANT_SHAPES)
def test_router_variants(name, renorm, aux):
    wl, inp, logits = _layer_case(name)
    say(f"  renorm={renorm} aux_coef={aux}")
    ref = run_oracle(wl, inp, logits, renorm=renorm, aux_coef=aux)
    gpu = run_gpu(wl, inp, logits, renorm=renorm, aux_coef=aux)
    compare(wl, gpu, ref)
    if renorm:
        np.testing.assert_allclose(gpu["topk_w"].sum(axis=1), 1.0, rtol=2e-6)
    if aux:
        el = abs(float(gpu["aux_loss"][0]) - ref["aux_loss"]) / abs(ref["aux_loss"])
        ed = relerr(gpu["aux_dp"], ref["aux_dp"])
        say(f"  aux_loss relerr {el:.2e}, aux_dp relerr {ed:.2e}")
        assert el <= 1e-5 and ed <= 1e-6


@pytest.mark.parametrize("T,E,k,skew", [(1, 1, 1, 0.0), (63, 5, 2, 0.0), (5000, 128, 8, 1.5),
                                        (4097, 256, 16, 0.0)])
def test_route_aux_entry(T, E, k, skew):
    """moe_route_aux alone on oracle routing: several 64-token blocks, a
    ragged last block, skewed (Zipf-like) and uniform expert loads."""
    import routing_grouped_gemm_amd as rgg
    say(f"[case] route_aux T={T} E={E} k={k} skew={skew}")
    rng = np.random.Generator(np.random.PCG64(T + E))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg += (skew * -np.log1p(np.arange(E))).astype(np.float32)[None, :]
    idx, _, _ = O.route(lg, k, "fp32")
    counts = np.bincount(idx.reshape(-1), minlength=E).astype(np.int32)
    ref_L, ref_dp = O.aux_loss(lg, idx, E, 0.01, "fp64")
    ws = torch.empty(max(rgg.moe_workspace_size("route_aux", T, 64, E, 64, k, torch.bfloat16,
                                                "bf16"), 256), dtype=torch.uint8, device="cuda")
    loss = torch.full((1,), float("nan"), device="cuda")
    dp = torch.full((E,), float("nan"), device="cuda")
    rgg.moe_route_aux(rgg.upload(lg), rgg.upload(counts), k, 0.01, loss, dp, ws)
    torch.cuda.synchronize()
    el = abs(float(loss.item()) - ref_L) / abs(ref_L)
    ed = relerr(to_np(dp), ref_dp)
    say(f"  aux_loss {loss.item():.6f} vs {ref_L:.6f}: relerr {el:.2e}, aux_dp {ed:.2e}")
    assert el <= 1e-5 and ed <= 1e-6


@pytest.mark.parametrize("name", ["tiny_fp32", "mid_bf16_E64", "edge_E6_bf16"])
def test_route_bwd_aux_gradient_alone(name):
    """moe_route_bwd with a zero top-k weight gradient: dlogits, dWr and dx
    come from the load-balancing loss's gradient alone."""
    import routing_grouped_gemm_amd as rgg
    wl, inp, logits = _layer_case(name)
    T, d, E, k = wl.T, wl.d, wl.E, wl.k
    dt = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
    idx, _, _ = O.route(logits, k, "fp32")
    _, aux_dp = O.aux_loss(logits, idx, E, 1.0, "fp32")
    ref = O.router_backward(inp["x"], inp["Wr"], logits, idx, np.zeros((T, k)), np.zeros((T, d)),
                            wl.prec, False, aux_dp)
    x, Wr = dev_tensor(inp, "x", dt), dev_tensor(inp, "Wr", dt)
    dlog = torch.empty(T, E, device="cuda")
    dWr = torch.empty(d, E, dtype=dt, device="cuda")
    dx = torch.zeros(T, d, dtype=dt, device="cuda")
    n = rgg.moe_workspace_size("route_bwd", T, d, E, wl.f, k, dt, wl.prec)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    rgg.moe_route_bwd(x, Wr, rgg.upload(logits.astype(np.float32)), rgg.upload(idx),
                      torch.zeros(T, k, device="cuda"), dlog, dWr, dx, ws,
                      aux_dp=rgg.upload(np.asarray(aux_dp, np.float32)))
    torch.cuda.synchronize()
    tol = 1e-4 if wl.dtype == "fp32" else 2e-2
    e1, e2, e3 = (relerr(to_np(g), r) for g, r in
                  ((dlog, ref["dlogits"]), (dWr, ref["dWr"]), (dx, ref["dx"])))
    say(f"  dlogits {e1:.2e} dWr {e2:.2e} dx {e3:.2e}")
    assert e1 <= 1e-4 and e2 <= tol and e3 <= tol


@pytest.mark.parametrize("name", ["mid_bf16_E64", "share_zipf_bf16", "mid_mxfp8_E8", "tiny_fp32",
                                  "order_mix_bf16"])
def test_wgrad_f32(name):
    """Float32 weight gradients of a bf16 layer (MOE_WGRAD_F32) against the
    oracle's float32 variant; a float32 layer is unchanged by the option."""
    wl, inp, logits = _layer_case(name)
    ref = run_oracle(wl, inp, logits, wgrad_f32=True)
    gpu = run_gpu(wl, inp, logits, wgrad_f32=True)
    compare(wl, gpu, ref)


@pytest.mark.parametrize("name", ["mid_bf16_E64", "mid_mxfp8_E8"])
def test_wgrad_f32_accumulation_keeps_small_increments(name):
    """Accumulating into float32 gradients that hold 1024: every increment is
    below half a bf16 unit there (4), so bf16 accumulation would drop them
    all; in float32 they survive and dW - 1024 matches the oracle."""
    wl, inp, logits = _layer_case(name)
    ref = run_oracle(wl, inp, logits, wgrad_f32=True)
    big = max(float(np.max(np.abs(ref[n]))) for n in ("dWg", "dWu", "dWd"))
    say(f"  largest |dW| {big:.2e}")
    assert big < 4.0
    gpu = run_gpu(wl, inp, logits, wgrad_f32=True, wgrad_init=1024.0)
    for n in ("dWg", "dWu", "dWd"):
        e = relerr(gpu[n] - 1024.0, ref[n])
        say(f"  {n}: relerr of dW - 1024: {e:.2e}")
        assert e <= 2e-2, (n, e)


@pytest.mark.parametrize("name", ["mid_bf16_E64", "share_zipf_bf16", "mid_bf16_E8",
                                  "order_mix_bf16"])
def test_wgrad_bf16_accumulation(name):
    """bf16 weight gradients accumulated into buffers that hold random
    bf16 values G0 (the same order of magnitude as dW): the result is G0 + dW
    with one bf16 rounding, including the experts that receive no rows (Zipf
    loads), whose gradients must keep G0.  The Zipf loads of order_mix_bf16
    (the largest expert several times the mean, about four rounds of
    weight-gradient tiles) take the longest-first, alternating-round tile
    order."""
    wl, inp, logits = _layer_case(name)
    ref = run_oracle(wl, inp, logits)
    rng = np.random.default_rng(7)
    init = {}
    for n in ("dWg", "dWu", "dWd"):
        scale = float(np.sqrt(np.mean(ref[n] ** 2))) + 1e-3
        g0 = (rng.standard_normal(ref[n].shape) * scale).astype(np.float32)
        init[n] = torch.as_tensor(g0).to(torch.bfloat16).float().numpy()
    gpu = run_gpu(wl, inp, logits, wgrad_init=init)
    for n in ("dWg", "dWu", "dWd"):
        e = relerr(gpu[n], init[n].astype(np.float64) + ref[n])
        say(f"  {n}: relerr of G0 + dW {e:.2e}")
        assert e <= 2e-2, (n, e)
    if name in ("share_zipf_bf16", "order_mix_bf16"):
        empty = np.flatnonzero(np.diff(gpu["offsets"]) == 0)
        say(f"  empty experts {empty.tolist()}")
        assert empty.size > 0
        for n in ("dWg", "dWu", "dWd"):
            np.testing.assert_array_equal(gpu[n][empty], init[n][empty])


@pytest.mark.parametrize("name,f32", [("tiny_mxfp8", False), ("mid_mxfp8_E8", False),
                                      ("mid_mxfp8_E64", True), ("share_zipf_mxfp8", False),
                                      ("order_mix_mxfp8", True)])
def test_mx_weight_gradients(name, f32):
    """MOE_WGRAD_MX: the weight gradients in MXFP8 too, operands quantised
    along each expert's tokens (odd segment lengths, experts with more and
    fewer than 128 rows, empty experts), against the oracle's variant; the
    result is far closer to it than to the bf16 weight gradients, so the
    token-axis quantisation really happens."""
    wl, inp, logits = _layer_case(name)
    say(f"  mx_wgrad, float32 gradients={f32}")
    ref = run_oracle(wl, inp, logits, wgrad_f32=f32, mx_wgrad=True)
    gpu = run_gpu(wl, inp, logits, wgrad_f32=f32, mx_wgrad=True)
    compare(wl, gpu, ref)
    plain = run_oracle(wl, inp, logits, wgrad_f32=f32, mx_wgrad=False)
    for n in ("dWg", "dWu", "dWd"):
        e_mx, e_plain = relerr(gpu[n], ref[n]), relerr(gpu[n], plain[n])
        say(f"  {n}: vs MX oracle {e_mx:.2e}, vs bf16-gradient oracle {e_plain:.2e}")
        assert e_mx < 0.5 * e_plain, (n, e_mx, e_plain)


def test_all_rows_to_one_expert():
    """Logits that send every token to expert 2 first: one expert takes all
    T rows (several M tiles); the others are empty."""
    wl = workload("olmoe_bf16", name="one_expert", T=700, d=128, E=4, f=128, k=1)
    say(f"[case] one_expert T={wl.T}")
    inp = make_inputs(wl, seed=3)
    lg = np.zeros((wl.T, wl.E), np.float32)
    lg[:, 2] = 1.0
    ref = run_oracle(wl, inp, lg)
    gpu = run_gpu(wl, inp, lg)
    assert gpu["counts"].tolist() == [0, 0, wl.T, 0]
    compare(wl, gpu, ref)
    for e in (0, 1, 3):
        assert np.all(gpu["dWg"][e] == 0) and np.all(gpu["dWd"][e] == 0)


def test_determinism():
    """Two runs on identical inputs give identical bytes (no atomics on any
    result path)."""
    wl, inp, logits = _layer_case("mid_bf16_E64")
    a = run_gpu(wl, inp, None)
    b = run_gpu(wl, inp, None)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


@pytest.mark.parametrize("name", ["tiny_mxfp8", "mid_mxfp8_E8", "share_zipf_mxfp8"])
def test_mx_dispatch_codes(name):
    """The quantising dispatch writes the oracle's e4m3 codes and E8M0 block
    exponents of every dispatched row, bit for bit (both sides quantise the
    same bf16 values)."""
    wl, inp, logits = _layer_case(name)
    gpu = run_gpu(wl, inp, logits)
    R, d = wl.T * wl.k, wl.d
    idx = O.route(logits, wl.k, wl.prec)[0] if logits is not None else inp["topk_idx"]
    src = O.routing_metadata(idx, wl.E)[3]
    Xs = np.asarray(inp["x"], np.float64)[np.asarray(src, np.int64)]   # x is bf16-exact
    np.testing.assert_array_equal(gpu["Xs"], Xs)
    _, E, q = O.mx_quantize(Xs, axis=1)
    np.testing.assert_array_equal(gpu["Xq"], O.e4m3_encode(q))
    sc = gpu["Xq_scale"]
    assert sc.shape == (R, d // 32)
    np.testing.assert_array_equal(sc.astype(np.int64), E + 127)


def test_mx_combine_bwd_codes():
    """The combine backward's block-quantised dYs, bit for bit.  With every
    combine weight 1 the stored dYs rows are exactly the rows of dY (no
    rounding on either side), so the oracle quantises dY[src_token]."""
    wl, inp, _ = _layer_case("share_zipf_mxfp8")
    inp["topk_w"] = np.ones_like(inp["topk_w"])
    gpu = run_gpu(wl, inp, None)
    R, d = wl.T * wl.k, wl.d
    src = O.routing_metadata(inp["topk_idx"], wl.E)[3]
    dYs = np.asarray(inp["dY"], np.float64)[np.asarray(src, np.int64)]
    np.testing.assert_array_equal(gpu["dYs"], dYs)
    _, E, q = O.mx_quantize(dYs, axis=1)
    np.testing.assert_array_equal(gpu["dYs_q"], O.e4m3_encode(q))
    np.testing.assert_array_equal(gpu["dYs_q_scale"].astype(np.int64), E + 127)


def test_mx_quantisation_is_applied():
    """The four block-quantised GEMM outputs match the MXFP8 oracle far more
    closely than the same layer computed in plain bf16: the 6e-2 bound alone
    would also admit a path that skipped the quantisation."""
    wl, inp, logits = _layer_case("mid_mxfp8_E8")
    gpu = run_gpu(wl, inp, logits)
    ref_mx = run_oracle(wl, inp, logits)
    ref_bf = run_oracle(workload("olmoe_bf16", T=wl.T, d=wl.d, E=wl.E, f=wl.f, k=wl.k), inp, logits)
    for n in ("Hg", "Ys", "dHg", "dXs"):
        e_mx, e_bf = relerr(gpu[n], ref_mx[n]), relerr(gpu[n], ref_bf[n])
        say(f"  {n}: vs mxfp8 oracle {e_mx:.2e}, vs bf16 oracle {e_bf:.2e}")
        assert e_mx < 0.2 * e_bf, (n, e_mx, e_bf)


@pytest.mark.parametrize("T,k", [(700, 3), (40, 3)])
def test_out_of_range_slots_are_empty(T, k):
    """Pre-routed slots whose expert lies outside [0, E) (here -1, E and
    1000) are empty slots: no row (dest_row -1, counts without them), no
    contribution to y or dx, dtopk_w = 0, and nothing in the weight
    gradients.  Reference: the oracle on E + 1 experts with every such slot
    sent to the extra, last expert with weight 0 (whose rows then come after
    every real expert's rows and contribute exactly 0).  T = 40 runs the
    small-batch dispatch, experts and combine; T = 700 the general kernels."""
    import routing_grouped_gemm_amd as rgg
    E, d, f = 8, 256, 128
    say(f"[case] out-of-range slots T={T} k={k} E={E}")
    rng = np.random.Generator(np.random.PCG64(T + k))
    wl = workload("olmoe_bf16", name="oor", T=T, d=d, E=E, f=f, k=k)
    inp = make_inputs(wl, seed=3)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    bad = rng.random((T, k)) < 0.08
    bad[0, 0] = True
    idx_bad = idx.copy()
    idx_bad[bad] = rng.choice(np.array([-1, E, 1000], np.int32), int(bad.sum()))
    # reference: invalid slots -> expert E (zero weights), combine weight 0
    idx_ref = idx.copy(); idx_ref[bad] = E
    w_ref = w.copy(); w_ref[bad] = 0.0
    z = lambda a: np.concatenate([a, np.zeros((1,) + a.shape[1:], a.dtype)])
    ref = O.layer(inp["x"], None, z(inp["Wg"]), z(inp["Wu"]), z(inp["Wd"]), k, inp["dY"], "bf16",
                  topk_idx=idx_ref, topk_w=w_ref)
    dt = torch.bfloat16
    layer = rgg.ExpertLayer(T, d, E, f, k, dt, "bf16", router=False)
    layer.forward(dev_tensor(inp, "x", dt), None, dev_tensor(inp, "Wg", dt),
                  dev_tensor(inp, "Wu", dt), dev_tensor(inp, "Wd", dt),
                  topk_idx=rgg.upload(idx_bad), topk_w=rgg.upload(w))
    layer.backward(dev_tensor(inp, "dY", dt))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(layer.counts), ref["counts"][:E])
    np.testing.assert_array_equal(to_np(layer.offsets), ref["offsets"][:E + 1])
    dr = to_np(layer.dest_row)
    assert np.all(dr[bad] == -1)
    np.testing.assert_array_equal(dr[~bad], ref["dest_row"][~bad])
    dw = to_np(layer.dw)
    assert np.all(dw[bad] == 0.0)
    gpu = {n: to_np(getattr(layer, n)) for n in ("y", "dx", "dWg", "dWu", "dWd")}
    gpu["dw_valid"] = dw[~bad]
    refs = {"y": ref["y"], "dx": ref["dx"], "dWg": ref["dWg"][:E], "dWu": ref["dWu"][:E],
            "dWd": ref["dWd"][:E], "dw_valid": np.asarray(ref["dw"])[~bad]}
    errs = {}
    for n in refs:
        gate(n, gpu[n], refs[n], TOL["bf16"], errs)
    check_gates(f"out-of-range T={T}", errs, TOL["bf16"])


@pytest.mark.parametrize("name", ["mid_mxfp8_E8", "share_zipf_mxfp8"])
def test_mx_keep_weights_same_bytes(name):
    """The MXFP8 layer quantises each weight matrix once for both directions
    and hands the backward's codes over in the forward's workspace
    (MOE_MX_KEEP_WEIGHTS, the layer's default); the grouped FFN forward and
    backward run again without the flag, each quantising its own weights,
    give the same bytes in every output."""
    import routing_grouped_gemm_amd as rgg
    wl, inp, logits = _layer_case(name)
    dt = torch.bfloat16
    router = wl.routing == "router"
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, dt, "mxfp8", router=router)
    x = dev_tensor(inp, "x", dt)
    Wg, Wu, Wd = (dev_tensor(inp, n, dt) for n in ("Wg", "Wu", "Wd"))
    kw = dict(logits=rgg.upload(np.ascontiguousarray(logits, np.float32))) if router else \
        dict(topk_idx=rgg.upload(inp["topk_idx"]), topk_w=rgg.upload(inp["topk_w"]))
    layer.forward(x, dev_tensor(inp, "Wr", dt) if router else None, Wg, Wu, Wd, **kw)
    layer.backward(dev_tensor(inp, "dY", dt))
    torch.cuda.synchronize()
    kept = {n: getattr(layer, n).clone() for n in ("Hg", "Hu", "A", "Ys", "dH", "dXs", "dWg",
                                                    "dWu", "dWd")}
    T, d, E, f, k = wl.T, wl.d, wl.E, wl.f, wl.k
    ws_f = torch.empty(rgg.moe_workspace_size("ffn_fwd", T, d, E, f, k, dt, "mxfp8"),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(rgg.moe_workspace_size("ffn_bwd", T, d, E, f, k, dt, "mxfp8"),
                       dtype=torch.uint8, device="cuda")
    out = {n: torch.empty_like(v) for n, v in kept.items()}
    rgg.moe_grouped_ffn_fwd(layer.Xq, layer.Xq_scale, layer.offsets, T, k, Wg, Wu, Wd, out["Hg"],
                            out["Hu"], out["A"], out["Ys"], ws_f, "mxfp8")
    rgg.moe_grouped_ffn_bwd(layer.dYs, layer.Xs, out["Hg"], out["Hu"], out["A"], layer.offsets, T,
                            k, Wg, Wu, Wd, out["dH"], out["dXs"], out["dWg"], out["dWu"],
                            out["dWd"], ws_b, "mxfp8", False, layer.dYs_q, layer.dYs_q_scale)
    torch.cuda.synchronize()
    for n in kept:
        assert torch.equal(kept[n].view(torch.int16), out[n].view(torch.int16)), n
    say(f"  {name}: kept-code layer equals the self-quantising FFN bit for bit")


@pytest.mark.parametrize("T,E,k", [(5000, 64, 8), (300, 8, 2), (1, 256, 16)])
def test_check_routing(T, E, k):
    """moe_check_routing counts the entries outside [0, E) and the tokens
    with a repeated expert, as a host loop over the same indices does; a
    valid routing reports zeros."""
    import routing_grouped_gemm_amd as rgg
    say(f"[case] check_routing T={T} E={E} k={k}")
    rng = np.random.Generator(np.random.PCG64(T + E))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    rep = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    rgg.moe_check_routing(rgg.upload(idx), E, rep)
    torch.cuda.synchronize()
    assert to_np(rep)[:2].tolist() == [0, 0]
    bad = idx.copy()
    m = rng.random((T, k)) < 0.05
    bad[m] = rng.choice(np.array([-1, E, 1000, -7], np.int32), int(m.sum()))
    if k > 1:
        for t in rng.choice(T, max(1, T // 20), replace=False):
            bad[t, 1] = bad[t, 0] if 0 <= bad[t, 0] < E else bad[t, 1]
    n_bad = int(np.sum((bad < 0) | (bad >= E)))
    n_dup = 0
    for t in range(T):
        ok = [e for e in bad[t] if 0 <= e < E]
        n_dup += len(ok) != len(set(ok))
    rgg.moe_check_routing(rgg.upload(bad), E, rep)
    torch.cuda.synchronize()
    got = to_np(rep)[:2].tolist()
    say(f"  report {got}, expected {[n_bad, n_dup]}")
    assert got == [n_bad, n_dup]
