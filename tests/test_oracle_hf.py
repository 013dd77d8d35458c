"""Pins of the CPU oracle against the HF OLMoE modules that the "OLMoE in HF
Transformers" walkthrough describes (transformers.models.olmoe.modeling_olmoe):

  * section 2 (router): OlmoeTopKRouter -- float32 softmax of the logits,
    torch.topk of the top_k probabilities, optional norm_topk_prob;
  * section 3 (expert layer): OlmoeSparseMoeBlock / OlmoeExperts -- 3-D
    gate_up_proj [E, 2f, d] and down_proj [E, d, f], the per-expert loop and
    index_add_ back to the tokens; its autograd backward;
  * section 4 (load-balancing loss): load_balancing_loss_func in
    modeling_olmoe.py, which the causal-LM head scales by
    router_aux_loss_coef.

These are independent implementations of the same definitions (torch, the
HF code), run here in float64 where HF allows it.  HF's router takes its
softmax in float32 (the walkthrough says so), so its weights and the
gradients that pass through them carry float32 rounding: those comparisons
use float32-level tolerances, and the chosen indices are compared exactly
wherever the float32 probabilities have no tie at the k-th place.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

M = pytest.importorskip("transformers.models.olmoe.modeling_olmoe")
from transformers import OlmoeConfig  # noqa: E402


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _config(d, E, f, k, norm):
    cfg = OlmoeConfig(hidden_size=d, intermediate_size=f, num_experts=E,
                      num_experts_per_tok=k, norm_topk_prob=norm, hidden_act="silu")
    cfg._experts_implementation = "eager"   # the per-expert loop the page prints
    return cfg


def _block(Wr, Wg, Wu, Wd, k, norm):
    """OlmoeSparseMoeBlock in float64 holding the oracle's weights:
    gate.weight = Wr^T [E, d]; gate_up_proj[e] = [Wg[e]^T ; Wu[e]^T] [2f, d]
    (gate rows first, as its chunk(2) splits them); down_proj[e] = Wd[e]^T."""
    d, E = Wr.shape
    f = Wg.shape[2]
    blk = M.OlmoeSparseMoeBlock(_config(d, E, f, k, norm)).double()
    with torch.no_grad():
        blk.gate.weight.copy_(torch.from_numpy(Wr.T.copy()))
        gu = np.concatenate([np.transpose(Wg, (0, 2, 1)), np.transpose(Wu, (0, 2, 1))], axis=1)
        blk.experts.gate_up_proj.copy_(torch.from_numpy(gu))
        blk.experts.down_proj.copy_(torch.from_numpy(np.transpose(Wd, (0, 2, 1)).copy()))
    return blk


def _untied_rows(probs32, k):
    """Tokens whose float32 probabilities have distinct k-th and (k+1)-th
    values (where torch.topk's choice is unique)."""
    s = -np.sort(-probs32, axis=1)
    if k == probs32.shape[1]:
        return np.ones(probs32.shape[0], bool)
    return s[:, k - 1] > s[:, k]


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("T,d,E,k", [(200, 32, 8, 2), (128, 64, 64, 8), (64, 16, 5, 5)])
def test_router_matches_hf_topk_router(norm, T, d, E, k):
    rng = _rng(101 + E)
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((d, E)) * 0.3
    cfg = _config(d, E, 16, k, norm)
    r = M.OlmoeTopKRouter(cfg).double()
    with torch.no_grad():
        r.weight.copy_(torch.from_numpy(Wr.T.copy()))
        hl, hw, hi = r(torch.from_numpy(x))
    logits = O.router_logits(x, Wr, "fp64")
    np.testing.assert_allclose(logits, hl.numpy(), rtol=1e-12, atol=1e-12)
    idx, w, p = O.route(logits, k, "fp64", renorm=norm)
    p32 = torch.softmax(torch.from_numpy(logits), dim=-1, dtype=torch.float).numpy()
    ok = _untied_rows(p32, k)
    assert ok.mean() > 0.9
    # HF orders its slots by probability, then (for equal float32 values) as
    # torch.topk leaves them; the oracle by (logit desc, index asc).  Compare
    # the slot order where the float32 probabilities of the slots differ.
    np.testing.assert_array_equal(np.sort(idx[ok], axis=1), np.sort(hi.numpy()[ok], axis=1))
    strict = ok & np.all(np.diff(-np.take_along_axis(p32, hi.numpy(), 1), axis=1) > 0, axis=1)
    np.testing.assert_array_equal(idx[strict], hi.numpy()[strict])
    # weights: HF's are float32 softmax values (renormalised in float32)
    hw = hw.numpy()
    order = np.argsort(hi.numpy(), axis=1)
    mine = np.take_along_axis(w, np.argsort(idx, axis=1), 1)
    theirs = np.take_along_axis(hw, order, 1)
    np.testing.assert_allclose(mine[ok], theirs[ok], rtol=2e-6, atol=1e-9)


@pytest.mark.parametrize("norm", [False, True])
def test_expert_layer_matches_hf_sparse_moe_block(norm):
    """Forward: O.layer_forward given HF's routing equals OlmoeSparseMoeBlock
    to float64 rounding.  Backward (autograd of sum <y, dY>): the expert
    weight gradients and the expert part of dx equal O.layer_backward given
    HF's routing to float64 rounding; the router weight gradient and the full
    dx, which pass through HF's float32 softmax, within float32 rounding."""
    rng = _rng(7 + norm)
    T, d, E, f, k = 96, 24, 6, 40, 2
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((d, E)) * 0.3
    Wg, Wu, Wd = (rng.standard_normal(s) * 0.2 for s in ((E, d, f), (E, d, f), (E, f, d)))
    dY = rng.standard_normal((T, d))
    blk = _block(Wr, Wg, Wu, Wd, k, norm)
    xt = torch.from_numpy(x.copy()).requires_grad_(True)
    with torch.no_grad():
        _, hw, hi = blk.gate(xt)
    y = blk(xt.view(1, T, d)).view(T, d)
    (y * torch.from_numpy(dY)).sum().backward()
    hi, hw = hi.numpy().astype(np.int32), hw.numpy()

    fwd = O.layer_forward(x, Wg, Wu, Wd, hi, hw, "fp64")
    np.testing.assert_allclose(fwd["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    bwd = O.layer_backward(fwd, x, Wg, Wu, Wd, hi, hw, dY, "fp64")
    gu = blk.experts.gate_up_proj.grad.numpy()
    np.testing.assert_allclose(bwd["dWg"], np.transpose(gu[:, :f], (0, 2, 1)), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(bwd["dWu"], np.transpose(gu[:, f:], (0, 2, 1)), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(bwd["dWd"], np.transpose(blk.experts.down_proj.grad.numpy(), (0, 2, 1)),
                               rtol=1e-11, atol=1e-13)
    # router backward: HF's weights come from a float32 softmax
    logits = O.router_logits(x, Wr, "fp64")
    rb = O.router_backward(x, Wr, logits, hi, bwd["dw"], bwd["dx"], "fp64", renorm=norm)
    dWr_hf = blk.gate.weight.grad.numpy().T
    assert np.linalg.norm(rb["dWr"] - dWr_hf) / np.linalg.norm(dWr_hf) < 1e-6
    dx_hf = xt.grad.numpy()
    assert np.linalg.norm(rb["dx"] - dx_hf) / np.linalg.norm(dx_hf) < 1e-6
    # and the whole oracle layer (its own routing, float64 softmax) agrees
    # with HF on y where HF's routing equals the oracle's
    full = O.layer(x, Wr, Wg, Wu, Wd, k, dY, "fp64", renorm=norm)
    np.testing.assert_array_equal(full["topk_idx"], hi)
    assert np.linalg.norm(full["y"] - fwd["y"]) / np.linalg.norm(fwd["y"]) < 1e-6
    for n, ref in (("dWr", dWr_hf), ("dx", dx_hf)):
        assert np.linalg.norm(full[n] - ref) / np.linalg.norm(ref) < 1e-6, n


@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (512, 64, 8), (100, 16, 1)])
def test_aux_loss_matches_hf_load_balancing_loss(T, E, k):
    """O.aux_loss(coef=1) equals load_balancing_loss_func (one layer, no
    attention mask); its gradient with respect to the logits (through the
    softmax backward, with the routing held fixed) equals torch autograd of
    that function."""
    rng = _rng(200 + E)
    logits = rng.standard_normal((T, E)) * 1.5
    # skewed routing, so that the counts differ from expert to expert
    logits[:, 0] += 1.0
    lt = torch.from_numpy(logits.copy()).requires_grad_(True)
    L_hf = M.load_balancing_loss_func((lt,), num_experts=E, top_k=k)
    L_hf.backward()
    idx, _, p = O.route(logits, k, "fp64")
    L, dp = O.aux_loss(logits, idx, E, 1.0, "fp64")
    # HF averages its one-hot expert mask in float32, so its f_e = counts_e/T
    # carries float32 rounding unless T is a power of two
    rtol = 1e-12 if T & (T - 1) == 0 else 2e-7
    assert abs(L - L_hf.item()) <= rtol * abs(L_hf.item()), (L, L_hf.item())
    rb = O.router_backward(np.zeros((T, 1)), np.zeros((1, E)), logits, idx, np.zeros((T, k)),
                           np.zeros((T, 1)), "fp64", aux_dp=dp)
    if rtol == 1e-12:
        np.testing.assert_allclose(rb["dlogits"], lt.grad.numpy(), rtol=1e-10, atol=1e-15)
    else:   # float32 f_e: compare normwise (the softmax backward cancels)
        g = lt.grad.numpy()
        assert np.linalg.norm(rb["dlogits"] - g) / np.linalg.norm(g) < 1e-6
    # the scale the causal-LM head applies: coef * aux_loss
    L2, dp2 = O.aux_loss(logits, idx, E, 0.01, "fp64")
    assert abs(L2 - 0.01 * L_hf.item()) <= rtol * abs(L_hf.item())
    np.testing.assert_allclose(dp2, 0.01 * dp, rtol=1e-14)
