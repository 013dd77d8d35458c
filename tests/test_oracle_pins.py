"""Pins of the CPU oracle to things other than itself.

Each test fixes part of the oracle against a library routine, a closed form,
a brute-force enumeration, an invariant, a hand-worked case or finite
differences, so that a dropped term, a wrong sign or index or a transposed
operand in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_round_bf16_matches_torch():
    rng = _rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        rng.standard_normal(2000) * 1e-39,            # bf16 subnormal range
    ]).astype(np.float32)
    # exact ties: low 16 bits = 0x8000, both even and odd kept mantissas
    expo = rng.integers(1, 255, 4000, dtype=np.uint32)
    kept = rng.integers(0, 1 << 7, 4000, dtype=np.uint32)      # kept bf16 mantissa bits
    ties = ((expo << 23) | (kept << 16) | 0x8000).astype(np.uint32).view(np.float32)
    assert np.all(np.isfinite(ties))
    vals = np.concatenate([vals, ties, -ties])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(vals.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("scale_exp", [-10, 0, 5])
def test_e4m3_matches_torch_exhaustive_bf16(scale_exp):
    """Every finite bf16 value divided by 2^s: oracle e4m3 rounding and byte
    code equal torch.float8_e4m3fn wherever torch does not overflow to NaN,
    and saturate to +-448 above."""
    v = (_all_finite_bf16().astype(np.float64) / 2.0 ** scale_exp)
    inr = np.abs(v) <= 448.0
    t = torch.from_numpy(v[inr].astype(np.float32)).to(torch.float8_e4m3fn)
    ref_val = t.to(torch.float64).numpy()
    ref_code = t.view(torch.uint8).numpy()
    got = O.e4m3_round(v[inr])
    np.testing.assert_array_equal(got, ref_val)
    np.testing.assert_array_equal(O.e4m3_encode(got), ref_code)
    np.testing.assert_array_equal(O.e4m3_decode(ref_code), ref_val)
    out = v[~inr]
    np.testing.assert_array_equal(O.e4m3_round(out), np.copysign(448.0, out))


def test_mx_scale_closed_forms():
    # zero block -> exponent 0, codes 0
    deq, E, q = O.mx_quantize(np.zeros((1, 32)), axis=1)
    assert E[0, 0] == 0 and np.all(q == 0) and np.all(deq == 0)
    for j in range(-20, 21):
        amax = 448.0 * 2.0 ** j
        assert O.mx_scale_exponent(amax) == j
        assert O.mx_scale_exponent(np.nextafter(amax, np.inf)) == j + 1
        assert O.mx_scale_exponent(np.nextafter(amax, 0)) == j
    # clamp to the E8M0 range
    assert O.mx_scale_exponent(1e-300) == -127
    assert O.mx_scale_exponent(1e300) == 127


def test_mx_worked_blocks():
    # amax 500: least E with 448*2^E >= 500 is 1; 250 -> 256, 125 -> 128 (e4m3 spacing 16 and 8)
    blk = np.zeros(32); blk[:3] = [500.0, 250.0, 3.0]
    deq, E, q = O.mx_quantize(blk[None], axis=1)
    assert E[0, 0] == 1
    np.testing.assert_array_equal(q[0, :3], [256.0, 128.0, 1.5])
    np.testing.assert_array_equal(deq[0, :3], [512.0, 256.0, 3.0])
    # amax 1: E = -8; 0.3*256 = 76.8 -> 80, -0.05*256 = -12.8 -> -13, 1e-4*256 -> 13 * 2^-9 (subnormal)
    blk = np.zeros(32); blk[:4] = [1.0, 0.3, -0.05, 1e-4]
    deq, E, q = O.mx_quantize(blk[None], axis=1)
    assert E[0, 0] == -8
    np.testing.assert_array_equal(q[0, :4], [256.0, 80.0, -13.0, 13 * 2.0 ** -9])


def test_mx_grid_values_roundtrip():
    rng = _rng(2)
    codes = rng.integers(0, 256, size=(16, 64)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E            # avoid the NaN codes
    vals = O.e4m3_decode(codes)
    vals[:, 0::32] = 448.0                          # every block hits amax 448 -> E = 0
    deq, E, q = O.mx_quantize(vals * 2.0 ** 3, axis=1)
    assert np.all(E == 3)
    np.testing.assert_array_equal(deq, vals * 2.0 ** 3)


def test_mx_block_axis_power_of_two_equivariance():
    """Blocks run along the given axis: scaling one row by 2^j scales that
    row's quantised values by exactly 2^j and leaves every other row alone;
    scaling one column changes other columns in general."""
    rng = _rng(3)
    a = rng.standard_normal((8, 64))
    base = O.mx_quantize(a, axis=1)[0]
    b = a.copy(); b[3] *= 2.0 ** 5
    got = O.mx_quantize(b, axis=1)[0]
    np.testing.assert_array_equal(got[3], base[3] * 2.0 ** 5)
    np.testing.assert_array_equal(np.delete(got, 3, 0), np.delete(base, 3, 0))
    c = a.copy(); c[:, 7] *= 2.0 ** 9
    got_c = O.mx_quantize(c, axis=1)[0]
    assert not np.array_equal(np.delete(got_c, 7, 1), np.delete(base, 7, 1))


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def _brute_topk(l, k):
    """Best k-subset by exhaustive search: compare the members sorted by
    (logit desc, index asc) lexicographically on (logit, -index)."""
    best = None
    for S in itertools.combinations(range(len(l)), k):
        key = sorted(((l[e], -e) for e in S), reverse=True)
        if best is None or key > best[0]:
            best = (key, [-ne for _, ne in key])
    return best[1]


def test_topk_brute_force_with_ties():
    rng = _rng(4)
    T, E, k = 300, 8, 2
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float64)   # many ties
    logits[:20] = 0.0
    idx = O.topk_select(logits, k)
    for t in range(T):
        assert list(idx[t]) == _brute_topk(list(logits[t]), k)
    for kk in (1, 3, 8):
        idx = O.topk_select(logits[:50], kk)
        for t in range(50):
            assert list(idx[t]) == _brute_topk(list(logits[t]), kk)


def test_topk_pairwise_condition_large_E():
    rng = _rng(5)
    T, E, k = 64, 128, 8
    logits = np.round(rng.standard_normal((T, E)), 1)
    idx = O.topk_select(logits, k)
    for t in range(T):
        S = list(idx[t])
        assert len(set(S)) == k
        for a, b in zip(S, S[1:]):                  # slot order
            assert (logits[t, a], -a) > (logits[t, b], -b)
        rest = [e for e in range(E) if e not in S]
        worst = S[-1]
        for e in rest:
            assert (logits[t, worst], -worst) > (logits[t, e], -e)


def test_softmax_and_router_backward_invariants():
    rng = _rng(6)
    T, d, E, k = 40, 16, 8, 3
    logits = rng.standard_normal((T, E))
    p = O.softmax(logits)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-15)
    idx, w, _ = O.route(logits, E, "fp64")         # k = E: weights sum to 1
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-15)
    idx, w, _ = O.route(logits, k, "fp64")
    dw = rng.standard_normal((T, k))
    rb = O.router_backward(rng.standard_normal((T, d)), rng.standard_normal((d, E)),
                           logits, idx, dw, np.zeros((T, d)), "fp64")
    np.testing.assert_allclose(rb["dlogits"].sum(1), 0.0, atol=1e-14)


# ---------------------------------------------------------------------------
# routing metadata
# ---------------------------------------------------------------------------

def _random_idx(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (37, 8, 2), (256, 64, 8), (100, 5, 5)])
def test_metadata_invariants(T, E, k):
    rng = _rng(7)
    idx = _random_idx(rng, T, E, k)
    counts, offsets, dest, src = O.routing_metadata(idx, E)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
    np.testing.assert_array_equal(np.diff(offsets), counts)
    assert sorted(dest.ravel().tolist()) == list(range(T * k))      # bijection
    for t in range(T):
        for j in range(k):
            r = dest[t, j]
            assert src[r] == t
            assert offsets[idx[t, j]] <= r < offsets[idx[t, j] + 1]
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                              # ascending tokens


def test_metadata_empty_experts():
    idx = np.array([[2], [2], [4]], dtype=np.int32)
    counts, offsets, dest, src = O.routing_metadata(idx, 6)
    assert counts.tolist() == [0, 0, 2, 0, 1, 0]
    assert offsets.tolist() == [0, 0, 0, 2, 2, 3, 3]
    assert dest.ravel().tolist() == [0, 1, 2] and src.tolist() == [0, 1, 2]


# ---------------------------------------------------------------------------
# hand-worked layer (tests/golden/hand_worked_layer.json)
# ---------------------------------------------------------------------------

def test_hand_worked_layer():
    with open(os.path.join(GOLDEN, "hand_worked_layer.json")) as fh:
        g = json.load(fh)
    arr = {n: np.array(g[n], dtype=np.float64) for n in ("x", "Wr", "Wg", "Wu", "Wd", "dY")}
    out = O.layer(arr["x"], arr["Wr"], arr["Wg"], arr["Wu"], arr["Wd"], g["k"], arr["dY"], "fp64")
    ex = g["expect"]
    for key in ("topk_idx", "counts", "offsets", "dest_row", "src_token"):
        assert out[key].tolist() == ex[key], key
    for key in ("topk_w", "y", "dw"):
        np.testing.assert_allclose(out[key], np.array(ex[key]), rtol=0, atol=2e-11, err_msg=key)
    # the fixture's numbers are the closed forms of its derivation
    e = math.e; s1 = e / (e + 1)
    np.testing.assert_allclose(ex["topk_w"], [[e / (2 * e + 1)] * 2, [e * e / (e * e + 2), 1 / (e * e + 2)]], atol=1e-11)
    np.testing.assert_allclose(np.array(ex["y"])[:, 0], [3 * s1 * e / (2 * e + 1), s1 * (3 * e * e + 1) / (e * e + 2)], atol=1e-11)


# ---------------------------------------------------------------------------
# special cases that reduce to dense torch computations
# ---------------------------------------------------------------------------

def _weights(rng, d, E, f, scale=0.3):
    return (rng.standard_normal((E, d, f)) * scale, rng.standard_normal((E, d, f)) * scale,
            rng.standard_normal((E, f, d)) * scale)


def _torch_ffn(x, Wg, Wu, Wd):
    x, Wg, Wu, Wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, Wg, Wu, Wd))
    return (torch.nn.functional.silu(x @ Wg) * (x @ Wu) @ Wd).numpy()


def test_single_expert_is_dense_swiglu():
    rng = _rng(8)
    T, d, f = 33, 16, 24
    x = rng.standard_normal((T, d)); Wr = rng.standard_normal((d, 1))
    Wg, Wu, Wd = _weights(rng, d, 1, f)
    out = O.layer(x, Wr, Wg, Wu, Wd, 1, None, "fp64")
    assert np.all(out["topk_w"] == 1.0)
    np.testing.assert_allclose(out["y"], _torch_ffn(x, Wg[0], Wu[0], Wd[0]), rtol=1e-12, atol=1e-12)


def test_k_equals_E_is_dense_mixture():
    rng = _rng(9)
    T, d, E, f = 20, 8, 5, 12
    x = rng.standard_normal((T, d)); Wr = rng.standard_normal((d, E))
    Wg, Wu, Wd = _weights(rng, d, E, f)
    out = O.layer(x, Wr, Wg, Wu, Wd, E, None, "fp64")
    p = torch.softmax(torch.from_numpy(x @ Wr), dim=1).numpy()
    ref = sum(p[:, e:e + 1] * _torch_ffn(x, Wg[e], Wu[e], Wd[e]) for e in range(E))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_identical_experts():
    rng = _rng(10)
    T, d, E, f, k = 30, 8, 6, 10, 3
    x = rng.standard_normal((T, d)); Wr = rng.standard_normal((d, E))
    g, u, dd = _weights(rng, d, 1, f)
    Wg, Wu, Wd = (np.repeat(a, E, axis=0) for a in (g, u, dd))
    out = O.layer(x, Wr, Wg, Wu, Wd, k, None, "fp64")
    ref = out["topk_w"].sum(1, keepdims=True) * _torch_ffn(x, g[0], u[0], dd[0])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_zero_token_row():
    rng = _rng(11)
    T, d, E, f, k = 6, 8, 5, 10, 3
    x = rng.standard_normal((T, d)); x[2] = 0.0
    Wr = rng.standard_normal((d, E))
    Wg, Wu, Wd = _weights(rng, d, E, f)
    out = O.layer(x, Wr, Wg, Wu, Wd, k, None, "fp64")
    assert np.all(out["logits"][2] == 0.0)
    assert out["topk_idx"][2].tolist() == [0, 1, 2]
    np.testing.assert_allclose(out["topk_w"][2], 1.0 / E, rtol=1e-15)
    assert np.all(out["y"][2] == 0.0)


def test_zero_upstream_gradient():
    rng = _rng(12)
    T, d, E, f, k = 10, 8, 4, 6, 2
    x = rng.standard_normal((T, d)); Wr = rng.standard_normal((d, E))
    Wg, Wu, Wd = _weights(rng, d, E, f)
    out = O.layer(x, Wr, Wg, Wu, Wd, k, np.zeros((T, d)), "fp64")
    for key in ("dw", "dx", "dWg", "dWu", "dWd", "dWr", "dlogits"):
        assert np.all(out[key] == 0.0), key


def test_all_rows_to_one_expert_is_dense_gemm():
    rng = _rng(13)
    T, d, E, f = 25, 8, 4, 6
    x = rng.standard_normal((T, d))
    idx = np.full((T, 1), 2, dtype=np.int32); w = np.ones((T, 1))
    Wg, Wu, Wd = _weights(rng, d, E, f)
    fwd = O.layer_forward(x, Wg, Wu, Wd, idx, w, "fp64")
    assert fwd["counts"].tolist() == [0, 0, T, 0]
    np.testing.assert_allclose(fwd["y"], _torch_ffn(x, Wg[2], Wu[2], Wd[2]), rtol=1e-12, atol=1e-12)
    dY = rng.standard_normal((T, d))
    bwd = O.layer_backward(fwd, x, Wg, Wu, Wd, idx, w, dY, "fp64")
    for e in (0, 1, 3):                            # empty experts get zero gradients
        assert np.all(bwd["dWg"][e] == 0) and np.all(bwd["dWd"][e] == 0)


# ---------------------------------------------------------------------------
# backward: torch autograd and finite differences
# ---------------------------------------------------------------------------

def _torch_layer_loss(x, Wr, Wg, Wu, Wd, idx, dY):
    """Dense torch formulation with fixed routing: every token runs every
    chosen expert directly (no permutation), weights from torch.softmax."""
    p = torch.softmax(x @ Wr, dim=1)
    y = torch.zeros_like(x)
    for j in range(idx.shape[1]):
        e = idx[:, j]
        h = torch.einsum("td,tdf->tf", x, Wg[e])
        u = torch.einsum("td,tdf->tf", x, Wu[e])
        o = torch.einsum("tf,tfd->td", torch.nn.functional.silu(h) * u, Wd[e])
        y = y + p.gather(1, e[:, None]) * o
    return (y * dY).sum()


def test_backward_matches_torch_autograd():
    rng = _rng(14)
    T, d, E, f, k = 24, 8, 6, 10, 3
    x = rng.standard_normal((T, d)); Wr = rng.standard_normal((d, E))
    Wg, Wu, Wd = _weights(rng, d, E, f)
    dY = rng.standard_normal((T, d))
    out = O.layer(x, Wr, Wg, Wu, Wd, k, dY, "fp64")
    ts = {n: torch.tensor(a, requires_grad=True) for n, a in
          dict(x=x, Wr=Wr, Wg=Wg, Wu=Wu, Wd=Wd).items()}
    idx = torch.from_numpy(out["topk_idx"].astype(np.int64))
    L = _torch_layer_loss(ts["x"], ts["Wr"], ts["Wg"], ts["Wu"], ts["Wd"], idx, torch.from_numpy(dY))
    L.backward()
    for n, key in (("x", "dx"), ("Wr", "dWr"), ("Wg", "dWg"), ("Wu", "dWu"), ("Wd", "dWd")):
        np.testing.assert_allclose(out[key], ts[n].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=key)


def test_finite_differences_tiny():
    """Central differences (h = 1e-5) of L = sum <y, dY> on the tiny layer
    (T=256, d=64, E=8, f=128, k=2, seed 0): all of Wr plus 256 seeded
    coordinates of each of x, Wg, Wu, Wd, skipping (and counting) any
    coordinate where the routing changes between theta +- h."""
    from moe_synth import workload, make_inputs
    wl = workload("tiny_fp32")
    assert (wl.T, wl.d, wl.E, wl.f, wl.k) == (256, 64, 8, 128, 2)
    inp = make_inputs(wl, seed=0)
    arrs = {n: inp[n].astype(np.float64) for n in ("x", "Wr", "Wg", "Wu", "Wd", "dY")}
    out = O.layer(arrs["x"], arrs["Wr"], arrs["Wg"], arrs["Wu"], arrs["Wd"], wl.k, arrs["dY"], "fp64")
    grads = dict(x=out["dx"], Wr=out["dWr"], Wg=out["dWg"], Wu=out["dWu"], Wd=out["dWd"])
    rng = _rng(15)
    h = 1e-5
    skipped = 0
    for name in ("Wr", "x", "Wg", "Wu", "Wd"):
        a = arrs[name]
        if name == "Wr":
            coords = list(np.ndindex(a.shape))
        else:
            flat = rng.choice(a.size, 256, replace=False)
            coords = [np.unravel_index(i, a.shape) for i in flat]
        fd, an = [], []
        for c in coords:
            vals = []
            routes = []
            for sgn in (1, -1):
                b = {n: v for n, v in arrs.items()}
                b[name] = a.copy(); b[name][c] += sgn * h
                # the expert weights do not change the routing
                if name in ("x", "Wr"):
                    routes.append(O.topk_select(b["x"] @ b["Wr"], wl.k))
                vals.append(O.loss(b["x"], b["Wr"], b["Wg"], b["Wu"], b["Wd"], wl.k, b["dY"]))
            if routes and not np.array_equal(routes[0], routes[1]):
                skipped += 1
                continue
            fd.append((vals[0] - vals[1]) / (2 * h))
            an.append(grads[name][c])
        fd, an = np.array(fd), np.array(an)
        err = np.linalg.norm(fd - an) / np.linalg.norm(an)
        print(f"FD {name}: {len(fd)} coordinates, normwise relative error {err:.2e}")
        assert err <= 1e-6, (name, err)
    print(f"FD: {skipped} coordinates skipped for a routing change")
    assert skipped <= 16, skipped


def test_mx_layer_block_axes():
    """Each MX GEMM operand is blocked along that GEMM's contraction axis.
    Scaling by 2^16 a slice that lies inside whole blocks scales exactly the
    outputs it feeds and leaves the rest bit-identical.  Blocked along the
    wrong axis, the scaled slice would share blocks with other elements and
    push them 2^16 below their block maximum, into e4m3's subnormal range,
    changing other outputs."""
    S = 2.0 ** 16
    rng = _rng(16)
    T, d, E, f = 32, 64, 2, 64
    x = rng.standard_normal((T, d))
    Wg, Wu, Wd = _weights(rng, d, E, f, 0.1)
    idx = (np.arange(T) % E).astype(np.int32)[:, None]
    w = np.full((T, 1), 0.5)
    dY = rng.standard_normal((T, d))

    def run(x, Wg, Wu, Wd):
        fwd = O.layer_forward(x, Wg, Wu, Wd, idx, w, "mxfp8")
        fwd.update(O.layer_backward(fwd, x, Wg, Wu, Wd, idx, w, dY, "mxfp8"))
        return fwd

    base = run(x, Wg, Wu, Wd)
    rows0 = slice(int(base["offsets"][0]), int(base["offsets"][1]))
    # gate/up forward: Xs rows blocked along d
    x2 = x.copy(); x2[4] *= S
    r = run(x2, Wg, Wu, Wd)
    rr = base["dest_row"][4, 0]
    for key in ("Hg", "Hu"):
        np.testing.assert_array_equal(r[key][rr], base[key][rr] * S)
        np.testing.assert_array_equal(np.delete(r[key], rr, 0), np.delete(base[key], rr, 0))
    # gate/up forward: Wg[e] columns blocked along d
    Wg2 = Wg.copy(); Wg2[0][:, 5] *= S
    r = run(x, Wg2, Wu, Wd)
    np.testing.assert_array_equal(r["Hg"][rows0, 5], base["Hg"][rows0, 5] * S)
    np.testing.assert_array_equal(np.delete(r["Hg"], 5, 1), np.delete(base["Hg"], 5, 1))
    np.testing.assert_array_equal(r["Hu"], base["Hu"])
    # down forward: Wd[e] columns blocked along f
    Wd2 = Wd.copy(); Wd2[0][:, 7] *= S
    r = run(x, Wg, Wu, Wd2)
    np.testing.assert_array_equal(r["Ys"][rows0, 7], base["Ys"][rows0, 7] * S)
    np.testing.assert_array_equal(np.delete(r["Ys"], 7, 1), np.delete(base["Ys"], 7, 1))
    # down dgrad: Wd[e] rows blocked along d
    Wd3 = Wd.copy(); Wd3[0][9, :] *= S
    r = run(x, Wg, Wu, Wd3)
    for key in ("dHg", "dHu"):
        np.testing.assert_array_equal(r[key][rows0, 9], base[key][rows0, 9] * S)
        np.testing.assert_array_equal(np.delete(r[key], 9, 1), np.delete(base[key], 9, 1))
    # gate/up dgrad: Wg[e], Wu[e] rows blocked along f (the forward kept fixed,
    # so only the backward sees the scaled weights)
    fwd = O.layer_forward(x, Wg, Wu, Wd, idx, w, "mxfp8")
    b0 = O.layer_backward(fwd, x, Wg, Wu, Wd, idx, w, dY, "mxfp8")
    Wg4, Wu4 = Wg.copy(), Wu.copy()
    Wg4[0][11, :] *= S; Wu4[0][11, :] *= S
    r = O.layer_backward(fwd, x, Wg4, Wu4, Wd, idx, w, dY, "mxfp8")
    np.testing.assert_array_equal(r["dXs"][rows0, 11], b0["dXs"][rows0, 11] * S)
    np.testing.assert_array_equal(np.delete(r["dXs"], 11, 1), np.delete(b0["dXs"], 11, 1))
    # gate/up dgrad: dH rows blocked along 2f (one token's upstream gradient
    # scaled: its dYs row, dA row, dHg and dHu rows scale; only its dXs row follows)
    dY5 = dY.copy(); dY5[6] *= S
    r = O.layer_backward(fwd, x, Wg, Wu, Wd, idx, w, dY5, "mxfp8")
    r6 = fwd["dest_row"][6, 0]
    np.testing.assert_array_equal(r["dXs"][r6], b0["dXs"][r6] * S)
    np.testing.assert_array_equal(np.delete(r["dXs"], r6, 0), np.delete(b0["dXs"], r6, 0))


# ---------------------------------------------------------------------------
# sampled forms used by the full-size GPU checks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("prec", ["fp64", "bf16", "mxfp8"])
@pytest.mark.parametrize("router", [True, False])
def test_sampled_forms_match_full_layer(prec, router):
    """layer_tokens and expert_columns restate the layer for chosen tokens and
    for chosen d_ff columns of one expert; on a small layer they must give the
    full oracle's values at those places (up to float64 summation order)."""
    rng = _rng(21)
    T, d, E, f, k = 96, 64, 4, 64, 2
    q = (lambda a: O.round_bf16(a)) if prec != "fp64" else (lambda a: a)
    x = q(rng.standard_normal((T, d)))
    Wg, Wu, Wd = (q(a) for a in _weights(rng, d, E, f, 0.1))
    dY = q(rng.standard_normal((T, d)))
    if router:
        Wr = q(rng.standard_normal((d, E)) * 0.1)
        ref = O.layer(x, Wr, Wg, Wu, Wd, k, dY, prec)
        idx, w, logits = ref["topk_idx"], ref["topk_w"], ref["logits"]
    else:
        Wr, logits = None, None
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        w = rng.uniform(0, 1, (T, k)).astype(np.float32)
        ref = O.layer(x, None, Wg, Wu, Wd, k, dY, prec, topk_idx=idx, topk_w=w)
    tokens = np.array([0, 5, 17, 40, 95])
    s = O.layer_tokens(x, Wr, Wg, Wu, Wd, idx, w, dY, tokens, prec, logits=logits)
    close = dict(rtol=1e-9, atol=1e-12)
    rows = s["rows"]
    for key in ("Hg", "Hu", "A", "Ys", "dYs", "dHg", "dHu", "dXs"):
        np.testing.assert_allclose(s[key], ref[key][rows], err_msg=key, **close)
    for key in ("y", "dx") + (("dlogits",) if router else ()):
        np.testing.assert_allclose(s[key], np.asarray(ref[key])[tokens], err_msg=key, **close)
    np.testing.assert_allclose(s["dw"], ref["dw"][tokens], **close)
    cols = np.array([3, 30, 63])
    for e in range(E):
        c = O.expert_columns(x, Wg, Wu, Wd, idx, w, dY, e, cols, prec)
        np.testing.assert_allclose(c["dWg"], ref["dWg"][e][:, cols], **close)
        np.testing.assert_allclose(c["dWu"], ref["dWu"][e][:, cols], **close)
        np.testing.assert_allclose(c["dWd"], ref["dWd"][e][cols, :], **close)
    if prec == "mxfp8":
        # MXFP8 weight gradients (operands blocked along each expert's tokens)
        if router:
            refm = O.layer(x, Wr, Wg, Wu, Wd, k, dY, prec, mx_wgrad=True)
        else:
            refm = O.layer(x, None, Wg, Wu, Wd, k, dY, prec, topk_idx=idx, topk_w=w, mx_wgrad=True)
        for n in ("dWg", "dWu", "dWd"):
            assert np.any(refm[n] != ref[n]), n
        for e in range(E):
            c = O.expert_columns(x, Wg, Wu, Wd, idx, w, dY, e, cols, prec, mx_wgrad=True)
            np.testing.assert_allclose(c["dWg"], refm["dWg"][e][:, cols], **close)
            np.testing.assert_allclose(c["dWu"], refm["dWu"][e][:, cols], **close)
            np.testing.assert_allclose(c["dWd"], refm["dWd"][e][cols, :], **close)


# ---------------------------------------------------------------------------
# router variants: top-k renormalisation and the load-balancing loss
# ---------------------------------------------------------------------------

def test_renorm_closed_forms():
    rng = _rng(31)
    T, E, k = 40, 8, 3
    logits = rng.standard_normal((T, E))
    idx, w, p = O.route(logits, k, "fp64")
    idx_r, w_r, _ = O.route(logits, k, "fp64", renorm=True)
    np.testing.assert_array_equal(idx, idx_r)                      # same choice
    np.testing.assert_allclose(w_r.sum(axis=1), 1.0, rtol=1e-12)   # weights add to 1
    np.testing.assert_allclose(w_r[:, 1:] / w_r[:, :1], w[:, 1:] / w[:, :1], rtol=1e-12)
    # k = E: the chosen probabilities already add to 1
    _, wE, _ = O.route(logits, E, "fp64")
    _, wE_r, _ = O.route(logits, E, "fp64", renorm=True)
    np.testing.assert_allclose(wE_r, wE, rtol=1e-12)


def test_aux_loss_closed_forms():
    """Closed forms of load_balancing_loss_func's normalisation (HF OLMoE
    walkthrough, section 4): L = coef * E * sum_e (counts_e / T) * P_e."""
    T, E, k, c = 64, 8, 2, 0.01
    # all logits equal: p = 1/E, ties choose experts 0..k-1 for every token:
    # f = 1 on those k experts, L = c * E * k * (1/E) = c * k
    logits = np.zeros((T, E))
    idx, _, _ = O.route(logits, k, "fp64")
    L, dp = O.aux_loss(logits, idx, E, c, "fp64")
    assert abs(L - c * k) < 1e-15
    f = np.zeros(E); f[:k] = 1.0
    np.testing.assert_allclose(dp, c * E * f / T, rtol=1e-15)
    # balanced routing (every expert gets T*k/E slots), any probabilities:
    # f_e = k/E, sum_e P_e = 1, L = c * k
    rng = _rng(32)
    logits = rng.standard_normal((T, E))
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], np.int32)
    L, _ = O.aux_loss(logits, idx, E, c, "fp64")
    assert abs(L - c * k) < 1e-12
    # collapse: top-1 to expert 0 with p_0 -> 1 gives L -> c * E
    logits = np.full((T, E), -60.0); logits[:, 0] = 60.0
    idx, _, _ = O.route(logits, 1, "fp64")
    L, _ = O.aux_loss(logits, idx, E, c, "fp64")
    assert abs(L - c * E) < 1e-12


@pytest.mark.parametrize("renorm,aux", [(True, 0.0), (False, 0.05), (True, 0.05)])
def test_finite_differences_router_variants(renorm, aux):
    """Central differences of L = sum <y, dY> (+ the load-balancing loss) with
    renormalised weights and/or the auxiliary loss, on all of Wr and 32 seeded
    coordinates of x, skipping coordinates where the routing changes."""
    from moe_synth import workload, make_inputs
    wl = workload("tiny_fp32", T=48)
    inp = make_inputs(wl, seed=1)
    arrs = {n: inp[n].astype(np.float64) for n in ("x", "Wr", "Wg", "Wu", "Wd", "dY")}
    out = O.layer(arrs["x"], arrs["Wr"], arrs["Wg"], arrs["Wu"], arrs["Wd"], wl.k, arrs["dY"],
                  "fp64", renorm=renorm, aux_coef=aux)
    grads = dict(x=out["dx"], Wr=out["dWr"])
    rng = _rng(33)
    h = 1e-5
    skipped = 0
    for name in ("Wr", "x"):
        a = arrs[name]
        if name == "Wr":
            coords = list(np.ndindex(a.shape))
        else:
            coords = [np.unravel_index(i, a.shape) for i in rng.choice(a.size, 32, replace=False)]
        fd, an = [], []
        for c in coords:
            vals, routes = [], []
            for sgn in (1, -1):
                b = dict(arrs)
                b[name] = a.copy(); b[name][c] += sgn * h
                routes.append(O.topk_select(b["x"] @ b["Wr"], wl.k))
                vals.append(O.loss(b["x"], b["Wr"], b["Wg"], b["Wu"], b["Wd"], wl.k, b["dY"],
                                   renorm, aux))
            if not np.array_equal(routes[0], routes[1]):
                skipped += 1
                continue
            fd.append((vals[0] - vals[1]) / (2 * h))
            an.append(grads[name][c])
        fd, an = np.array(fd), np.array(an)
        err = np.linalg.norm(fd - an) / np.linalg.norm(an)
        assert err <= 1e-6, (name, err)
    assert skipped <= 8, skipped


def test_wgrad_f32_variant():
    """Float32 weight-gradient accumulation (OLMo-core 3 release summary,
    technical principle section): the same sums as the bf16 layer, kept in
    float32.  Rounding them to bf16 gives the bf16 layer's gradients (up to
    the rare double-rounding tie, never more than one bf16 unit apart);
    nothing else in the layer changes; a float32 layer is unaffected."""
    rng = _rng(41)
    T, d, E, f, k = 40, 16, 5, 24, 2
    x = O.round_bf16(rng.standard_normal((T, d)))
    Wr = O.round_bf16(rng.standard_normal((d, E)) * 0.3)
    Wg, Wu, Wd = (O.round_bf16(a) for a in _weights(rng, d, E, f))
    dY = O.round_bf16(rng.standard_normal((T, d)))
    a = O.layer(x, Wr, Wg, Wu, Wd, k, dY, "bf16")
    b = O.layer(x, Wr, Wg, Wu, Wd, k, dY, "bf16", wgrad_f32=True)
    for n in a:
        if n not in ("dWg", "dWu", "dWd"):
            np.testing.assert_array_equal(np.asarray(a[n]), np.asarray(b[n]), err_msg=n)
    for n in ("dWg", "dWu", "dWd"):
        w32, w16 = np.asarray(b[n]), np.asarray(a[n])
        np.testing.assert_array_equal(w32, w32.astype(np.float32).astype(np.float64))
        assert np.mean(O.round_bf16(w32) == w16) > 0.999, n
        ulp = np.abs(w16) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(w32 - w16) <= ulp), n
        assert np.any(w32 != w16), n   # the variant really keeps more bits
    c = O.layer(x, Wr, Wg, Wu, Wd, k, dY, "fp32")
    e = O.layer(x, Wr, Wg, Wu, Wd, k, dY, "fp32", wgrad_f32=True)
    for n in ("dWg", "dWu", "dWd"):
        np.testing.assert_array_equal(c[n], e[n])


def test_mx_weight_gradient_token_blocks():
    """MXFP8 weight gradients block their operands along the tokens of each
    expert: scaling one feature column of an operand by 2^16 scales exactly
    the gradient entries it feeds (every token block of that column scales by
    a power of two) and leaves every other entry bit-identical (blocked along
    the features instead, the scaled column would share blocks with the
    others and push them into e4m3's subnormals).  Blocks start at each
    expert's first row: scaling all of expert 0's rows leaves expert 1's
    gradients unchanged although expert 0 ends inside a 32-row block of the
    whole tensor."""
    S = 2.0 ** 16
    rng = _rng(43)
    R, d, f = 20 + 45, 48, 40
    offsets = np.array([0, 20, 65])
    Xs, A = rng.standard_normal((R, d)), rng.standard_normal((R, f))
    dHg, dHu = rng.standard_normal((R, f)), rng.standard_normal((R, f))
    dYs = rng.standard_normal((R, d))
    base = O.weight_gradients(Xs, dHg, dHu, A, dYs, offsets, mx_tokens=True)
    exact = O.weight_gradients(Xs, dHg, dHu, A, dYs, offsets, mx_tokens=False)
    for b, x in zip(base, exact):
        err = np.linalg.norm(b - x) / np.linalg.norm(x)
        assert 1e-4 < err < 0.1, err        # quantised, within MX error

    def check(args, changed):
        got = O.weight_gradients(*args, offsets, mx_tokens=True)
        for name, g, b in zip(("dWg", "dWu", "dWd"), got, base):
            m = changed.get(name)
            if m is None:
                np.testing.assert_array_equal(g, b, err_msg=name)
            else:
                np.testing.assert_array_equal(g[m], b[m] * S, err_msg=name)
                rest = np.ones(b.shape, bool); rest[m] = False
                np.testing.assert_array_equal(g[rest], b[rest], err_msg=name)

    X2 = Xs.copy(); X2[:, 5] *= S
    check((X2, dHg, dHu, A, dYs), {"dWg": (slice(None), 5), "dWu": (slice(None), 5)})
    G2 = dHg.copy(); G2[:, 7] *= S
    check((Xs, G2, dHu, A, dYs), {"dWg": (slice(None), slice(None), 7)})
    A2 = A.copy(); A2[:, 3] *= S
    check((Xs, dHg, dHu, A2, dYs), {"dWd": (slice(None), 3)})
    Y2 = dYs.copy(); Y2[:, 11] *= S
    check((Xs, dHg, dHu, A, Y2), {"dWd": (slice(None), slice(None), 11)})
    X3 = Xs.copy(); X3[:20] *= S
    check((X3, dHg, dHu, A, dYs), {"dWg": (0,), "dWu": (0,)})
