"""CPU oracle of the dropless top-k MoE expert layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library and never calls
it.  It is plain and slow on purpose: numpy in float64, a Python loop over
experts as in the HF OLMoE expert layer, no blocking or fusion.

Sources (page title, section):
  * "OLMoE in HF Transformers" walkthrough, section 2 (router): softmax of the
    router logits over experts in float32, torch.topk of the top_k experts,
    optional top-k renormalisation (default off), router weight without bias.
  * same page, section 3 (expert layer): experts stored as 3-D tensors; for
    each expert the routed tokens are gathered, gate/up projections, SiLU of
    gate times up, down projection, multiplied by the top-k weight and
    index-added back to the token rows.
  * olmoforge README, module table: row-wise expert parallel (token rows
    written straight into the expert's input buffer), grouped GEMM (the many
    small per-expert matmuls merged into one kernel), GPU-resident routing
    table; MXFP8 snippet (per-block shared scale, block size 32, e4m3 max 448).
  * OLMo-core 3 release notes (wedoingai summary, features / technical
    principle sections): paired SwiGLU backward, bf16-rounded weight-gradient
    accumulation.

Readings where the pages are silent or garbled (each also listed in the
design notes):
  * top-k ties go to the lower expert index; slots ordered by (logit desc,
    index asc); selection is made on the fp32 logits (softmax is monotone, so
    the chosen set is the same as selecting on probabilities).
  * weights are the softmax probabilities of the chosen experts, no
    renormalisation (the page's default).
  * rows of one expert's segment are in ascending token order (the HF loop
    visits tokens in order).
  * MX block scale 2^E with E the least integer such that 448 * 2^E >= amax
    (amax = 0 gives E = 0; E clamped to [-127, 127]); elements rounded to the
    nearest OCP e4m3 value, ties to even, saturating at +-448.  The printed
    snippet divides by amax/448 and rounds to an integer; that scale is not a
    power of two and an integer is not an e4m3 code, so the snippet is read
    for its intent (no overflow, zero block gets scale 1).
  * precision emulation: the oracle computes in float64 and rounds exactly
    the tensors the layer stores in its storage type (x-side rows Xs, Hg, Hu,
    A, Ys, y, dYs, dHg, dHu, dXs, dx, dW*).  Logits, weights, dw and dlogits
    are float32.

Pins (tests/test_oracle_pins.py, run with -m "not gpu"): bf16 and e4m3
rounding against torch's conversions; MX scale closed forms and worked
blocks; top-k against brute-force enumeration; metadata invariants; a
hand-worked routed layer (tests/golden/hand_worked_layer.json); special
cases reducing to dense torch computations; the backward against torch
autograd and against central finite differences.  tests/test_oracle_hf.py
pins the router, the expert layer (forward and autograd backward) and the
load-balancing loss against the HF OLMoE modules themselves
(transformers.models.olmoe.modeling_olmoe: OlmoeTopKRouter,
OlmoeSparseMoeBlock, load_balancing_loss_func).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

F64 = np.float64

# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------


def round_fp32(a) -> np.ndarray:
    """Nearest float32 (numpy's IEEE conversion), returned as float64."""
    return np.asarray(a, dtype=F64).astype(np.float32).astype(F64)


def _round_binary(a, p: int, emin: int) -> np.ndarray:
    """Round to the nearest value of a binary format with p significant bits
    and minimum normal exponent emin, ties to even (no overflow handling).

    A value in [2^e, 2^(e+1)) has spacing 2^(e-p+1); below 2^emin the
    spacing is that of the subnormals, 2^(emin-p+1)."""
    a = np.asarray(a, dtype=F64)
    mag = np.abs(a)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(mag)                   # mag = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)                # mag in [2^e, 2^(e+1))
    q = np.ldexp(1.0, e - p + 1)                # spacing
    return np.rint(a / q) * q                   # rint: ties to even


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(a) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, 8 exponent bits), ties to
    even, overflow to inf.  Pinned against torch's bf16 conversion."""
    r = _round_binary(a, 8, -126)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)


E4M3_MAX = 448.0


def e4m3_round(v) -> np.ndarray:
    """Nearest OCP FP8 e4m3 value (bias 7, 3 mantissa bits, normal exponents
    -6..8, subnormal spacing 2^-9, no infinities), ties to even, saturating
    at +-448.  Pinned against torch.float8_e4m3fn inside its range."""
    r = _round_binary(v, 4, -6)
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(v) -> np.ndarray:
    """Byte code (sign | 4-bit biased exponent | 3-bit mantissa) of values
    that already lie on the e4m3 grid."""
    v = np.asarray(v, dtype=F64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    mag = np.abs(v)
    sub = mag < 2.0 ** -6
    code = np.where(sub, np.rint(mag / 2.0 ** -9).astype(np.int64), 0)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(np.where(sub, 1.0, mag))
    e = ex - 1                                  # mag in [2^e, 2^(e+1))
    man = np.rint((np.where(sub, 1.0, mag) / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    norm_code = ((e + 7) << 3) | man
    code = np.where(sub, code, norm_code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Value of e4m3 byte codes (0x7F/0xFF, the NaN codes, are not produced)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.ldexp(1.0, ex - 7))
    return s * val


def mx_scale_exponent(amax) -> np.ndarray:
    """Shared block exponent E: least integer with 448 * 2^E >= amax;
    amax = 0 gives 0; clamped to [-127, 127] (the E8M0 range)."""
    amax = np.asarray(amax, dtype=F64)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    top = ex - 1                                 # amax in [2^top, 2^(top+1))
    # 448 * 2^(top-9) < 2^top <= amax and 448 * 2^(top-7) > 2^(top+1) > amax,
    # so E is top-8 or top-7: step up from top-9 while 448 * 2^E < amax
    E = top - 9
    for _ in range(3):
        E = np.where(E4M3_MAX * np.ldexp(1.0, E) >= amax, E, E + 1)
    E = np.where(amax > 0, E, 0)
    return np.clip(E, -127, 127).astype(np.int64)


def mx_quantize(a, axis: int, block: int = 32):
    """Block-quantise along `axis` in blocks of `block` consecutive elements.

    Returns (deq, E, q): dequantised values q * 2^E (float64), the block
    exponents, and the e4m3 grid values q (float64)."""
    a = np.asarray(a, dtype=F64)
    a_m = np.moveaxis(a, axis, -1)
    n = a_m.shape[-1]
    if n % block:
        raise ValueError("axis length must be a multiple of the block size")
    blocks = a_m.reshape(a_m.shape[:-1] + (n // block, block))
    E = mx_scale_exponent(np.max(np.abs(blocks), axis=-1))
    scale = np.ldexp(1.0, E)[..., None]
    q = e4m3_round(blocks / scale)
    deq = (q * scale).reshape(a_m.shape)
    return (np.moveaxis(deq, -1, axis), E,
            np.moveaxis(q.reshape(a_m.shape), -1, axis))


# ---------------------------------------------------------------------------
# router (HF OLMoE walkthrough, section 2)
# ---------------------------------------------------------------------------


def _f32(prec: str):
    """float32 rounding of router-side tensors; none in the exact fp64 mode."""
    return (lambda a: np.asarray(a, dtype=F64)) if prec == "fp64" else round_fp32


def router_logits(x, Wr, prec: str = "bf16") -> np.ndarray:
    """logits = x . Wr, summed in float64 and stored as float32."""
    return _f32(prec)(np.asarray(x, F64) @ np.asarray(Wr, F64))


def topk_select(logits, k: int) -> np.ndarray:
    """Per token, the k experts with the largest logit, slots ordered by
    (logit desc, expert index asc).  Pinned by brute force over all subsets."""
    logits = np.asarray(logits, dtype=F64)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    experts = np.arange(E)
    for t in range(T):
        order = np.lexsort((experts, -logits[t]))   # primary: -logit, then index
        idx[t] = order[:k]
    return idx


def softmax(logits) -> np.ndarray:
    """Softmax over experts in float64 of the (float32) logits."""
    l = np.asarray(logits, dtype=F64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def route(logits, k: int, prec: str = "bf16", renorm: bool = False):
    """Top-k experts and their softmax weights, float32.

    renorm (the page's optional top-k renormalisation, off by default): the k
    chosen probabilities are divided by their sum, so each token's weights
    add up to 1."""
    idx = topk_select(logits, k)
    p = softmax(logits)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        w = w / np.sum(w, axis=1, keepdims=True)
    return idx, _f32(prec)(w), p


def aux_loss(logits, topk_idx, E: int, coef: float = 0.01, prec: str = "bf16"):
    """Switch-style load-balancing loss of one layer (HF OLMoE walkthrough,
    section 4: load_balancing_loss_func in modeling_olmoe.py -- the experts'
    assignment frequencies times their mean router probabilities, summed;
    scaled by router_aux_loss_coef, default 0.01, before it joins the loss).

    f_e = counts_e / T is the fraction of tokens that route one of their k
    slots to expert e (the per-slot one-hot averaged over tokens and summed
    over the k slots, so sum_e f_e = k), P_e the mean over tokens of the
    softmax probability of e, and L = coef * E * sum_e f_e * P_e; perfectly
    balanced routing gives L = coef * k.  The top-k choice (so f) is piecewise
    constant in the logits; the gradient reaches the logits through P only:
    dL/dp[t,e] = coef * E * f_e / T for every token t.
    Returns (L, dL/dp per expert [E], float32 unless prec is fp64)."""
    p = softmax(logits)
    T = p.shape[0]
    idx = np.asarray(topk_idx, np.int64)
    k = idx.shape[1]
    counts = np.zeros(E)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    f = counts / T
    P = np.mean(p, axis=0)
    L = coef * E * float(np.sum(f * P))
    return L, _f32(prec)(coef * E * f / T)


# ---------------------------------------------------------------------------
# routing metadata (row-wise dispatch: each (token, slot) gets one row of
# its expert's segment; segments in expert order, tokens ascending inside)
# ---------------------------------------------------------------------------


def routing_metadata(topk_idx, E: int):
    """counts[E], offsets[E+1], dest_row[T,k], src_token[R] by plain loops."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    dest_row = np.empty((T, k), dtype=np.int64)
    src_token = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            dest_row[t, j] = fill[e]
            src_token[fill[e]] = t
            fill[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            dest_row.astype(np.int32), src_token.astype(np.int32))


# ---------------------------------------------------------------------------
# expert layer forward / backward
# ---------------------------------------------------------------------------


def sigmoid(z):
    """1/(1+e^-z), evaluated through e^-|z| so that it never overflows."""
    z = np.asarray(z, dtype=F64)
    ez = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))


def silu(z):
    return z * sigmoid(z)


def dsilu(z):
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def _storage_round(prec: str):
    if prec == "fp64":
        return lambda a: np.asarray(a, dtype=F64)
    if prec == "fp32":
        return round_fp32
    if prec in ("bf16", "mxfp8"):
        return round_bf16
    raise ValueError(prec)


def layer_forward(x, Wg, Wu, Wd, topk_idx, topk_w, prec: str = "fp64") -> Dict[str, np.ndarray]:
    """Forward of the expert part, given the routing.

    Per expert e (loop as in the HF expert layer): the rows of its segment
    are the routed tokens in ascending order; Hg = Xs.Wg[e], Hu = Xs.Wu[e],
    A = silu(Hg) * Hu, Ys = A.Wd[e]; then y[t] = sum_j w[t,j] * Ys[row(t,j)].

    prec 'fp64' rounds nothing; 'fp32'/'bf16' round the stored tensors;
    'mxfp8' additionally block-quantises both operands of the two forward
    GEMMs along their contraction axis."""
    rnd = _storage_round(prec)
    mx = prec == "mxfp8"
    x = np.asarray(x, F64)
    T, d = x.shape
    E, _, f = np.shape(Wg)
    k = np.shape(topk_idx)[1]
    counts, offsets, dest_row, src_token = routing_metadata(topk_idx, E)
    R = T * k
    Xs = rnd(x[src_token.astype(np.int64)])
    Hg = np.zeros((R, f)); Hu = np.zeros((R, f)); A = np.zeros((R, f)); Ys = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        Xe = Xs[lo:hi]
        Wge, Wue, Wde = (np.asarray(W[e], F64) for W in (Wg, Wu, Wd))
        if mx:
            Xe = mx_quantize(Xe, axis=1)[0]
            Wge = mx_quantize(Wge, axis=0)[0]
            Wue = mx_quantize(Wue, axis=0)[0]
        hg = Xe @ Wge
        hu = Xe @ Wue
        Hg[lo:hi] = rnd(hg)
        Hu[lo:hi] = rnd(hu)
        A[lo:hi] = rnd(silu(hg) * hu)
        Ae = A[lo:hi]
        if mx:
            Ae = mx_quantize(Ae, axis=1)[0]
            Wde = mx_quantize(Wde, axis=0)[0]
        Ys[lo:hi] = rnd(Ae @ Wde)
    w = np.asarray(topk_w, F64)
    y = np.zeros((T, d))
    for t in range(T):
        acc = np.zeros(d)
        for j in range(k):
            acc += w[t, j] * Ys[dest_row[t, j]]
        y[t] = acc
    y = rnd(y)
    return dict(counts=counts, offsets=offsets, dest_row=dest_row, src_token=src_token,
                Xs=Xs, Hg=Hg, Hu=Hu, A=A, Ys=Ys, y=y)


def mx_quantize_rows(a, block: int = 32):
    """Block-quantise along the row axis (axis 0) in blocks of `block` rows
    starting at row 0; a last partial block is taken as if padded with zero
    rows (zeros change neither its largest magnitude nor any product).
    Returns the dequantised values (float64)."""
    a = np.asarray(a, dtype=F64)
    n = a.shape[0]
    pad = (-n) % block
    if pad:
        a = np.concatenate([a, np.zeros((pad,) + a.shape[1:])], axis=0)
    return mx_quantize(a, axis=0, block=block)[0][:n]


def weight_gradients(Xs, dHg, dHu, A, dYs, offsets, mx_tokens: bool = False):
    """Per expert e with rows [lo, hi): dWg[e] = Xs^T.dHg, dWu[e] = Xs^T.dHu,
    dWd[e] = A^T.dYs over the expert's rows, float64 sums (an expert without
    rows gets zeros).  mx_tokens: every operand is first block-quantised
    along its contraction axis, the tokens of the expert's segment, in blocks
    of 32 rows from the segment's first row (mx_quantize_rows)."""
    E = len(offsets) - 1
    d, f, dm = np.shape(Xs)[1], np.shape(dHg)[1], np.shape(dYs)[1]
    dWg = np.zeros((E, d, f)); dWu = np.zeros((E, d, f)); dWd = np.zeros((E, f, dm))
    q = mx_quantize_rows if mx_tokens else (lambda a: np.asarray(a, dtype=F64))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xs, g, u, a, y = (q(t[lo:hi]) for t in (Xs, dHg, dHu, A, dYs))
        dWd[e] = a.T @ y
        dWg[e] = xs.T @ g
        dWu[e] = xs.T @ u
    return dWg, dWu, dWd


def layer_backward(fwd, x, Wg, Wu, Wd, topk_idx, topk_w, dY, prec: str = "fp64",
                   wgrad_f32: bool = False, mx_wgrad: bool = False) -> Dict[str, np.ndarray]:
    """Backward of the expert part for the loss L = sum_t <y[t], dY[t]>.

    dw[t,j] = <dY[t], Ys[row]>; dYs[row] = w[t,j] dY[t];
    dA = dYs.Wd[e]^T; paired SwiGLU backward
      dHg = dA * Hu * silu'(Hg),  dHu = dA * silu(Hg)   (from the stored Hg, Hu);
    dXs = dHg.Wg[e]^T + dHu.Wu[e]^T; dx[t] = sum_j dXs[row(t,j)];
    dWd[e] = A^T.dYs, dWg[e] = Xs^T.dHg, dWu[e] = Xs^T.dHu (empty expert: 0).
    'mxfp8' quantises both operands of the two dgrad GEMMs along their
    contraction axis; weight gradients use the unquantised operands.
    wgrad_f32 (OLMo-core 3 release summary, technical principle section:
    optional FP32 gradient accumulation): the weight gradients are kept in
    float32 instead of being rounded to the storage type.
    mx_wgrad ('mxfp8' only; olmoforge README, MXFP8 block quantisation applied
    to the weight-gradient GEMMs as well): their operands are block-quantised
    along the tokens of each expert (weight_gradients)."""
    rnd = _storage_round(prec)
    wrnd = _f32(prec) if wgrad_f32 else rnd
    mx = prec == "mxfp8"
    T, d = np.shape(x)
    E, _, f = np.shape(Wg)
    k = np.shape(topk_idx)[1]
    dest_row, offsets = fwd["dest_row"], fwd["offsets"]
    R = T * k
    dY = np.asarray(dY, F64)
    w = np.asarray(topk_w, F64)
    Ys = fwd["Ys"]
    dw = np.zeros((T, k))
    dYs = np.zeros((R, d))
    for t in range(T):
        for j in range(k):
            r = dest_row[t, j]
            dw[t, j] = dY[t] @ Ys[r]
            dYs[r] = w[t, j] * dY[t]
    dw = _f32(prec)(dw)
    dYs = rnd(dYs)
    dHg = np.zeros((R, f)); dHu = np.zeros((R, f)); dXs = np.zeros((R, d))
    Hg, Hu, A, Xs = fwd["Hg"], fwd["Hu"], fwd["A"], fwd["Xs"]
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        Wge, Wue, Wde = (np.asarray(W[e], F64) for W in (Wg, Wu, Wd))
        g = dYs[lo:hi]
        gq, Wdq = g, Wde
        if mx:
            gq = mx_quantize(g, axis=1)[0]
            Wdq = mx_quantize(Wde, axis=1)[0]
        dA = gq @ Wdq.T
        hg, hu = Hg[lo:hi], Hu[lo:hi]
        dHg[lo:hi] = rnd(dA * hu * dsilu(hg))
        dHu[lo:hi] = rnd(dA * silu(hg))
        a_g, a_u, Wgq, Wuq = dHg[lo:hi], dHu[lo:hi], Wge, Wue
        if mx:
            a_g = mx_quantize(a_g, axis=1)[0]
            a_u = mx_quantize(a_u, axis=1)[0]
            Wgq = mx_quantize(Wge, axis=1)[0]
            Wuq = mx_quantize(Wue, axis=1)[0]
        dXs[lo:hi] = rnd(a_g @ Wgq.T + a_u @ Wuq.T)
    dWg, dWu, dWd = weight_gradients(Xs, dHg, dHu, A, dYs, offsets, mx and mx_wgrad)
    dWg, dWu, dWd = wrnd(dWg), wrnd(dWu), wrnd(dWd)
    dx = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            dx[t] += dXs[dest_row[t, j]]
    dx = rnd(dx)
    return dict(dw=dw, dYs=dYs, dHg=dHg, dHu=dHu, dXs=dXs, dx=dx, dWg=dWg, dWu=dWu, dWd=dWd)


def router_backward(x, Wr, logits, topk_idx, dw, dx_experts, prec: str = "fp64",
                    renorm: bool = False, aux_dp=None):
    """Router backward: dp[t,e] = dw[t,j] where e = idx[t,j], else 0;
    dlogits = p * (dp - <p, dp>) (softmax backward); dWr = x^T.dlogits;
    dx = dx_experts + dlogits.Wr^T.  dlogits is float32.

    renorm: w_j = p_{e_j} / S with S the sum of the chosen probabilities, so
    dp[t, e_m] = (dw_m - sum_j dw_j w_j) / S for the chosen experts (0 for the
    others).  aux_dp (from aux_loss): added to dp[t, e] for every token."""
    rnd = _storage_round(prec)
    p = softmax(logits)
    T, E = p.shape
    dp = np.zeros((T, E))
    idx = np.asarray(topk_idx, np.int64)
    dw = np.asarray(dw, F64)
    for t in range(T):
        if renorm:
            pc = p[t, idx[t]]
            S = float(np.sum(pc))
            w = pc / S
            inner_w = float(np.sum(dw[t] * w))
            for j in range(idx.shape[1]):
                dp[t, idx[t, j]] = (dw[t, j] - inner_w) / S
        else:
            for j in range(idx.shape[1]):
                dp[t, idx[t, j]] = dw[t, j]
    if aux_dp is not None:
        dp += np.asarray(aux_dp, F64)[None, :]
    inner = np.sum(p * dp, axis=1, keepdims=True)
    dlogits = _f32(prec)(p * (dp - inner))
    x = np.asarray(x, F64)
    dWr = rnd(x.T @ dlogits)
    dx = rnd(np.asarray(dx_experts, F64) + dlogits @ np.asarray(Wr, F64).T)
    return dict(dlogits=dlogits, dWr=dWr, dx=dx)


def layer(x, Wr, Wg, Wu, Wd, k, dY, prec: str = "fp64", logits=None,
          topk_idx=None, topk_w=None, renorm: bool = False,
          aux_coef: float = 0.0, wgrad_f32: bool = False,
          mx_wgrad: bool = False) -> Dict[str, np.ndarray]:
    """Whole layer forward + backward.

    With a router (Wr given): logits = x.Wr unless `logits` is passed in,
    then top-k routing (renormalised with `renorm`).  aux_coef > 0 adds the
    load-balancing loss (aux_loss) to the loss whose gradient the backward
    computes.  Without a router (pre-routed rows) topk_idx / topk_w are
    inputs and there is no router backward."""
    out: Dict[str, np.ndarray] = {}
    aux_dp = None
    if Wr is not None:
        if logits is None:
            logits = router_logits(x, Wr, prec)
        topk_idx, topk_w, _ = route(logits, k, prec, renorm)
        out.update(logits=np.asarray(logits, F64), topk_idx=topk_idx, topk_w=topk_w)
        if aux_coef:
            L, aux_dp = aux_loss(logits, topk_idx, np.shape(Wg)[0], aux_coef, prec)
            out.update(aux_loss=L, aux_dp=aux_dp)
    fwd = layer_forward(x, Wg, Wu, Wd, topk_idx, topk_w, prec)
    out.update(fwd)
    if dY is not None:
        bwd = layer_backward(fwd, x, Wg, Wu, Wd, topk_idx, topk_w, dY, prec, wgrad_f32, mx_wgrad)
        out.update(bwd)
        if Wr is not None:
            rb = router_backward(x, Wr, logits, topk_idx, bwd["dw"], bwd["dx"], prec, renorm,
                                 aux_dp)
            out["dx_experts"] = bwd["dx"]
            out.update(rb)
    return out


def loss(x, Wr, Wg, Wu, Wd, k, dY, renorm: bool = False, aux_coef: float = 0.0) -> float:
    """L = sum_t <y[t], dY[t]> (+ the load-balancing loss) of the layer in
    float64 with no rounding, routing taken on unrounded logits (used by the
    finite-difference pins)."""
    logits = router_logits(x, Wr, "fp64")
    idx, w, _ = route(logits, k, "fp64", renorm)
    y = layer_forward(x, Wg, Wu, Wd, idx, w, "fp64")["y"]
    L = float(np.sum(y * np.asarray(dY, F64)))
    if aux_coef:
        L += aux_loss(logits, idx, np.shape(Wg)[0], aux_coef, "fp64")[0]
    return L


# ---------------------------------------------------------------------------
# sampled forms (full-size checks): the same definitions as layer_forward /
# layer_backward / router_backward, evaluated only for chosen tokens or for
# chosen columns of one expert, so that a full-size layer can be checked
# without computing every output.
# ---------------------------------------------------------------------------


def _mxq(a, axis):
    return mx_quantize(a, axis=axis)[0]


def layer_tokens(x, Wr, Wg, Wu, Wd, topk_idx, topk_w, dY, tokens, prec: str = "fp64",
                 logits=None) -> Dict[str, object]:
    """Per-token forward + backward for the given tokens.

    topk_idx / topk_w / logits are the routing of every token (logits only
    with a router); the metadata is derived from topk_idx as in
    routing_metadata.  Returns per-token arrays y, dw, dx (and dlogits with a
    router) indexed like `tokens`, and per-row arrays Hg, Hu, A, Ys, dYs, dHg,
    dHu, dXs for the rows rows = dest_row[tokens] (shape [len(tokens), k])."""
    rnd = _storage_round(prec)
    mx = prec == "mxfp8"
    x = np.asarray(x, F64)
    E = np.shape(Wg)[0]
    idx = np.asarray(topk_idx, np.int64)
    k = idx.shape[1]
    _, _, dest_row, _ = routing_metadata(topk_idx, E)
    w = np.asarray(topk_w, F64)
    dYa = np.asarray(dY, F64)
    tokens = np.asarray(tokens, np.int64)
    n = len(tokens)
    f = np.shape(Wg)[2]
    d = x.shape[1]
    shp_f, shp_d = (n, k, f), (n, k, d)
    Hg, Hu, A, dHg, dHu = (np.zeros(shp_f) for _ in range(5))
    Ys, dYs, dXs = (np.zeros(shp_d) for _ in range(3))
    y, dx_e = np.zeros((n, d)), np.zeros((n, d))
    dw = np.zeros((n, k))
    cache: Dict[int, tuple] = {}
    for a, t in enumerate(tokens):
        for j in range(k):
            e = int(idx[t, j])
            if e not in cache:
                Wge, Wue, Wde = (np.asarray(W[e], F64) for W in (Wg, Wu, Wd))
                if mx:
                    cache[e] = (_mxq(Wge, 0), _mxq(Wue, 0), _mxq(Wde, 0),
                                _mxq(Wde, 1), _mxq(Wge, 1), _mxq(Wue, 1))
                else:
                    cache[e] = (Wge, Wue, Wde, Wde, Wge, Wue)
            Wgf, Wuf, Wdf, Wdb, Wgb, Wub = cache[e]
            xs = rnd(x[t])[None, :]
            xq = _mxq(xs, 1) if mx else xs
            hg, hu = xq @ Wgf, xq @ Wuf
            Hg[a, j], Hu[a, j] = rnd(hg)[0], rnd(hu)[0]
            A[a, j] = rnd(silu(hg) * hu)[0]
            aq = _mxq(A[a, j][None, :], 1) if mx else A[a, j][None, :]
            Ys[a, j] = rnd(aq @ Wdf)[0]
    for a, t in enumerate(tokens):
        acc = np.zeros(d)
        for j in range(k):
            acc += w[t, j] * Ys[a, j]
        y[a] = acc
    y = rnd(y)
    for a, t in enumerate(tokens):
        for j in range(k):
            e = int(idx[t, j])
            _, _, _, Wdb, Wgb, Wub = cache[e]
            dw[a, j] = dYa[t] @ Ys[a, j]
            dYs[a, j] = rnd(w[t, j] * dYa[t])
            g = dYs[a, j][None, :]
            gq = _mxq(g, 1) if mx else g
            dA = (gq @ Wdb.T)[0]
            dHg[a, j] = rnd(dA * Hu[a, j] * dsilu(Hg[a, j]))
            dHu[a, j] = rnd(dA * silu(Hg[a, j]))
            ag, au = dHg[a, j][None, :], dHu[a, j][None, :]
            if mx:
                ag, au = _mxq(ag, 1), _mxq(au, 1)
            dXs[a, j] = rnd(ag @ Wgb.T + au @ Wub.T)[0]
        for j in range(k):
            dx_e[a] += dXs[a, j]
    dw = _f32(prec)(dw)
    dx_e = rnd(dx_e)
    out: Dict[str, object] = dict(rows=dest_row[tokens], y=y, dw=dw, Hg=Hg, Hu=Hu, A=A, Ys=Ys,
                                  dYs=dYs, dHg=dHg, dHu=dHu, dXs=dXs, dx=dx_e)
    if Wr is not None:
        p = softmax(np.asarray(logits)[tokens])
        dp = np.zeros_like(p)
        for a, t in enumerate(tokens):
            for j in range(k):
                dp[a, idx[t, j]] = dw[a, j]
        inner = np.sum(p * dp, axis=1, keepdims=True)
        dl = _f32(prec)(p * (dp - inner))
        out["dlogits"] = dl
        out["dx"] = rnd(dx_e + dl @ np.asarray(Wr, F64).T)
    return out


def expert_columns(x, Wg, Wu, Wd, topk_idx, topk_w, dY, e: int, cols,
                   prec: str = "fp64", mx_wgrad: bool = False) -> Dict[str, np.ndarray]:
    """Weight gradients of expert e at the given columns c of d_ff:
    dWg[e][:, cols], dWu[e][:, cols] and dWd[e][cols, :], each summed over all
    of e's rows exactly as layer_backward does (the column c of Hg, Hu, A, dA
    depends only on column c of Wg, Wu and on row c of Wd; with mx_wgrad the
    token-axis blocks of a column depend only on that column)."""
    rnd = _storage_round(prec)
    mx = prec == "mxfp8"
    E = np.shape(Wg)[0]
    _, offsets, _, src_token = routing_metadata(topk_idx, E)
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    d = np.shape(x)[1]
    cols = np.asarray(cols, np.int64)
    if hi == lo:
        z = np.zeros((d, len(cols)))
        return dict(dWg=z, dWu=z.copy(), dWd=np.zeros((len(cols), d)))
    # weight of each row of e: the (t, j) slot that lands on it
    idx = np.asarray(topk_idx, np.int64)
    w = np.asarray(topk_w, F64)
    rows_w = np.zeros(hi - lo)
    tok = np.asarray(src_token[lo:hi], np.int64)
    for r, t in enumerate(tok):
        rows_w[r] = w[t, list(idx[t]).index(e)]
    Xs = rnd(np.asarray(x, F64)[tok])
    Xq = _mxq(Xs, 1) if mx else Xs
    Wgc = np.asarray(Wg[e], F64)[:, cols]
    Wuc = np.asarray(Wu[e], F64)[:, cols]
    Wdr = np.asarray(Wd[e], F64)[cols, :]
    if mx:
        Wgc, Wuc = _mxq(Wgc, 0), _mxq(Wuc, 0)
    hg, hu = Xq @ Wgc, Xq @ Wuc
    Hg, Hu = rnd(hg), rnd(hu)
    A = rnd(silu(hg) * hu)
    dYs = rnd(rows_w[:, None] * np.asarray(dY, F64)[tok])
    g = _mxq(dYs, 1) if mx else dYs
    Wdb = _mxq(Wdr, 1) if mx else Wdr
    dA = g @ Wdb.T
    dHg = rnd(dA * Hu * dsilu(Hg))
    dHu = rnd(dA * silu(Hg))
    if mx and mx_wgrad:
        Xs, dHg, dHu, A, dYs = (mx_quantize_rows(t) for t in (Xs, dHg, dHu, A, dYs))
    return dict(dWg=rnd(Xs.T @ dHg), dWu=rnd(Xs.T @ dHu), dWd=rnd(A.T @ dYs))
