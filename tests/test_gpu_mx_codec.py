"""Exhaustive check of the MXFP8 block codec on the GPU against the oracle.

Every finite bf16 value goes through the quantising dispatch (moe_dispatch
with prec MXFP8, one expert, top-1, so the dispatched rows are the input
rows in order), in 32-element blocks, and the e4m3 bytes and E8M0 scale
bytes must equal the oracle's (mx_quantize along the row, e4m3_encode) bit
for bit.  Three arrangements: bit patterns in order (blocks of neighbouring
magnitudes), a seeded shuffle (blocks mixing magnitudes, so many elements
fall to subnormal codes or zero), and blocks whose largest magnitude is
pinned to 448 * 2^j for j in {-10, 0, 5} (block exponent exactly j) with the
other 31 values drawn from all patterns of smaller magnitude.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.parity import say

pytestmark = pytest.mark.gpu

D = 64  # row width: two blocks per row


def _finite_patterns() -> np.ndarray:
    p = np.arange(65536, dtype=np.uint32)
    exp = (p >> 7) & 0xFF
    return p[exp != 0xFF].astype(np.uint16)


def _bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rows(bits: np.ndarray) -> np.ndarray:
    n = (len(bits) + D - 1) // D * D
    out = np.zeros(n, np.uint16)
    out[: len(bits)] = bits
    return out.reshape(-1, D)


def _gpu_quantise(rows_bits: np.ndarray):
    import routing_grouped_gemm_amd as rgg
    T = rows_bits.shape[0]
    x = rgg.upload(rows_bits, torch.bfloat16)
    idx = torch.zeros(T, 1, dtype=torch.int32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    counts, offsets = torch.empty(1, **i32), torch.empty(2, **i32)
    dest, src = torch.empty(T, 1, **i32), torch.empty(T, **i32)
    Xs = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    Xq = torch.empty(T, D, dtype=torch.uint8, device="cuda")
    Xq_scale = torch.empty(rgg.mx_scale_shape(T, D), dtype=torch.uint8, device="cuda")
    n = rgg.moe_workspace_size("dispatch", T, D, 1, 64, 1, torch.bfloat16, "mxfp8")
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    rgg.moe_dispatch(x, idx, 1, counts, offsets, dest, src, Xs, ws, Xq, Xq_scale, "mxfp8")
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), rgg.mx_scale_rows(Xq_scale, T, D).cpu().numpy()


def _check(rows_bits: np.ndarray, label: str):
    q_gpu, s_gpu = _gpu_quantise(rows_bits)
    vals = _bits_to_f64(rows_bits)
    _, E, q = O.mx_quantize(vals, axis=1)
    codes = O.e4m3_encode(q)
    bad = int(np.count_nonzero(q_gpu != codes))
    say(f"  {label}: {rows_bits.size} values, {bad} code mismatches")
    np.testing.assert_array_equal(q_gpu, codes)
    np.testing.assert_array_equal(s_gpu.astype(np.int64), E + 127)


def test_codec_all_bf16_in_order():
    _check(_rows(_finite_patterns()), "in order")


def test_codec_all_bf16_shuffled():
    bits = _finite_patterns()
    rng = np.random.default_rng(0)
    _check(_rows(bits[rng.permutation(len(bits))]), "shuffled")


@pytest.mark.parametrize("j", [-10, 0, 5])
def test_codec_pinned_block_exponent(j):
    bits = _finite_patterns()
    v = _bits_to_f64(bits)
    anchor = 448.0 * 2.0 ** j
    small = bits[np.abs(v) <= anchor]
    rng = np.random.default_rng(100 + j)
    small = small[rng.permutation(len(small))]
    nblk = (len(small) + 30) // 31
    blocks = np.zeros((nblk, 32), np.uint16)
    flat = np.zeros(nblk * 31, np.uint16)
    flat[: len(small)] = small
    blocks[:, 1:] = flat.reshape(nblk, 31)
    anchor_bits = (np.array([anchor], np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
    assert _bits_to_f64(np.array([anchor_bits]))[0] == anchor
    blocks[:, 0] = anchor_bits
    if nblk % 2:
        blocks = np.concatenate([blocks, blocks[:1]])
    _check(blocks.reshape(-1, D), f"block exponent {j}")
    _, E, _ = O.mx_quantize(_bits_to_f64(blocks.reshape(-1, D)), axis=1)
    assert np.all(E == j)
