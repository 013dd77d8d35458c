"""moe_dispatch_noalloc (the dispatch on the library's static scratch, for
callers that cannot allocate) against moe_dispatch with a caller workspace,
through the C ABI: bit-identical routing metadata and dispatched rows (and,
for MXFP8, codes and block scales), on two calls in a row, the second with a
smaller problem, so that the scratch holds the first call's tables when the
second one starts.  The metadata is also checked against the oracle."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.parity import say, to_np

pytestmark = pytest.mark.gpu


def _inputs(T, d, E, k, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    return x, idx


def _buffers(T, d, E, k, mx):
    import routing_grouped_gemm_amd as rgg
    R = T * k
    i32 = dict(dtype=torch.int32, device="cuda")
    b = dict(counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
             dest_row=torch.full((T, k), -7, **i32), src_token=torch.full((R,), -7, **i32),
             Xs=torch.full((R, d), -3.0, dtype=torch.bfloat16, device="cuda"))
    if mx:
        b["Xq"] = torch.full((R, d), 0x55, dtype=torch.uint8, device="cuda")
        b["Xq_scale"] = torch.full(rgg.mx_scale_shape(R, d), 0x55, dtype=torch.uint8,
                                   device="cuda")
    return b


def _run_pair(T, d, E, k, prec, seed):
    import routing_grouped_gemm_amd as rgg
    mx = prec == "mxfp8"
    say(f"[case] dispatch_noalloc T={T} d={d} E={E} k={k} {prec} seed={seed}")
    x_h, idx_h = _inputs(T, d, E, k, seed)
    x, idx = x_h.cuda(), rgg.upload(idx_h)
    ref, got = _buffers(T, d, E, k, mx), _buffers(T, d, E, k, mx)
    ws = torch.empty(rgg.moe_workspace_size("dispatch", T, d, E, 64, k, torch.bfloat16, prec),
                     dtype=torch.uint8, device="cuda")
    q = lambda b: dict(Xq=b.get("Xq"), Xq_scale=b.get("Xq_scale"))
    rgg.moe_dispatch(x, idx, E, ref["counts"], ref["offsets"], ref["dest_row"], ref["src_token"],
                     ref["Xs"], ws, prec=prec, **q(ref))
    rgg.moe_dispatch_noalloc(x, idx, E, got["counts"], got["offsets"], got["dest_row"],
                             got["src_token"], got["Xs"], prec=prec, **q(got))
    torch.cuda.synchronize()
    for n in ref:
        a, b = ref[n], got[n]
        if n == "Xq_scale":
            a, b = rgg.mx_scale_rows(a, T * k, d), rgg.mx_scale_rows(b, T * k, d)
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (n, T, E)
    counts, offsets, dest_row, src_token = O.routing_metadata(idx_h, E)
    np.testing.assert_array_equal(to_np(got["counts"]), counts)
    np.testing.assert_array_equal(to_np(got["offsets"]), offsets)
    np.testing.assert_array_equal(to_np(got["dest_row"]), dest_row)
    np.testing.assert_array_equal(to_np(got["src_token"]), src_token)
    xs = to_np(got["Xs"])
    np.testing.assert_array_equal(xs, x_h.float().numpy().astype(np.float64)[src_token])
    say(f"  equal to moe_dispatch and the oracle ({T * k} rows)")


@pytest.mark.parametrize("prec,big,small", [
    ("bf16", (4096, 512, 64, 8), (1000, 256, 32, 4)),
    ("mxfp8", (2048, 256, 16, 4), (300, 128, 8, 2)),
])
def test_dispatch_noalloc_matches_dispatch(prec, big, small):
    _run_pair(*big, prec, seed=1)
    _run_pair(*small, prec, seed=2)
