"""GPU: the allocation-free forward (hca_attn_fwd_noalloc) through the C ABI.

It must give the same O and LSE as hca_attn_fwd (same kernels, the library's
scratch in place of the caller's workspace), bit for bit, on two calls in a
row where the second is smaller than the first, so it reuses scratch the first
call left filled.
"""

import math

import pytest
import torch

import block_sparse_compressed_amd as hca
from hca_inputs import draw, starts_csr

pytestmark = pytest.mark.gpu


def run_pair(B, S, H, D, r, W, dtype, lengths, seed):
    Sc = S // r
    q, kv, kvc, _ = draw(B, S, H, D, Sc, dtype, seed, device="cuda")
    starts, counts = starts_csr(lengths, B)
    att = hca.HcaAttention(B, S, H, D, r, W, dtype, starts, counts)
    assert att.info.ws_fwd_bytes <= hca.NOALLOC_SCRATCH_BYTES
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = att.new_outputs()
    att.forward(q, kv, kvc, scale, o_ref, lse_ref)
    o, lse = att.new_outputs()
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    hca.hca_attn_fwd_noalloc(att.plan, q, kv, kvc if Sc > 0 else None, scale, o, lse)
    torch.cuda.synchronize()
    view = (lambda t: t.view(torch.int16)) if o.dtype == torch.bfloat16 else (lambda t: t)
    assert torch.equal(view(o), view(o_ref))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
    return att.info.ws_fwd_bytes


def test_noalloc_matches_workspace_forward_two_calls():
    """Head dim 512 (the forward's tile images live in the scratch array): two
    calls in a row, the second smaller, each equal to the workspace forward."""
    big = run_pair(1, 12000, 64, 512, 64, 128, "bf16", [[5000, 7000]], seed=31)
    small = run_pair(1, 1500, 64, 512, 16, 100, "bf16", None, seed=32)
    assert 0 < small < big


@pytest.mark.parametrize("dtype_d", [("f32", 64), ("bf16", 128)])
def test_noalloc_needs_no_scratch_below_d512(dtype_d):
    """float32 and head dim 64 / 128 forwards use no workspace: the entry point
    runs them without touching the scratch array."""
    dtype, D = dtype_d
    H = 4 if dtype == "f32" else 16
    assert run_pair(1, 489, H, D, 16, 64, dtype, None, seed=33) == 0
