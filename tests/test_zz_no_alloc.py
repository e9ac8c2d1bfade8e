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


@pytest.mark.parametrize("dtype_d", [("bf16", 512), ("bf16", 128)])
def test_noalloc_matches_workspace_forward_two_calls(dtype_d):
    dtype, D = dtype_d
    H = 64 if D == 512 else 16
    big = run_pair(1, 12000, H, D, 64, 128, dtype, [[5000, 7000]], seed=31)
    small = run_pair(1, 1500, H, D, 16, 100, dtype, None, seed=32)
    assert small < big


def test_noalloc_float32_needs_no_scratch():
    assert run_pair(1, 489, 4, 64, 16, 64, "f32", None, seed=33) == 0
