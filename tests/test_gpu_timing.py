"""GPU: the library's per-kernel timing (hca_timing_enable / hca_timing_read).

Each kernel family of a call is one timed region: per forward call the tile
images (head dim 512) and the forward kernel, per backward call the images,
the P / dS pass, the dQ pass, the key-stationary pass and the reduction.  A
read returns the regions since the previous read and recycles their events,
so a second round of calls reports the same counts; with timing disabled
nothing is recorded.
"""

import math

import pytest
import torch

import block_sparse_compressed_amd as hca
from hca_inputs import draw

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,H,expect", [
    (512, 64, {"transpose": 4, "fwd": 2, "bwd_pds": 2, "bwd_dq": 2, "bwd_dkv": 2,
               "dkv_reduce": 2}),
    (128, 16, {"fwd": 2, "bwd_dq": 2, "bwd_dkv": 2, "dkv_reduce": 2}),
])
def test_timing_counts_each_family_per_call(D, H, expect):
    S, r, W = 1024, 16, 128
    print(f"case timing D={D} H={H} S={S}", flush=True)
    q, kv, kvc, dout = draw(1, S, H, D, S // r, "bf16", 43, device="cuda")
    att = hca.HcaAttention(1, S, H, D, r, W, "bf16", None, None)
    scale = 1.0 / math.sqrt(D)
    o, lse = att.new_outputs()
    grads = att.new_grads()
    hca.hca_timing_read()  # drop anything recorded earlier
    try:
        for rnd in range(2):
            hca.hca_timing_enable(True)
            for _ in range(2):
                att.forward(q, kv, kvc, scale, o, lse)
                att.backward(q, kv, kvc, o, lse, dout, scale, grads=grads)
            hca.hca_timing_enable(False)
            t = hca.hca_timing_read()
            assert {k: v[0] for k, v in t.items()} == expect, (rnd, t)
            assert all(v[1] > 0.0 for v in t.values()), t
        att.forward(q, kv, kvc, scale, o, lse)
        att.backward(q, kv, kvc, o, lse, dout, scale, grads=grads)
        torch.cuda.synchronize()
        assert hca.hca_timing_read() == {}
    finally:
        hca.hca_timing_enable(False)
        hca.hca_timing_read()
