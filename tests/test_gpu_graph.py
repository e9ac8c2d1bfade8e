"""GPU: forward and backward captured in a HIP graph (torch.cuda.graph) and
replayed, each replay bitwise equal to the eager calls.

The backward with stored P and dS forks its dQ pass onto the library's second
stream and joins it back with events; under capture the fork and join become
graph edges.  Between replays the outputs are NaN-filled by eager work, and
each replay is checked, so nothing is taken from a previous replay.  The
allocation-free forward (the callers it serves include code under capture) is
captured the same way.
"""

import math

import pytest
import torch

import block_sparse_compressed_amd as hca
from hca_inputs import draw

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def check_replays(g, outs, ref, n=3):
    for rep in range(n):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(bits(a), bits(b)), ("replay", rep)


@pytest.mark.parametrize("D,H", [(512, 64), (128, 16)])
def test_forward_backward_graph_replays(D, H):
    S, r, W = 2048, 16, 128
    print(f"case D={D} H={H} S={S} r={r} W={W}", flush=True)
    q, kv, kvc, dout = draw(1, S, H, D, S // r, "bf16", 41, device="cuda")
    att = hca.HcaAttention(1, S, H, D, r, W, "bf16", None, None)
    assert (att.info.ws_pds_bytes > 0) == (D == 512)
    scale = 1.0 / math.sqrt(D)
    o, lse = att.new_outputs()
    grads = att.new_grads()
    att.forward(q, kv, kvc, scale, o, lse)
    att.backward(q, kv, kvc, o, lse, dout, scale, grads=grads)
    torch.cuda.synchronize()
    outs = (o, lse) + tuple(grads)
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        att.forward(q, kv, kvc, scale, o, lse, stream=s)
        att.backward(q, kv, kvc, o, lse, dout, scale, grads=grads, stream=s)
    check_replays(g, outs, ref)


def test_noalloc_forward_graph_replays():
    S, H, D, r, W = 2048, 64, 512, 16, 128
    print(f"case noalloc D={D} H={H} S={S}", flush=True)
    q, kv, kvc, _ = draw(1, S, H, D, S // r, "bf16", 42, device="cuda")
    att = hca.HcaAttention(1, S, H, D, r, W, "bf16", None, None)
    assert 0 < att.info.ws_fwd_bytes <= hca.NOALLOC_SCRATCH_BYTES
    scale = 1.0 / math.sqrt(D)
    o, lse = att.new_outputs()
    att.forward(q, kv, kvc, scale, o, lse)
    torch.cuda.synchronize()
    ref = [o.clone(), lse.clone()]
    # an eager call first: it resolves the scratch address on this device
    hca.hca_attn_fwd_noalloc(att.plan, q, kv, kvc, scale, o, lse)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        hca.hca_attn_fwd_noalloc(att.plan, q, kv, kvc, scale, o, lse, stream=s)
    check_replays(g, (o, lse), ref)
