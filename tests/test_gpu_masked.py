"""GPU: plans whose compressed-key pattern is a given mask (the dense-mask
comparison path) or a per-query top-k selection (the CSA form), through the
C ABI, against the oracle's MASK mode on every element.  The mask of the HCA
rule itself must reproduce the analytic plan's outputs bit for bit (same tile
lists, same visibility, same arithmetic)."""

import math

import numpy as np
import pytest
import torch

import block_sparse_compressed_amd as hca
import oracle
from hca_inputs import draw, random_lengths, segment_ids, starts_csr, to_host_bits

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(msg):
    print(msg, flush=True)


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    s = np.abs(want).max() if want.size else 0.0
    return float(np.abs(got - want).max() / s) if s > 0 else float(np.abs(got).max())


def as_np(t):
    return t.detach().float().cpu().numpy()


def run(att, q, kv, kvc, dout, scale, poison=True):
    o, lse = att.new_outputs()
    dq, dkv, dkvc = att.new_grads()
    if poison:
        for t in (o, lse, dq, dkv, dkvc):
            t.fill_(float("nan"))
    att.forward(q, kv, kvc, scale, o, lse)
    att.backward(q, kv, kvc, o, lse, dout, scale, grads=(dq, dkv, dkvc))
    torch.cuda.synchronize()
    return o, lse, dq, dkv, dkvc


def check_against_oracle(name, B, S, H, W, Sc, mask, lengths, plan, seed):
    D = 512
    scale = 1.0 / math.sqrt(D)
    q, kv, kvc, dout = draw(B, S, H, D, Sc, "bf16", seed, device="cuda")
    att = hca.HcaAttention(B, S, H, D, 1, W, "bf16", plan=plan)
    assert att.info.kernel_ok == 1 and att.info.comp_masked == 1
    o, lse, dq, dkv, dkvc = run(att, q, kv, kvc, dout, scale)
    prob = oracle.Problem(B, S, H, D, 1, W, Sc, scale, segment_ids(lengths, B, S), oracle.MASK,
                          "bf16", comp_mask=mask)
    ref = oracle.full(prob, *[to_host_bits(t) for t in (q, kv, kvc, dout)])
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(as_np(lse)), fin)
    errs = dict(o=rel_err(as_np(o), ref["o"]), dq=rel_err(as_np(dq), ref["dq"]),
                dkv=rel_err(as_np(dkv), ref["dkv"]), dkvc=rel_err(as_np(dkvc), ref["dkvc"]),
                lse=rel_err(as_np(lse)[fin], ref["lse"][fin]))
    say(f"{name}: errors {errs}")
    from test_gpu_parity import record
    record(name + " (every element)", errs)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    for t in (o, dq, dkv, dkvc):
        assert not torch.isnan(t).any()


@pytest.mark.parametrize("density", [0.05, 0.5])
def test_random_mask_every_element(density):
    rng = np.random.default_rng(int(density * 1000))
    B, S, H, W, Sc = 1, 523, 64, 96, 150
    lengths = [random_lengths(rng, S, 60, 300)]
    mask = (rng.random((B, S, Sc)) < density).astype(np.uint8)
    starts, counts = starts_csr(lengths, B)
    plan = hca.hca_block_mask_build_masked(B, S, W, Sc, mask, starts, counts, H=H, D=512)
    check_against_oracle(f"masked_d{density}", B, S, H, W, Sc, mask, lengths, plan, seed=41)


def test_topk_selection_every_element():
    """CSA form: compress ratio 4 (S_c = S / 4), 48 selected entries per query
    among those completed before it, plus a 128-key raw window."""
    rng = np.random.default_rng(7)
    B, S, H, W, K = 2, 1030, 16, 128, 48
    Sc = S // 4
    idx = np.full((B, S, K), -1, np.int32)
    for b in range(B):
        for i in range(S):
            done = (i + 1) // 4  # entries completed at or before i
            if done:
                pick = rng.choice(done, size=min(K, done), replace=False)
                idx[b, i, :len(pick)] = pick
    mask = oracle.topk_mask(B, S, Sc, idx)
    plan = hca.hca_block_mask_build_topk(B, S, W, Sc, idx, H=H, D=512)
    check_against_oracle("topk_r4_k48", B, S, H, W, Sc, mask, None, plan, seed=42)


def test_hca_pattern_as_mask_matches_analytic_plan_bitwise():
    B, S, H, r, W = 1, 2100, 64, 32, 128
    lengths = [[900, 1200]]
    starts, counts = starts_csr(lengths, B)
    strict = oracle.Problem(B, S, H, 512, r, W, S // r, 0.1, segment_ids(lengths, B, S))
    Sc = S // r
    mask = np.zeros((B, S, Sc), np.uint8)
    for i in range(S):
        for c in range(Sc):
            mask[0, i, c] = oracle.vis_comp(strict, 0, i, c)
    scale = 1.0 / math.sqrt(512)
    q, kv, kvc, dout = draw(B, S, H, 512, Sc, "bf16", 43, device="cuda")
    analytic = hca.HcaAttention(B, S, H, 512, r, W, "bf16", starts, counts)
    masked = hca.HcaAttention(B, S, H, 512, r, W, "bf16", plan=hca.hca_block_mask_build_masked(
        B, S, W, Sc, mask, starts, counts, H=H, D=512))
    a = run(analytic, q, kv, kvc, dout, scale)
    m = run(masked, q, kv, kvc, dout, scale)
    for x, y in zip(a, m):
        bits = (lambda t: t.view(torch.int16)) if x.dtype == torch.bfloat16 else (lambda t: t)
        assert torch.equal(bits(x), bits(y))
