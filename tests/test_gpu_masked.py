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


@pytest.mark.parametrize("density,kv_keys", [(0.05, 0), (0.5, 0), (0.05, 128)])
def test_random_mask_every_element(density, kv_keys):
    """Random masks over ragged documents; the library's choice stores P and dS
    (64-key tiles), kv_keys = 128 runs the recomputing 128-key backward with
    the mask bits."""
    rng = np.random.default_rng(int(density * 1000))
    B, S, H, W, Sc = 1, 523, 64, 96, 150
    lengths = [random_lengths(rng, S, 60, 300)]
    mask = (rng.random((B, S, Sc)) < density).astype(np.uint8)
    starts, counts = starts_csr(lengths, B)
    plan = hca.hca_block_mask_build_masked(B, S, W, Sc, mask, starts, counts, H=H, D=512,
                                           tiles=(0, 0, 0, 0, 0, kv_keys))
    assert hca.hca_plan_get_info(plan).kv_keys == (kv_keys or 64)
    check_against_oracle(f"masked_d{density}_k{kv_keys or 64}", B, S, H, W, Sc, mask, lengths,
                         plan, seed=41)


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


@pytest.mark.parametrize("kv_keys", [64, 128])
def test_hca_pattern_as_mask_matches_analytic_plan_bitwise(kv_keys):
    """Both plans at the same key tile width, so the key-stationary items, and
    with them the summation order, are the same."""
    B, S, H, r, W = 1, 2100, 64, 32, 128
    tiles = (0, 0, 0, 0, 0, kv_keys)
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
    analytic = hca.HcaAttention(B, S, H, 512, r, W, "bf16", plan=hca.hca_block_mask_build(
        B, S, r, W, Sc, starts, counts, H, 512, hca.HCA_BF16, tiles=tiles))
    masked = hca.HcaAttention(B, S, H, 512, r, W, "bf16", plan=hca.hca_block_mask_build_masked(
        B, S, W, Sc, mask, starts, counts, H=H, D=512, tiles=tiles))
    ia, im = hca.hca_plan_export_items(analytic.plan), hca.hca_plan_export_items(masked.plan)
    assert np.array_equal(ia, im) and analytic.info.kv_keys == kv_keys
    a = run(analytic, q, kv, kvc, dout, scale)
    m = run(masked, q, kv, kvc, dout, scale)
    for x, y in zip(a, m):
        bits = (lambda t: t.view(torch.int16)) if x.dtype == torch.bfloat16 else (lambda t: t)
        assert torch.equal(bits(x), bits(y))


def test_csa_topk_workload_full_size_sampled():
    """The CSA-form workload the benchmark times (S = 16384, H = 64, D = 512,
    compress ratio 4, 512 selected entries per query, W = 128), NaN-poisoned
    outputs all written; sampled rows and two whole query tiles of 16
    positions over all heads, every raw key of one 128-key tile, and two
    compressed entries compared with the oracle's MASK mode."""
    from hca_inputs import CSA_TOPK, CSA_TOPK_K, draw_workload, topk_indices

    wl = CSA_TOPK
    idx = topk_indices(wl, CSA_TOPK_K)
    plan = hca.hca_block_mask_build_topk(wl.B, wl.S, wl.W, wl.Sc, idx, H=wl.H, D=wl.D)
    att = hca.HcaAttention(wl.B, wl.S, wl.H, wl.D, wl.r, wl.W, "bf16", plan=plan)
    q, kv, kvc, dout = draw_workload(wl, device="cuda")
    scale = 1.0 / math.sqrt(wl.D)
    o, lse, dq, dkv, dkvc = run(att, q, kv, kvc, dout, scale)
    for t in (o, dq, dkv, dkvc):
        assert not torch.isnan(t).any()
    say("  GPU pass done")
    mask = oracle.topk_mask(wl.B, wl.S, wl.Sc, idx)
    prob = oracle.Problem(wl.B, wl.S, wl.H, wl.D, wl.r, wl.W, wl.Sc, scale, None, oracle.MASK,
                          "bf16", comp_mask=mask)
    host = [to_host_bits(t) for t in (q, kv, kvc, dout)]
    rng = np.random.default_rng(6)
    rows = rng.integers(0, wl.H * wl.S, size=64)
    for qt in (3, wl.S // 16 - 1):
        pos = np.arange(qt * 16, qt * 16 + 16)
        rows = np.concatenate([rows, (np.arange(wl.H)[:, None] * wl.S + pos[None, :]).ravel()])
    rows = np.unique(rows)
    ro, rlse, _, rdq = oracle.rows(prob, *host, row_index=rows)
    flat = lambda t: t.reshape(-1, wl.D) if t.dim() == 4 else t.reshape(-1)
    ix = torch.as_tensor(rows, device="cuda")
    e = dict(o=rel_err(as_np(flat(o)[ix]), ro), dq=rel_err(as_np(flat(dq)[ix]), rdq),
             lse=rel_err(as_np(flat(lse)[ix]), rlse))
    # raw keys 8192 .. 8319: rows of positions 8192 .. 8446, all heads
    k0 = 8192
    pos = np.arange(k0, k0 + 128 + wl.W - 1)
    krows = (np.arange(wl.H)[:, None] * wl.S + pos[None, :]).ravel()
    _, klse, kdelta, _ = oracle.rows(prob, *host, row_index=krows)
    lse_all = np.full(wl.H * wl.S, np.nan)
    delta_all = np.full(wl.H * wl.S, np.nan)
    lse_all[krows], delta_all[krows] = klse, kdelta
    kidx = np.arange(k0, k0 + 128, dtype=np.int32)
    rk = oracle.keys(prob, *host, np.zeros_like(kidx), np.zeros_like(kidx), kidx, lse_all,
                     delta_all)
    e["dkv_tile"] = rel_err(as_np(dkv[0, k0:k0 + 128]), rk)
    # compressed entries selected by late queries only (one to a few hundred
    # positions see them, so the oracle recomputes their rows quickly)
    cidx = np.array([wl.Sc - 3, wl.Sc - 40, wl.Sc - 600], np.int32)
    rc = oracle.keys(prob, *host, np.ones_like(cidx), np.zeros_like(cidx), cidx)
    e["dkvc_entries"] = rel_err(np.stack([as_np(dkvc[0, c]) for c in cidx]), rc)
    say(f"  csa_topk sampled errors {e}")
    from test_gpu_parity import record
    record("csa_topk_bf16 (sampled)", e)
    for k, v in e.items():
        assert v <= TOL, (k, v)
