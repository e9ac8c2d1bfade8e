"""Plans with a given compressed-key mask (the dense-mask form of the
compressed pattern, and per-query top-k selections) against the oracle's
brute-force classifier in MASK mode, on the CPU (no GPU call).

The tile tables must match the element predicate bit for bit; the pair counts
must equal the mask's ones plus the window's pairs; a top-k plan must equal the
masked plan of its selection's mask; and the mask of the HCA pattern itself
must give the analytic plan's tables.
"""

import math

import numpy as np
import pytest

import block_sparse_compressed_amd as hca
import oracle
from hca_inputs import random_lengths, segment_ids, starts_csr


def masked_pair(B, S, H, W, Sc, mask, lengths=None):
    starts, counts = starts_csr(lengths, B)
    plan = hca.hca_block_mask_build_masked(B, S, W, Sc, mask, starts, counts, H=H, D=512)
    prob = oracle.Problem(B, S, H, 512, 1, W, Sc, 1.0 / math.sqrt(512),
                          segment_ids(lengths, B, S), oracle.MASK, comp_mask=mask)
    return plan, prob


def check_tables(plan, prob):
    info = hca.hca_plan_get_info(plan)
    raw, comp = hca.hca_plan_export_tiles(plan)
    np.testing.assert_array_equal(raw, oracle.tile_states(prob, 0, info.bq, info.bk_raw))
    np.testing.assert_array_equal(comp, oracle.tile_states(prob, 1, info.bq, info.bk_comp))
    assert info.pairs_raw == oracle.count_pairs(prob, 0)
    assert info.pairs_comp == oracle.count_pairs(prob, 1)


@pytest.mark.parametrize("density", [0.0, 0.02, 0.3, 1.0])
def test_random_mask_tables_bit_exact(density):
    rng = np.random.default_rng(int(density * 100))
    B, S, H, W, Sc = 2, 300, 64, 40, 77
    mask = (rng.random((B, S, Sc)) < density).astype(np.uint8)
    lengths = [random_lengths(rng, S, 20, 150) for _ in range(B)]
    plan, prob = masked_pair(B, S, H, W, Sc, mask, lengths)
    info = hca.hca_plan_get_info(plan)
    assert info.comp_masked == 1 and info.kernel_ok == 1 and info.S_c == Sc
    check_tables(plan, prob)


def test_topk_plan_equals_masked_plan_of_its_selection():
    rng = np.random.default_rng(5)
    B, S, H, W, Sc, K = 1, 257, 16, 64, 64, 9
    idx = rng.integers(-3, Sc, size=(B, S, K)).astype(np.int32)
    mask = oracle.topk_mask(B, S, Sc, idx)
    a = hca.hca_block_mask_build_topk(B, S, W, Sc, idx, H=H)
    b, prob = masked_pair(B, S, H, W, Sc, mask)
    for x, y in zip(hca.hca_plan_export_tiles(a), hca.hca_plan_export_tiles(b)):
        np.testing.assert_array_equal(x, y)
    ia, ib = hca.hca_plan_get_info(a), hca.hca_plan_get_info(b)
    assert (ia.pairs_comp, ia.items, ia.device_bytes) == (ib.pairs_comp, ib.items, ib.device_bytes)
    check_tables(a, prob)
    with pytest.raises(ValueError):
        hca.hca_block_mask_build_topk(B, S, W, Sc, np.full((B, S, K), Sc, np.int32), H=H)


def test_hca_pattern_as_a_mask_gives_the_analytic_tables():
    """The dense mask of the HCA rule itself must reproduce the analytic
    plan's tile tables and pair counts."""
    B, S, H, r, W = 1, 700, 64, 16, 64
    lengths = [[250, 450]]
    starts, counts = starts_csr(lengths, B)
    analytic = hca.hca_block_mask_build(B, S, r, W, S // r, starts, counts, H, 512)
    strict = oracle.Problem(B, S, H, 512, r, W, S // r, 0.1, segment_ids(lengths, B, S))
    mask = np.array([[[oracle.vis_comp(strict, 0, i, c) for c in range(S // r)]
                      for i in range(S)]], np.uint8)
    masked = hca.hca_block_mask_build_masked(B, S, W, S // r, mask, starts, counts, H=H)
    for x, y in zip(hca.hca_plan_export_tiles(analytic), hca.hca_plan_export_tiles(masked)):
        np.testing.assert_array_equal(x, y)
    ia, im = hca.hca_plan_get_info(analytic), hca.hca_plan_get_info(masked)
    assert (ia.pairs_raw, ia.pairs_comp) == (im.pairs_raw, im.pairs_comp)
    assert im.device_bytes > ia.device_bytes  # the mask bits travel with the plan


def test_masked_plan_needs_the_d512_kernels():
    mask = np.ones((1, 64, 8), np.uint8)
    for D, dt in ((128, hca.HCA_BF16), (64, hca.HCA_F32)):
        p = hca.hca_block_mask_build_masked(1, 64, 8, 8, mask, H=16, D=D, dtype=dt)
        assert hca.hca_plan_get_info(p).kernel_ok == 0
    with pytest.raises(ValueError):
        hca.hca_block_mask_build_masked(1, 64, 8, 8, np.ones((1, 64, 7), np.uint8), H=16)
