"""Block table and per-position intervals of the planner vs the oracle's element predicate.

The planner (libhca.so, host code) builds the table analytically from
intervals; the oracle classifies tiles by brute force over every element.  The
two must agree bit for bit.  Runs on the CPU (no GPU call is made).
"""

import itertools
import math

import numpy as np
import pytest

import block_sparse_compressed_amd as hca
import oracle
from hca_inputs import WORKLOADS, doc_lengths, random_lengths, segment_ids, starts_csr


def build_both(B, S, H, D, r, W, lengths, mode, tiles=None, dtype=hca.HCA_BF16):
    starts, counts = starts_csr(lengths, B)
    plan = hca.hca_block_mask_build(B, S, r, W, S // r, starts, counts, H, D, dtype, mode,
                                    tiles)
    seg = segment_ids(lengths, B, S)
    prob = oracle.Problem(B, S, H, D, r, W, S // r, 1.0 / math.sqrt(D), seg,
                          oracle.STRICT if mode == hca.HCA_COMPSEG_STRICT else oracle.LAST)
    return plan, prob


def check_full_tables(plan, prob):
    info = hca.hca_plan_get_info(plan)
    raw, comp = hca.hca_plan_export_tiles(plan)
    want_raw = oracle.tile_states(prob, 0, info.bq, info.bk_raw)
    want_comp = oracle.tile_states(prob, 1, info.bq, info.bk_comp)
    assert raw.shape == want_raw.shape and comp.shape == want_comp.shape
    np.testing.assert_array_equal(raw, want_raw)
    np.testing.assert_array_equal(comp, want_comp)
    assert info.tiles_raw == int((raw > 0).sum()) and info.full_raw == int((raw == 2).sum())
    assert info.tiles_comp == int((comp > 0).sum()) and info.full_comp == int((comp == 2).sum())


def check_rows(plan, prob, positions=None):
    """Exported intervals reproduce the oracle's visible sets position by position."""
    rows = hca.hca_plan_export_rows(plan)
    B, S, W, Sc = prob.B, prob.S, prob.W, prob.Sc
    for b in range(B):
        for i in (range(S) if positions is None else positions):
            lo, clo, chi = rows[b, i]
            cand = range(max(0, i - W - 1), min(S, i + 2))
            got_raw = [t for t in cand if lo <= t <= i]
            want_raw = [t for t in cand if oracle.vis_raw(prob, b, i, t)]
            assert got_raw == want_raw, (b, i)
            want_comp = [c for c in range(Sc) if oracle.vis_comp(prob, b, i, c)]
            assert list(range(clo, chi)) == want_comp, (b, i)


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_workload_tables_bit_exact(wid):
    wl = WORKLOADS[wid]
    dtype = hca.HCA_F32 if wl.dtype == "f32" else hca.HCA_BF16
    plan, prob = build_both(wl.B, wl.S, wl.H, wl.D, wl.r, wl.W, doc_lengths(wl),
                            hca.HCA_COMPSEG_STRICT, dtype=dtype)
    check_full_tables(plan, prob)
    info = hca.hca_plan_get_info(plan)
    assert info.kernel_ok == 1
    if wid <= 2:
        assert info.pairs_raw == oracle.count_pairs(prob, 0)
        assert info.pairs_comp == oracle.count_pairs(prob, 1)


@pytest.mark.parametrize("wid", [4, 5])
def test_workload_tables_sampled(wid):
    """Full-size tables: every non-empty tile, the tiles around them and a random sample."""
    wl = WORKLOADS[wid]
    plan, prob = build_both(wl.B, wl.S, wl.H, wl.D, wl.r, wl.W, doc_lengths(wl),
                            hca.HCA_COMPSEG_STRICT)
    info = hca.hca_plan_get_info(plan)
    assert info.kernel_ok == 1
    raw, comp = hca.hca_plan_export_tiles(plan)
    rng = np.random.default_rng(wid)
    for kind, table, bk in [(0, raw, info.bk_raw), (1, comp, info.bk_comp)]:
        nz = np.flatnonzero(table.reshape(-1))
        nkt = table.shape[2]
        # neighbours of non-empty tiles along the key axis (band edges)
        neigh = np.concatenate([nz - 1, nz + 1])
        neigh = neigh[(neigh >= 0) & (neigh < table.size)]
        sample = rng.integers(0, table.size, size=20000)
        # every tile of a few random query tiles
        qts = rng.integers(0, info.nqt, size=8)
        rowsel = (qts[:, None] * nkt + np.arange(nkt)[None, :]).reshape(-1)
        flat = np.unique(np.concatenate([nz, neigh, sample, rowsel]))
        want = oracle.tile_states_at(prob, kind, info.bq, bk, flat)
        np.testing.assert_array_equal(table.reshape(-1)[flat], want)
    positions = sorted(set(rng.integers(0, wl.S, size=64).tolist()) | {0, wl.S - 1, wl.r - 1,
                                                                        wl.r, wl.r - 2})
    check_rows(plan, prob, positions)


def sweep_cases():
    rng = np.random.default_rng(1234)
    out = []
    tiles_list = [None, (1, 1, 1), (4, 8, 4), (16, 32, 32), (3, 5, 7)]
    for S, r, W in itertools.product([1, 2, 15, 16, 17, 31, 33, 489, 4133],
                                     [1, 3, 16, 128, 5000], [0, 1, 5, 64, 128, 10000]):
        if rng.random() > 0.22:
            continue
        B = 2 if rng.random() < 0.3 else 1
        kind = rng.integers(0, 5)
        lengths = None
        if kind == 1:  # random documents
            lengths = [random_lengths(rng, S, 1, max(1, S // 3)) for _ in range(B)]
        elif kind == 2 and S > r:  # boundaries on multiples of r
            lengths = [[L for L in np.diff(sorted({0, S} | set(range(0, S, r * 2)))).tolist()]
                       for _ in range(B)]
        elif kind == 3:  # boundaries on tile edges (16)
            lengths = [[L for L in np.diff(sorted({0, S} | set(range(0, S, 16)))).tolist()]
                       for _ in range(B)]
        elif kind == 4:  # many length-1 documents then one long one
            lengths = [[1] * min(S - 1, 5) + ([S - min(S - 1, 5)] if S > 1 else [])
                       for _ in range(B)]
            lengths = [[L for L in ls if L > 0] for ls in lengths]
        tiles = tiles_list[rng.integers(0, len(tiles_list))]
        mode = int(rng.integers(0, 2))
        H = int(rng.choice([1, 4, 16, 64]))
        out.append((B, S, H, r, W, lengths, mode, tiles))
    return out


@pytest.mark.parametrize("case", sweep_cases(), ids=lambda c: "B%dS%dH%dr%dW%d" % c[:5])
def test_sweep_bit_exact(case):
    B, S, H, r, W, lengths, mode, tiles = case
    plan, prob = build_both(B, S, H, 128, r, W, lengths, mode, tiles)
    check_full_tables(plan, prob)
    if S <= 600:
        check_rows(plan, prob)
        info = hca.hca_plan_get_info(plan)
        assert info.pairs_raw == oracle.count_pairs(prob, 0)
        assert info.pairs_comp == oracle.count_pairs(prob, 1)


def test_unaligned_lengths_cover_padding_branches():
    """S = 489 with 2-, 16- and 32-wide tiles: padded rows and keys are never FULL."""
    for tiles in [(2, 32, 32), (16, 32, 32), (32, 16, 8)]:
        plan, prob = build_both(1, 489, 4, 64, 16, 64, None, hca.HCA_COMPSEG_STRICT, tiles)
        check_full_tables(plan, prob)
        raw, comp = hca.hca_plan_export_tiles(plan)
        info = hca.hca_plan_get_info(plan)
        last_q = raw[0, info.nqt - 1]
        if 489 % info.bq:
            assert not (last_q == hca.HCA_TILE_FULL).any()
        if 489 % info.bk_raw:
            assert not (raw[0, :, info.nkt_raw - 1] == hca.HCA_TILE_FULL).any()


def test_schedule_is_consistent():
    """Query-tile lists and key-tile work items cover the same non-empty tiles."""
    wl = WORKLOADS[2]
    lengths = doc_lengths(wl)
    starts, counts = starts_csr(lengths, wl.B)
    plan = hca.hca_block_mask_build(wl.B, wl.S, wl.r, wl.W, wl.Sc, starts, counts, wl.H, wl.D,
                                    hca.HCA_BF16, hca.HCA_COMPSEG_STRICT)
    info = hca.hca_plan_get_info(plan)
    # (the head dim 128 forward stages the row-major K itself: no workspace)
    assert info.device_bytes > 0 and info.ws_bwd_bytes > 0 and info.ws_fwd_bytes == 0
    # no device buffer is O(S^2): the plan image is linear in S
    assert info.device_bytes < 64 * wl.B * wl.S + 16 * (info.tiles_raw + info.tiles_comp) + 8192


# --------------------------------------------------------------------------- #
# key-stationary work items: visible halves and partial blocks
# --------------------------------------------------------------------------- #

def closed_form_intervals(S, r, W, lengths_row):
    """Visible raw keys [lo, i] and entries [clo, chi) per position, written from
    the definitions (contiguous documents, STRICT entries)."""
    start = np.zeros(S, np.int64)
    pos = 0
    for L in (lengths_row or [S]):
        start[pos:pos + L] = pos
        pos += L
    i = np.arange(S, dtype=np.int64)
    lo = np.maximum(i - W + 1, start)
    chi = (i + 1) // r
    clo = np.minimum(-(-start // r), chi)
    return lo, i + 1, clo, chi  # raw [lo, hi), comp [clo, chi)


@pytest.mark.parametrize("lengths", [None, [[15000, 25000]]], ids=["one_doc", "two_docs"])
def test_items_halves_and_partial_blocks(lengths):
    """At S = 40000, H = 64, D = 512 with 128-key tiles and half-tile marking
    on (the knob sets the threshold to one item), the planner marks items that see only
    one 64-key half of their tile.  Every item's mark must equal the halves
    that its query tiles see, and the items of a key tile must own
    consecutive partial blocks (the reduction relies on it)."""
    S, H, D, r, W = 40000, 64, 512, 128, 128
    plan, prob = build_both(1, S, H, D, r, W, lengths, hca.HCA_COMPSEG_STRICT,
                            tiles=(0, 0, 0, 1, 0, 128))
    info = hca.hca_plan_get_info(plan)
    items = hca.hca_plan_export_items(plan)
    assert len(items) >= 1000 and (items[:, 3] == 128).all()
    lo, hi, clo, chi = closed_form_intervals(S, r, W, lengths[0] if lengths else None)
    n_half = 0
    for b, kind, k0, nk, qa, qz, hmark, _ in items:
        halves = hmark & 3
        p = np.arange(qa * info.bq, min(S, (qz + 1) * info.bq))
        a, z = (clo[p], chi[p]) if kind else (lo[p], hi[p])
        nkeys = info.S_c if kind else S
        mid, end = min(k0 + nk // 2, nkeys), min(k0 + nk, nkeys)
        want = int((np.maximum(a, k0) < np.minimum(z, mid)).any()) | \
            (int((np.maximum(a, mid) < np.minimum(z, end)).any()) << 1)
        assert want != 0
        assert halves == (3 if want == 3 else want), (kind, k0, qa, qz, halves, want)
        n_half += halves != 3
    assert n_half > 0  # first and last items of sliding-window tiles
    # spot-check marked items against the oracle's element predicate
    rng = np.random.default_rng(0)
    half_items = items[(items[:, 6] & 3) != 3]
    for row in half_items[rng.choice(len(half_items), size=12, replace=False)]:
        b, kind, k0, nk, qa, qz, halves, _ = (int(x) for x in row)
        halves &= 3
        idle = range(k0 + nk // 2, k0 + nk) if halves == 1 else range(k0, k0 + nk // 2)
        vis = oracle.vis_comp if kind else oracle.vis_raw
        nkeys = info.S_c if kind else S
        for i in range(qa * info.bq, min(S, (qz + 1) * info.bq)):
            assert not any(vis(prob, b, i, t) for t in idle if t < nkeys)
    check_partial_blocks(items, D, info)


def check_partial_blocks(items, D, info):
    """Each key tile's items are consecutive and own consecutive partial blocks
    (the reduction sums a tile's blocks by position); a block is owned by one
    item, or shared by exactly one lower-half and one upper-half item of the
    tile, both marked shared; the tiles' block ranges tile [0, part_blocks)."""
    blk = items[0, 3] * D
    tiles = {}
    for row in items:
        key = (int(row[0]), int(row[1]), int(row[2]))
        assert not tiles or key in tiles or key > max(tiles), "items of a tile are consecutive"
        tiles.setdefault(key, []).append(row)
    covered = []
    for key, rows in tiles.items():
        offs = {}
        for row in rows:
            assert row[7] % blk == 0
            offs.setdefault(int(row[7]) // blk, []).append(int(row[6]))
        ids = sorted(offs)
        assert ids == list(range(ids[0], ids[0] + len(ids))), key
        covered += ids
        for owners in offs.values():
            if len(owners) == 1:
                assert owners[0] & 4 == 0
            else:
                assert sorted(owners) == [1 | 4, 2 | 4], owners
    assert sorted(covered) == list(range(info.part_blocks))


def test_items_half_tiles_marked_at_any_size():
    """With 128-key tiles the one-launch key-stationary kernel runs half-tile
    items beside the full ones, so the planner marks them at any size
    (S = 16384 here), and lower/upper pairs share partial blocks."""
    plan, _ = build_both(1, 16384, 64, 512, 128, 128, None, hca.HCA_COMPSEG_STRICT,
                         tiles=(0, 0, 0, 0, 0, 128))
    items = hca.hca_plan_export_items(plan)
    info = hca.hca_plan_get_info(plan)
    assert info.items == len(items) and info.items_half > 0
    assert info.part_blocks < len(items)
    check_partial_blocks(items, 512, info)


def test_half_items_knob():
    """With 128-key tiles, half_items_min = 1 marks half-tile items on a small problem (so the GPU
    tests can run that kernel at sizes the oracle checks element by element);
    half_items_min < 0 never marks them."""
    S, H, D, r, W = 1536, 8, 512, 16, 128
    plan, prob = build_both(1, S, H, D, r, W, None, hca.HCA_COMPSEG_STRICT,
                            tiles=(0, 0, 0, 1, 0, 128))
    info = hca.hca_plan_get_info(plan)
    items = hca.hca_plan_export_items(plan)
    half = (items[:, 6] & 3) != 3
    assert info.items_half == int(half.sum()) > 0
    assert ((items[:, 6] & 3) == 1).any() and ((items[:, 6] & 3) == 2).any()
    assert (items[:, 6] & 4).any()  # some lower/upper pairs share a block
    check_partial_blocks(items, D, info)
    assert info.part_blocks < len(items)
    # every marked item's idle half is invisible to all of its rows
    for row in items[half]:
        b, kind, k0, nk, qa, qz, halves, _ = (int(x) for x in row)
        idle = range(k0 + 64, k0 + 128) if halves & 3 == 1 else range(k0, k0 + 64)
        vis = oracle.vis_comp if kind else oracle.vis_raw
        nkeys = info.S_c if kind else S
        for i in range(qa * info.bq, min(S, (qz + 1) * info.bq)):
            assert not any(vis(prob, b, i, t) for t in idle if t < nkeys)
    plan2, _ = build_both(1, S, H, D, r, W, None, hca.HCA_COMPSEG_STRICT,
                          tiles=(0, 0, 0, -1, 0, 128))
    assert hca.hca_plan_get_info(plan2).items_half == 0
    assert (hca.hca_plan_export_items(plan2)[:, 6] == 3).all()


def test_kv_keys_choice():
    """Key tile width of the key-stationary backward: 64 keys at D = 512 (plans
    from the rule or from a given mask), 32 at other head dims; kv_keys
    overrides it where a kernel of that width exists.  64-key items always run
    over their whole tile (no half marks), and their partial blocks are
    64 x D."""
    S, H, r, W = 1536, 8, 16, 128
    rule, prob = build_both(1, S, H, 512, r, W, None, hca.HCA_COMPSEG_STRICT)
    info = hca.hca_plan_get_info(rule)
    items = hca.hca_plan_export_items(rule)
    assert info.kv_keys == 64 and (items[:, 3] == 64).all()
    assert info.items_half == 0 and (items[:, 6] == 3).all()
    assert info.part_blocks == len(items)
    check_partial_blocks(items, 512, info)
    # every visible key of the problem lies in some item's tile and query tiles
    covered = set()
    for b, kind, k0, nk, qa, qz, _, _ in items:
        covered.add((int(kind), int(k0) // 64, int(qa), int(qz)))
    for i in range(0, S, 97):
        qt = i // info.bq
        for t in range(S):
            if oracle.vis_raw(prob, 0, i, t):
                assert any(k == 0 and kt == t // 64 and qa <= qt <= qz
                           for k, kt, qa, qz in covered), (i, t)
    mask = np.zeros((1, S, S // r), np.uint8)
    mask[0, :, ::3] = 1
    masked = hca.hca_block_mask_build_masked(1, S, W, S // r, mask, None, None, H, 512,
                                             hca.HCA_BF16)
    assert hca.hca_plan_get_info(masked).kv_keys == 64
    masked128 = hca.hca_block_mask_build_masked(1, S, W, S // r, mask, None, None, H, 512,
                                                hca.HCA_BF16, tiles=(0, 0, 0, 0, 0, 128))
    info128 = hca.hca_plan_get_info(masked128)
    assert info128.kv_keys == 128 and info128.ws_pds_bytes == 0
    d128 = hca.hca_block_mask_build(1, S, r, W, S // r, None, None, H, 128, hca.HCA_BF16)
    assert hca.hca_plan_get_info(d128).kv_keys == 32
    # the library's 64-key choice stores P / dS only while that takes <= 32 GiB
    big = hca.hca_plan_get_info(hca.hca_block_mask_build(1, 262144, 128, 128, 2048, None, None,
                                                         64, 512, hca.HCA_BF16))
    assert big.kv_keys == 128 and big.ws_pds_bytes == 0
    forced = hca.hca_plan_get_info(hca.hca_block_mask_build(
        1, 262144, 128, 128, 2048, None, None, 64, 512, hca.HCA_BF16, tiles=(0, 0, 0, 0, 0, 64)))
    assert forced.kv_keys == 64 and forced.ws_pds_bytes > 32 * 2**30
    # stored P / dS keeps compressed items one chunk long (their partial sums
    # grow no faster than the store), also where every query tile lists every
    # compressed tile (top-k selections); the recomputing backward merges runs
    rng = np.random.default_rng(5)
    Sq, Sc = 16384, 4096
    idx = rng.integers(0, Sc, size=(1, Sq, 32)).astype(np.int32)
    tk = hca.hca_plan_get_info(hca.hca_block_mask_build_topk(1, Sq, 128, Sc, idx, H=8, D=512))
    assert tk.kv_keys == 64 and tk.comp_item_chunks == 1
    tk128 = hca.hca_plan_get_info(hca.hca_block_mask_build_topk(
        1, Sq, 128, Sc, idx, H=8, D=512, tiles=(0, 0, 0, 0, 0, 128)))
    assert tk128.kv_keys == 128 and tk128.comp_item_chunks > 1
    for D, bad in ((512, 32), (512, 96), (512, 256), (128, 64), (64, 128)):
        with pytest.raises(hca.HcaError, match="kv_keys"):
            hca.hca_block_mask_build(1, S, r, W, S // r, None, None, H, D, hca.HCA_BF16,
                                     tiles=(0, 0, 0, 0, 0, bad))


@pytest.mark.parametrize("chunks", [1, 3, 20])
def test_compressed_item_chunks_knob(chunks):
    """comp_item_chunks sets the 64-position chunks per compressed-tile item:
    the items of a compressed tile cover its list in runs on one global grid of
    `chunks` chunks; raw-tile items stay one chunk long."""
    S, H, D, r, W = 6000, 8, 512, 4, 64
    plan, _ = build_both(1, S, H, D, r, W, [[2500, 3500]], hca.HCA_COMPSEG_STRICT,
                         tiles=(0, 0, 0, 0, chunks))
    info = hca.hca_plan_get_info(plan)
    assert info.comp_item_chunks == chunks
    items = hca.hca_plan_export_items(plan)
    per_chunk = 64 // info.bq
    for b, kind, k0, nk, qa, qz, _, _ in items:
        run = per_chunk * (chunks if kind else 1)
        assert qa // run == qz // run, (kind, qa, qz)
    comp = items[items[:, 1] == 1]
    longest = int((comp[:, 5] - comp[:, 4]).max()) + 1
    assert longest <= per_chunk * chunks
    if chunks == 20:
        assert longest > 64  # lists past 64 entries (read beyond the lane-held part)
    check_partial_blocks(items, D, info)


def test_workspace_grows_linearly():
    """Without stored P and dS (128-key tiles) the backward workspace is O(S):
    compressed-tile items are merged once their partial blocks would pass
    twice the raw tiles' (which grow as S), so doubling S at most about doubles
    it (it grew as S^2 / r when every 64-position chunk of a compressed tile's
    rows was always an item).  With 64-key tiles the workspace adds the stored
    P and dS: exactly one 2 x (bq H) x 32 bf16 block per listed (query tile,
    32-key tile) pair, O(visible pairs)."""
    lean = (0, 0, 0, 0, 0, 128)
    ws = {}
    for S in (131072, 262144):
        p = hca.hca_block_mask_build(1, S, 128, 128, S // 128, None, None, 64, 512,
                                     hca.HCA_BF16, tiles=lean)
        info = hca.hca_plan_get_info(p)
        assert info.ws_pds_bytes == 0
        ws[S] = info.ws_bwd_bytes
    assert ws[262144] <= 2.05 * ws[131072]
    # S = 65536 keeps one-chunk compressed items (its compressed partials fit
    # in twice the raw ones) and needs less than before (1.27 GiB)
    p = hca.hca_block_mask_build(1, 65536, 128, 128, 512, None, None, 64, 512, hca.HCA_BF16,
                                 tiles=lean)
    info = hca.hca_plan_get_info(p)
    assert info.comp_item_chunks == 1 and info.ws_bwd_bytes < 1.2 * 2**30
    # stored P / dS: the listed pairs times one block each
    p = hca.hca_block_mask_build(1, 16384, 128, 128, 128, None, None, 64, 512, hca.HCA_BF16)
    info = hca.hca_plan_get_info(p)
    raw, comp = hca.hca_plan_export_tiles(p)
    listed = int((raw > 0).sum() + (comp > 0).sum())
    assert info.kv_keys == 64
    assert info.ws_pds_bytes == listed * 2 * info.bq * info.H * 32 * 2
    assert info.ws_bwd_bytes > info.ws_pds_bytes
