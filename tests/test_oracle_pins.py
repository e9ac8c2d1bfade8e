"""Pins for the CPU oracle: each test checks it against something other than itself.

Pins used (none re-types the oracle's own arithmetic):
  * hand-derived visible sets for a tiny problem (tests/golden/);
  * reduction to plain causal attention (torch SDPA, fp64) when the window
    covers the whole document and there are no compressed entries;
  * reduction of the compressed path to causal attention when r = 1 and the
    compressed entries equal the raw keys;
  * closed forms: Q = 0 (uniform weights), constant values (rows of P sum to 1),
    W = 1 (single visible key), duplicated keys (LSE shifts by ln 2);
  * the backward against fp64 central finite differences of sum(O * dO);
  * the identity delta_i = <dO_i, O_i>;
  * several key/value heads: the grouped form reduces to causal attention over
    each group's head (torch SDPA with repeat_interleave, fp64, autograd);
  * compressed visibility from a given dense mask (random, or a top-k index
    selection): attention with the explicit boolean mask over the
    concatenated keys (torch, fp64, autograd);
  * visible-pair counts against their closed forms.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
from hca_inputs import segment_ids

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, *shape):
    return rng.standard_normal(shape).astype(np.float64)


def make_problem(B, S, H, D, r, W, lengths=None, mode=oracle.STRICT, scale=None, Sc=None):
    seg = segment_ids(lengths, B, S)
    if Sc is None:
        Sc = S // r
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return oracle.Problem(B, S, H, D, r, W, Sc, scale, seg, mode, "f64")


# --------------------------------------------------------------------------- #
# hand-derived visible sets
# --------------------------------------------------------------------------- #

def read_golden(name):
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if "|" not in line:
                k, *v = line.split()
                meta[k] = [int(x) for x in v]
                continue
            cols = [c.strip() for c in line.split("|")]
            parse = lambda c: [] if c == "-" else [int(x) for x in c.split()]
            rows.append((int(cols[0]), parse(cols[1]), parse(cols[2]), parse(cols[3])))
    return meta, rows


@pytest.mark.parametrize("mode", [oracle.STRICT, oracle.LAST])
def test_golden_visible_sets(mode):
    meta, rows = read_golden("visible_sets_s12_r3_w2.txt")
    S, r, W = meta["S"][0], meta["r"][0], meta["W"][0]
    starts = meta["starts"] + [S]
    lengths = [[starts[j + 1] - starts[j] for j in range(len(starts) - 1)]]
    p = make_problem(1, S, 1, 4, r, W, lengths, mode)
    for i, raw, strict, last in rows:
        got_raw = [t for t in range(S) if oracle.vis_raw(p, 0, i, t)]
        got_comp = [c for c in range(S // r) if oracle.vis_comp(p, 0, i, c)]
        assert got_raw == raw, (i, got_raw, raw)
        assert got_comp == (strict if mode == oracle.STRICT else last), (i, got_comp)


@pytest.mark.parametrize("mode", [oracle.STRICT, oracle.LAST])
def test_tile_states_match_golden_sets(mode):
    """Tile states from the hand-derived sets, classified by hand-written loops."""
    meta, rows = read_golden("visible_sets_s12_r3_w2.txt")
    S, r, W = meta["S"][0], meta["r"][0], meta["W"][0]
    starts = meta["starts"] + [S]
    lengths = [[starts[j + 1] - starts[j] for j in range(len(starts) - 1)]]
    p = make_problem(1, S, 1, 4, r, W, lengths, mode)
    vis_raw = np.zeros((S, S), bool)
    vis_comp = np.zeros((S, S // r), bool)
    for i, raw, strict, last in rows:
        vis_raw[i, raw] = True
        vis_comp[i, strict if mode == oracle.STRICT else last] = True
    for bq, bk, bkc in [(4, 2, 2), (5, 3, 3), (1, 1, 1), (12, 12, 4), (7, 5, 3)]:
        for kind, vis, n, tb in [(0, vis_raw, S, bk), (1, vis_comp, S // r, bkc)]:
            got = oracle.tile_states(p, kind, bq, tb)[0]
            nqt, nkt = -(-S // bq), -(-n // tb)
            for qt in range(nqt):
                for kt in range(nkt):
                    block = vis[qt * bq:(qt + 1) * bq, kt * tb:(kt + 1) * tb]
                    nominal = block.shape == (bq, tb)
                    want = 0 if not block.any() else (2 if nominal and block.all() else 1)
                    assert got[qt, kt] == want, (kind, bq, tb, qt, kt)


# --------------------------------------------------------------------------- #
# reductions to causal attention (torch SDPA in fp64)
# --------------------------------------------------------------------------- #

def causal_reference(q, k, scale, dout):
    """Per-document-free causal attention: O, LSE, dQ, dK (k used as key and value)."""
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    H = q.shape[0]
    kk = kt.unsqueeze(0).expand(H, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kk, kk, is_causal=True, scale=scale)
    o.backward(torch.tensor(dout))
    logits = (qt.detach() @ kt.detach().T) * scale
    causal = torch.ones(q.shape[1], q.shape[1], dtype=torch.bool).tril()
    lse = torch.logsumexp(logits.masked_fill(~causal, -math.inf), dim=-1)
    return o.detach().numpy(), lse.numpy(), qt.grad.numpy(), kt.grad.numpy()


def per_document_causal(q, kv, scale, dout, lengths):
    """Runs causal attention separately inside each document of each batch row."""
    B, H, S, D = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, H, S))
    dq = np.zeros_like(q)
    dkv = np.zeros_like(kv)
    for b in range(B):
        pos = 0
        for L in (lengths[b] if lengths else [S]):
            sl = slice(pos, pos + L)
            ro, rl, rdq, rdk = causal_reference(q[b][:, sl], kv[b][sl], scale, dout[b][:, sl])
            o[b][:, sl], lse[b][:, sl], dq[b][:, sl], dkv[b][sl] = ro, rl, rdq, rdk
            pos += L
    return o, lse, dq, dkv


CASES = [
    (1, 37, 3, 8, None),
    (2, 29, 2, 16, [[10, 19], [1, 5, 23]]),
    (1, 33, 4, 4, [[1, 1, 31]]),
]


@pytest.mark.parametrize("B,S,H,D,lengths", CASES)
def test_raw_path_reduces_to_causal(B, S, H, D, lengths):
    rng = np.random.default_rng(11)
    q, kv, dout = rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, H, S, D)
    p = make_problem(B, S, H, D, r=S + 1, W=S, lengths=lengths)
    assert p.Sc == 0
    got = oracle.full(p, q, kv, np.zeros((B, 0, D)), dout)
    o, lse, dq, dkv = per_document_causal(q, kv, p.scale, dout, lengths)
    np.testing.assert_allclose(got["o"], o, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(got["lse"], lse, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(got["dq"], dq, atol=1e-11, rtol=1e-9)
    np.testing.assert_allclose(got["dkv"], dkv, atol=1e-11, rtol=1e-9)


@pytest.mark.parametrize("mode", [oracle.STRICT, oracle.LAST])
@pytest.mark.parametrize("B,S,H,D,lengths", CASES)
def test_compressed_path_reduces_to_causal(B, S, H, D, lengths, mode):
    """r = 1, W = 0, kv_comp = kv: entry c is raw position c, complete for i >= c."""
    rng = np.random.default_rng(12)
    q, kv, dout = rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, H, S, D)
    p = make_problem(B, S, H, D, r=1, W=0, lengths=lengths, mode=mode)
    assert p.Sc == S
    got = oracle.full(p, q, kv, kv.copy(), dout)
    o, lse, dq, dkv = per_document_causal(q, kv, p.scale, dout, lengths)
    np.testing.assert_allclose(got["o"], o, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(got["lse"], lse, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(got["dq"], dq, atol=1e-11, rtol=1e-9)
    np.testing.assert_allclose(got["dkvc"], dkv, atol=1e-11, rtol=1e-9)
    assert np.all(got["dkv"] == 0.0)


def causal_reference_grouped(q, kv, scale, dout):
    """Causal attention of query heads q [H, S, D] over key/value heads kv [G, S, D],
    head h reading kv[h // (H // G)] (torch repeat_interleave), in fp64 with
    autograd: O, LSE, dQ, dKV [G, S, D]."""
    H, G = q.shape[0], kv.shape[0]
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(kv, requires_grad=True)
    kk = kt.repeat_interleave(H // G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kk, kk, is_causal=True, scale=scale)
    o.backward(torch.tensor(dout))
    logits = (qt.detach() @ kk.detach().transpose(1, 2)) * scale
    causal = torch.ones(q.shape[1], q.shape[1], dtype=torch.bool).tril()
    lse = torch.logsumexp(logits.masked_fill(~causal, -math.inf), dim=-1)
    return o.detach().numpy(), lse.numpy(), qt.grad.numpy(), kt.grad.numpy()


@pytest.mark.parametrize("path", ["raw", "compressed"])
@pytest.mark.parametrize("H,G", [(4, 2), (6, 3), (4, 4)])
def test_grouped_kv_heads_reduce_to_causal(H, G, path):
    """Several key/value heads: with W >= S and no entries (raw path), or r = 1,
    W = 0 and kv_comp = kv (compressed path), every query head reduces to
    causal attention over its group's key/value head, which torch computes with
    repeat_interleave; a wrong head-to-group map (h % G) or a gradient summed
    over the wrong heads fails."""
    rng = np.random.default_rng(14 + H + G)
    B, S, D = 2, 17, 8
    q, kv, dout = rnd(rng, B, H, S, D), rnd(rng, B, G, S, D), rnd(rng, B, H, S, D)
    if path == "raw":
        p = make_problem(B, S, H, D, r=S + 1, W=S)
        got = oracle.full_gqa(p, G, q, kv, np.zeros((B, G, 0, D)), dout)
        key = "dkv"
    else:
        p = make_problem(B, S, H, D, r=1, W=0)
        got = oracle.full_gqa(p, G, q, kv, kv.copy(), dout)
        key = "dkvc"
        assert np.all(got["dkv"] == 0.0)
    for b in range(B):
        o, lse, dq, dkv = causal_reference_grouped(q[b], kv[b], p.scale, dout[b])
        np.testing.assert_allclose(got["o"][b], o, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(got["lse"][b], lse, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(got["dq"][b], dq, atol=1e-11, rtol=1e-9)
        np.testing.assert_allclose(got[key][b], dkv, atol=1e-11, rtol=1e-9)


def explicit_mask_reference(q, kv, kvc, comp_mask, scale, dout):
    """Attention of q [H, S, D] over the raw keys kv [S, D] under the causal mask
    and the compressed keys kvc [Sc, D] under the given mask [S, Sc], as one
    softmax over the concatenated key axis (torch, fp64, autograd)."""
    S, Sc = kv.shape[0], kvc.shape[0]
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(kv, requires_grad=True)
    ct = torch.tensor(kvc, requires_grad=True)
    keys = torch.cat([kt, ct], 0)
    allowed = torch.cat([torch.ones(S, S, dtype=torch.bool).tril(),
                         torch.tensor(comp_mask, dtype=torch.bool)], 1)
    logits = (qt @ keys.T) * scale
    logits = logits.masked_fill(~allowed, -math.inf)
    p = torch.softmax(logits, -1)
    o = p @ keys
    o.backward(torch.tensor(dout))
    lse = torch.logsumexp(logits.detach(), -1)
    return o.detach().numpy(), lse.numpy(), qt.grad.numpy(), kt.grad.numpy(), ct.grad.numpy()


@pytest.mark.parametrize("kind", ["random", "topk"])
def test_mask_mode_matches_explicit_mask_attention(kind):
    """MASK mode (compressed visibility from a given dense mask): with a causal
    raw window (W >= S) it must equal attention with the explicit boolean mask
    [causal | given mask] over the concatenated keys; the mask is random, or
    the one of a per-query top-k index selection (with padding and repeats)."""
    rng = np.random.default_rng(21 if kind == "random" else 22)
    B, S, H, D, Sc = 2, 19, 3, 8, 11
    q, kv, kvc, dout = (rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, Sc, D),
                        rnd(rng, B, H, S, D))
    if kind == "random":
        mask = (rng.random((B, S, Sc)) < 0.35).astype(np.uint8)
    else:
        idx = rng.integers(-2, Sc, size=(B, S, 4))  # negatives are padding
        idx[:, :, 3] = idx[:, :, 0]                  # a repeated pick
        mask = oracle.topk_mask(B, S, Sc, idx)
        for b in range(B):
            for i in range(S):
                assert set(np.nonzero(mask[b, i])[0]) == {int(x) for x in idx[b, i] if x >= 0}
    p = oracle.Problem(B, S, H, D, 1, S, Sc, 1.0 / math.sqrt(D), None, oracle.MASK, "f64",
                       comp_mask=mask)
    got = oracle.full(p, q, kv, kvc, dout)
    for b in range(B):
        o, lse, dq, dkv, dkvc = explicit_mask_reference(q[b], kv[b], kvc[b], mask[b], p.scale,
                                                        dout[b])
        np.testing.assert_allclose(got["o"][b], o, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(got["lse"][b], lse, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(got["dq"][b], dq, atol=1e-11, rtol=1e-9)
        np.testing.assert_allclose(got["dkv"][b], dkv, atol=1e-11, rtol=1e-9)
        np.testing.assert_allclose(got["dkvc"][b], dkvc, atol=1e-11, rtol=1e-9)


def test_mask_mode_with_the_hca_pattern_matches_strict():
    """The dense mask of the HCA pattern itself (completed windows of the
    query's document) in MASK mode gives the STRICT results."""
    rng = np.random.default_rng(23)
    B, S, H, D, r, W = 1, 40, 2, 8, 4, 6
    lengths = [[13, 27]]
    q, kv, kvc, dout = (rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, S // r, D),
                        rnd(rng, B, H, S, D))
    strict = make_problem(B, S, H, D, r, W, lengths)
    mask = np.zeros((B, S, S // r), np.uint8)
    for i in range(S):
        for c in range(S // r):
            mask[0, i, c] = oracle.vis_comp(strict, 0, i, c)
    masked = oracle.Problem(B, S, H, D, r, W, S // r, strict.scale, segment_ids(lengths, B, S),
                            oracle.MASK, "f64", comp_mask=mask)
    a, b = oracle.full(strict, q, kv, kvc, dout), oracle.full(masked, q, kv, kvc, dout)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_duplicated_keys_shift_lse_by_ln2():
    """r = 1, W >= S, kv_comp = kv: every key is seen twice with equal weight."""
    rng = np.random.default_rng(13)
    B, S, H, D = 1, 21, 2, 8
    lengths = [[7, 14]]
    q, kv, dout = rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, H, S, D)
    p = make_problem(B, S, H, D, r=1, W=S, lengths=lengths)
    got = oracle.full(p, q, kv, kv.copy(), dout)
    o, lse, dq, dkv = per_document_causal(q, kv, p.scale, dout, lengths)
    np.testing.assert_allclose(got["o"], o, atol=1e-12)
    np.testing.assert_allclose(got["lse"], lse + math.log(2.0), atol=1e-12)
    np.testing.assert_allclose(got["dq"], dq, atol=1e-11)
    np.testing.assert_allclose(got["dkv"], dkv / 2, atol=1e-11)
    np.testing.assert_allclose(got["dkvc"], dkv / 2, atol=1e-11)


# --------------------------------------------------------------------------- #
# closed forms
# --------------------------------------------------------------------------- #

def interval_sets(S, r, W, lengths, mode):
    """Visible raw range [lo, i] and compressed range [clo, chi) per position,
    written as intervals (the closed form of the masking rule for contiguous
    documents)."""
    seg_start = np.zeros(S, np.int64)
    pos = 0
    for L in (lengths or [S]):
        seg_start[pos:pos + L] = pos
        pos += L
    out = []
    for i in range(S):
        a = seg_start[i]
        lo = max(i - W + 1, a)
        chi = (i + 1) // r
        clo = -(-a // r) if mode == oracle.STRICT else a // r
        out.append((lo, max(clo, 0), max(chi, clo)))
    return out


@pytest.mark.parametrize("mode", [oracle.STRICT, oracle.LAST])
def test_zero_query_closed_form(mode):
    rng = np.random.default_rng(14)
    B, S, H, D, r, W = 1, 45, 2, 8, 4, 5
    lengths = [[6, 11, 28]]
    kv, dout = rnd(rng, B, S, D), rnd(rng, B, H, S, D)
    kvc = rnd(rng, B, S // r, D)
    q = np.zeros((B, H, S, D))
    p = make_problem(B, S, H, D, r, W, lengths, mode)
    got = oracle.full(p, q, kv, kvc, dout)
    sets = interval_sets(S, r, W, lengths[0], mode)
    want_dkv = np.zeros((S, D))
    want_dkvc = np.zeros((S // r, D))
    for i, (lo, clo, chi) in enumerate(sets):
        n = (i - lo + 1) + (chi - clo)
        assert n >= 1
        mean = (kv[0, lo:i + 1].sum(0) + kvc[0, clo:chi].sum(0)) / n
        for h in range(H):
            np.testing.assert_allclose(got["o"][0, h, i], mean, atol=1e-13)
            assert abs(got["lse"][0, h, i] - math.log(n)) < 1e-13
            want_dkv[lo:i + 1] += dout[0, h, i] / n
            want_dkvc[clo:chi] += dout[0, h, i] / n
    np.testing.assert_allclose(got["dkv"][0], want_dkv, atol=1e-12)
    np.testing.assert_allclose(got["dkvc"][0], want_dkvc, atol=1e-12)


def test_constant_values_rows_sum_to_one():
    """All key rows equal v: O = v exactly when the weights of a row sum to 1."""
    rng = np.random.default_rng(15)
    B, S, H, D, r, W = 2, 40, 3, 8, 3, 6
    lengths = [[40], [13, 27]]
    v = rnd(rng, D)
    kv = np.broadcast_to(v, (B, S, D)).copy()
    kvc = np.broadcast_to(v, (B, S // r, D)).copy()
    q, dout = rnd(rng, B, H, S, D), rnd(rng, B, H, S, D)
    p = make_problem(B, S, H, D, r, W, lengths)
    got = oracle.full(p, q, kv, kvc, dout)
    for b in range(B):
        sets = interval_sets(S, r, W, lengths[b], oracle.STRICT)
        for i, (lo, clo, chi) in enumerate(sets):
            n = (i - lo + 1) + (chi - clo)
            for h in range(H):
                np.testing.assert_allclose(got["o"][b, h, i], v, atol=1e-13)
                want = p.scale * float(q[b, h, i] @ v) + math.log(n)
                assert abs(got["lse"][b, h, i] - want) < 1e-12
    # every dP_k is <dO, v>, so dS = 0 and dQ = 0.
    assert np.abs(got["dq"]).max() < 1e-13


def test_window_one_no_entries():
    rng = np.random.default_rng(16)
    B, S, H, D = 1, 17, 3, 8
    q, kv, dout = rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, H, S, D)
    p = make_problem(B, S, H, D, r=S + 1, W=1)
    got = oracle.full(p, q, kv, np.zeros((B, 0, D)), dout)
    np.testing.assert_allclose(got["o"][0], np.broadcast_to(kv[0], (H, S, D)), atol=1e-14)
    np.testing.assert_allclose(got["lse"][0], p.scale * np.einsum("hsd,sd->hs", q[0], kv[0]),
                               atol=1e-13)
    assert np.abs(got["dq"]).max() < 1e-14
    np.testing.assert_allclose(got["dkv"][0], dout[0].sum(0), atol=1e-13)


def test_rows_without_keys():
    rng = np.random.default_rng(17)
    B, S, H, D, r = 1, 10, 2, 4, 4
    q, kv, dout = rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, H, S, D)
    kvc = rnd(rng, B, S // r, D)
    p = make_problem(B, S, H, D, r, W=0)
    got = oracle.full(p, q, kv, kvc, dout)
    # rows 0..2 complete no entry (entry 0 completes at i = 3) and see no raw key
    assert np.all(np.isneginf(got["lse"][0, :, :3]))
    assert np.all(np.isfinite(got["lse"][0, :, 3:]))
    assert np.all(got["o"][0, :, :3] == 0) and np.all(got["dq"][0, :, :3] == 0)
    assert np.all(got["dkv"] == 0)
    # entry 0 alone at i = 3..6: O = kvc[0]
    np.testing.assert_allclose(got["o"][0, :, 3:7], np.broadcast_to(kvc[0, 0], (H, 4, D)),
                               atol=1e-14)


# --------------------------------------------------------------------------- #
# backward: finite differences and the delta identity
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("mode", [oracle.STRICT, oracle.LAST])
def test_backward_matches_finite_differences(mode):
    rng = np.random.default_rng(18)
    B, S, H, D, r, W = 1, 19, 2, 4, 4, 3
    lengths = [[9, 10]]
    q, kv, kvc, dout = (rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, S // r, D),
                        rnd(rng, B, H, S, D))
    p = make_problem(B, S, H, D, r, W, lengths, mode)
    got = oracle.full(p, q, kv, kvc, dout)

    def loss(q_, kv_, kvc_):
        o, _, _, _ = oracle.rows(p, q_, kv_, kvc_, None, need_grad=False)
        return float((o.reshape(B, H, S, D) * dout).sum())

    h = 1e-6
    for name, arr, grad in [("q", q, got["dq"]), ("kv", kv, got["dkv"]), ("kvc", kvc, got["dkvc"])]:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args = {"q": q, "kv": kv, "kvc": kvc}
            args[name] = plus
            lp = loss(args["q"], args["kv"], args["kvc"])
            args[name] = minus
            lm = loss(args["q"], args["kv"], args["kvc"])
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - grad).max() / max(np.abs(fd).max(), 1e-30)
        assert err < 1e-6, (name, err)
        assert np.abs(grad).max() > 1e-3, name


def test_delta_equals_output_dot_dout():
    rng = np.random.default_rng(19)
    B, S, H, D, r, W = 2, 33, 2, 8, 4, 6
    q, kv, kvc, dout = (rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, S // r, D),
                        rnd(rng, B, H, S, D))
    p = make_problem(B, S, H, D, r, W, [[12, 21], [33]])
    got = oracle.full(p, q, kv, kvc, dout)
    np.testing.assert_allclose(got["delta"], np.einsum("bhsd,bhsd->bhs", got["o"], dout),
                               atol=1e-12)


def test_key_pass_with_and_without_row_stats_agree():
    rng = np.random.default_rng(20)
    B, S, H, D, r, W = 1, 30, 2, 8, 4, 5
    q, kv, kvc, dout = (rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, S // r, D),
                        rnd(rng, B, H, S, D))
    p = make_problem(B, S, H, D, r, W, [[11, 19]])
    got = oracle.full(p, q, kv, kvc, dout)
    kinds = np.array([0, 0, 1, 1], np.int32)
    idx = np.array([0, 29, 2, 6], np.int32)
    sampled = oracle.keys(p, q, kv, kvc, dout, kinds, np.zeros(4, np.int32), idx)
    np.testing.assert_allclose(sampled[0], got["dkv"][0, 0], atol=1e-13)
    np.testing.assert_allclose(sampled[1], got["dkv"][0, 29], atol=1e-13)
    np.testing.assert_allclose(sampled[2], got["dkvc"][0, 2], atol=1e-13)
    np.testing.assert_allclose(sampled[3], got["dkvc"][0, 6], atol=1e-13)


# --------------------------------------------------------------------------- #
# pair counts and input widths
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("S,r,W", [(489, 16, 64), (1000, 128, 128), (37, 1, 0), (5, 7, 2)])
def test_pair_counts_single_document(S, r, W):
    p = make_problem(1, S, 1, 4, r, W)
    want_raw = sum(min(W, i + 1) for i in range(S))
    m = S // r
    want_comp = r * m * (m - 1) // 2 + m * (S - m * r + 1)
    assert oracle.count_pairs(p, 0) == want_raw
    assert oracle.count_pairs(p, 1) == want_comp


def test_bf16_and_f32_inputs_widen_exactly():
    rng = np.random.default_rng(21)
    B, S, H, D, r, W = 1, 20, 2, 8, 4, 5
    q, kv, kvc, dout = (rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, S // r, D),
                        rnd(rng, B, H, S, D))
    bf = lambda a: torch.tensor(a, dtype=torch.float32).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    vals = lambda t: t.to(torch.float64).numpy()
    tq, tkv, tkvc, tdo = bf(q), bf(kv), bf(kvc), bf(dout)
    p64 = make_problem(B, S, H, D, r, W)
    a = oracle.full(p64, vals(tq), vals(tkv), vals(tkvc), vals(tdo))
    b = oracle.full(p64.with_dtype("bf16"), bits(tq), bits(tkv), bits(tkvc), bits(tdo))
    c = oracle.full(p64.with_dtype("f32"), *(vals(t).astype(np.float32)
                                             for t in (tq, tkv, tkvc, tdo)))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k


def test_results_independent_of_thread_count():
    """The oracle's per-key gradient sums rows in fixed blocks and adds the
    blocks in order, so its outputs are bitwise the same for any number of
    threads (two fresh processes, one and five threads)."""
    import hashlib
    import subprocess
    import sys as _sys

    code = (
        "import sys, hashlib, numpy as np\n"
        "sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import oracle\n"
        "from test_oracle_pins import make_problem, rnd\n"
        "rng = np.random.default_rng(5)\n"
        "B, S, H, D, r, W = 1, 300, 4, 16, 8, 20\n"
        "q, kv, kvc, dout = (rnd(rng, B, H, S, D), rnd(rng, B, S, D), rnd(rng, B, S // r, D),"
        " rnd(rng, B, H, S, D))\n"
        "out = oracle.full(make_problem(B, S, H, D, r, W, [[120, 180]]), q, kv, kvc, dout)\n"
        "print(oracle.num_threads(), hashlib.sha1(b''.join(np.ascontiguousarray(out[k]).tobytes()"
        " for k in sorted(out))).hexdigest())\n"
    ) % (ROOT, os.path.join(ROOT, "tests"))
    got = {}
    for t in (1, 5):
        env = dict(os.environ, OMP_NUM_THREADS=str(t))
        r = subprocess.run([_sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=120)
        assert r.returncode == 0, r.stderr
        n, h = r.stdout.split()
        assert int(n) == t
        got[t] = h
    assert got[1] == got[5]
