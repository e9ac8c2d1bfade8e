// hca_plan.cpp -- analytic block table and schedules for HCA attention (host only).
//
// The HCA pattern is deterministic, so the tile-level block mask can be built
// from coordinates on the host ahead of time, with no S x S mask anywhere
// ("Add HCA Static Compilation for Splash Attention [Deepseek v4]",
// Description: the static block mask is evaluated on the CPU from coordinates
// rather than materialised in device memory).  Each query position i of a
// document starting at a_i sees
//   raw keys          [max(i - W + 1, a_i), i]                    (none if W = 0)
//   compressed entries [lo_c, floor((i + 1) / r))
// with lo_c = ceil(a_i / r) under the STRICT document rule (the entry's whole
// window lies in the document) and floor(a_i / r) under the LAST rule (the
// window's last position lies in the document).  Both follow from the element
// rule (entry c is complete for i iff (c+1) r <= i + 1) for contiguous
// documents.  Tiles are classified from these intervals row by row; the
// element predicate itself is never evaluated here.
#include <algorithm>
#include <climits>
#include <cstring>
#include <new>
#include <numeric>

#include "hca_internal.h"

namespace hca {

namespace {

constexpr uint64_t kAlign = 256;
inline uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Positions covered by one work item of the key-stationary backward kernels;
// longer query-tile lists are split into several items whose partial
// gradients are summed afterwards in a fixed order.  64 positions keep a
// compressed tile's items about as short as a raw tile's (whose keys are seen
// by at most W + bk - 1 positions), so no few long items form the tail, and
// give enough items to fill every CU at S = 16384 (128 positions left its
// launch at 1.5 items per CU; 64 cut that dKV kernel 2.1 -> 1.65 ms, and the
// extra partial sums cost little once the reduction streamed them in groups).
constexpr int64_t kItemPositions = 64;

// Items of a compressed key tile span a run of chunks: its rows can number up
// to S x H, so one item per chunk would make the partial gradients grow as
// S^2 / r.  Runs are kept as short as possible, though: items of different
// key tiles over the same chunk stream the same rows, and when a compressed
// tile's item covers several chunks it reads them long after the raw tiles'
// items over the same chunks did, so the rows come from HBM twice (S = 65536:
// dKV 9.0 ms with one-chunk runs, 10.3 with two, 10.5 with four).  By
// default the run doubles from one chunk only until the compressed tiles'
// partial blocks fit in twice the raw tiles' (which grow as S), with a floor
// of 4 kCuTarget blocks: the workspace stays O(S) and shorter problems keep
// one-chunk items.
constexpr int64_t kCuTarget = 256;
// float32 dKV: visits per workgroup of a compressed entry, and at most this
// many workgroups per entry.
constexpr int64_t kF32SplitVisits = 256;
constexpr int64_t kF32SplitMax = 64;
constexpr int64_t kF32PartBudget = 256ll << 20;

// Half-tile items (128-key tiles whose item sees one 64-key half) share the
// key-stationary launch with the items over whole tiles, so by default they
// are used at any size.
constexpr int64_t kHalfItemsMin = 1;

// State of query tile qt (positions qt*bq .. +bq-1) against keys [k0, k0+bk)
// of `kind`, from the per-position intervals `rw` ([S][4]).
int classify_tile(const int32_t *rw, int64_t S, int64_t qt, int bq, int kind, int64_t k0,
                  int64_t bk, int64_t nk) {
  const int64_t i0 = qt * bq, i1 = std::min<int64_t>(S, i0 + bq);
  const int64_t k1 = k0 + bk, kend = std::min<int64_t>(k1, nk);
  bool any = false, all = i0 + bq <= S && k1 <= nk;
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t lo = kind ? rw[i * 4 + 1] : rw[i * 4];
    const int64_t hi = kind ? rw[i * 4 + 2] : i + 1;
    if (std::max(lo, k0) < std::min(hi, kend)) any = true;
    if (!(lo <= k0 && k1 <= hi)) all = false;
  }
  return any ? (all ? HCA_TILE_FULL : HCA_TILE_PARTIAL) : HCA_TILE_EMPTY;
}

// State of query tile qt against compressed entries [k0, k0 + bk) when their
// visibility is a given dense mask `m` ([S][Sc] of one batch row).
int classify_tile_mask(const uint8_t *m, int64_t S, int64_t Sc, int64_t qt, int bq, int64_t k0,
                       int64_t bk) {
  const int64_t i0 = qt * bq, i1 = std::min<int64_t>(S, i0 + bq);
  const int64_t kend = std::min<int64_t>(k0 + bk, Sc);
  bool any = false, all = i0 + bq <= S && k0 + bk <= Sc;
  for (int64_t i = i0; i < i1; ++i)
    for (int64_t c = k0; c < kend; ++c) {
      const bool v = m[i * Sc + c] != 0;
      any |= v;
      all &= v;
    }
  return any ? (all ? HCA_TILE_FULL : HCA_TILE_PARTIAL) : HCA_TILE_EMPTY;
}

}  // namespace

// Keys per key tile of the key-stationary backward (a work item covers one
// tile).  Head dim 512, bf16: 64 -- the backward then stores P and dS in its
// first pass and the key-stationary pass reads them (see the key-tile section
// of build_plan; above kPdsBudget of stored tiles the library's choice falls
// back to 128, which recomputes S and dP with an O(S) workspace).  Other
// kernels: the forward's 32-key tile.  `want` (the tile configuration's
// kv_keys) overrides where the width has a kernel; 0 if it has none.
constexpr uint64_t kPdsBudget = 32ull << 30;  // bytes of stored P and dS, library choice
static int kv_tile_keys(int dtype, int D, int want) {
  if (dtype == HCA_BF16 && D == 512) {
    if (want == 0) return 64;
    return want == 64 || want == 128 ? want : 0;
  }
  return want == 0 || want == 32 ? 32 : 0;
}

void default_tiles(int dtype, int D, int H, int *bq, int *bk_raw, int *bk_comp) {
  if (dtype == HCA_BF16 && H >= 1 && H <= 128 && 128 % H == 0) {
    // D = 512 kernels want at least 16 positions per tile (one wave = 16
    // consecutive positions of one head); the others take 128 rows per tile.
    *bq = D == 512 ? std::max(16, 128 / H) : 128 / H;
  } else {
    *bq = 16;
  }
  *bk_raw = 32;
  *bk_comp = 32;
}

std::string kernel_supports(int dtype, int D, int H, int bq, int bk_raw, int bk_comp) {
  if (dtype == HCA_BF16) {
    if (bk_raw != 32 || bk_comp != 32) return "bfloat16 kernels need 32-key tiles";
    const int64_t rows = (int64_t)bq * H;
    if (D == 64 || D == 128)
      return rows == 128 ? "" : "head dim 64/128 kernels need bq * H == 128";
    // D = 512: bq >= 16 and bq * H >= 128, both powers of two.
    if (D == 512)
      return bq >= 16 && (bq & (bq - 1)) == 0 && rows >= 128 && (rows & (rows - 1)) == 0 &&
                     rows <= 1 << 20
                 ? ""
                 : "head dim 512 kernels need bq >= 16 and bq * H >= 128, both powers of two";
    return "no bfloat16 kernel for this head dim (64, 128 and 512 are built)";
  }
  // float32 path: vector kernels, any tile shape.
  return D % 64 == 0 && D >= 64 && D <= 512 ? ""
                                           : "float32 kernels need a head dim in 64..512, "
                                             "a multiple of 64";
}

// The D = 512 kernels address a key tensor's tile images (4 D bytes per key:
// K and K^T in bfloat16) with 32-bit buffer offsets; the D = 64 / 128 and
// float32 kernels index with 64-bit offsets.
std::string kernel_sizes_ok(int dtype, int D, int64_t S_pad, int64_t Sc_pad) {
  if (dtype == HCA_BF16 && D == 512) {
    const int64_t lim = (int64_t)1 << 31;
    if (S_pad * D * 4 >= lim || Sc_pad * D * 4 >= lim)
      return "sequence too long for the head dim 512 kernels' 32-bit tile-image offsets "
             "(padded keys x 2048 bytes must stay below 2^31)";
  }
  return "";
}

}  // namespace hca

using namespace hca;

// Builds the plan of B batch rows x G kv heads.  Query head h uses kv head
// h / (H / G), so each (batch row, kv head) pair with its H / G query heads is
// one MQA problem with the same documents, and their tensors are contiguous
// slices of q [B][H][S][D] and kv [B][G][S][D]: the plan holds B * G such
// rows of H / G heads, and the kernels run them unchanged.
// cmask: NULL, or a dense mask [B][S][S_c] that decides the visibility of
// every compressed pair (G = 1); the raw window keeps its rule.
static hca_status build_plan(const char *fn, int32_t B, int32_t G, int32_t S, int32_t r,
                             int32_t W, int32_t S_c, const int32_t *seg_starts,
                             const int32_t *seg_counts, int32_t H, int32_t D, hca_dtype dtype,
                             hca_compseg_mode mode, const hca_tile_cfg *tiles, hca_plan **out,
                             const uint8_t *cmask = nullptr) {
  const std::string F(fn);
  if (!out) {
    set_error(F + ": out is NULL");
    return HCA_ERR_INVALID_ARG;
  }
  *out = nullptr;
  if (B < 1 || S < 1 || H < 1 || D < 1) {
    set_error(F + ": B, S, H and D must all be >= 1");
    return HCA_ERR_INVALID_ARG;
  }
  if (G < 1 || H % G != 0) {
    set_error(F + ": kv_heads must be >= 1 and divide H");
    return HCA_ERR_INVALID_ARG;
  }
  if ((int64_t)B * G > (1 << 20)) {
    set_error(F + ": B x kv_heads must be at most 2^20");
    return HCA_ERR_INVALID_ARG;
  }
  if (r < 1) {
    set_error(F + ": compression ratio r must be >= 1");
    return HCA_ERR_INVALID_ARG;
  }
  if (W < 0) {
    set_error(F + ": window W must be >= 0");
    return HCA_ERR_INVALID_ARG;
  }
  if (!cmask && S_c != S / r) {
    set_error(F + ": S_c must equal floor(S / r) = " + std::to_string(S / r) +
              ", got " + std::to_string(S_c));
    return HCA_ERR_INVALID_ARG;
  }
  if (dtype != HCA_F32 && dtype != HCA_BF16) {
    set_error(F + ": unknown dtype");
    return HCA_ERR_INVALID_ARG;
  }
  if (mode != HCA_COMPSEG_STRICT && mode != HCA_COMPSEG_LAST) {
    set_error(F + ": unknown compressed-segment mode");
    return HCA_ERR_INVALID_ARG;
  }
  if ((seg_starts == nullptr) != (seg_counts == nullptr)) {
    set_error(F + ": seg_starts and seg_counts must both be NULL or both set");
    return HCA_ERR_INVALID_ARG;
  }
  // Document lists: per row strictly increasing, first 0, all < S.
  std::vector<int64_t> seg_off(B + 1, 0);
  if (seg_counts) {
    for (int b = 0; b < B; ++b) {
      if (seg_counts[b] < 1 || seg_counts[b] > S) {
        set_error(F + ": seg_counts[" + std::to_string(b) +
                  "] must be in [1, S]");
        return HCA_ERR_INVALID_ARG;
      }
      seg_off[b + 1] = seg_off[b] + seg_counts[b];
    }
    for (int b = 0; b < B; ++b) {
      const int32_t *st = seg_starts + seg_off[b];
      int64_t n = seg_off[b + 1] - seg_off[b];
      if (st[0] != 0) {
        set_error(F + ": first document start of row " + std::to_string(b) +
                  " must be 0");
        return HCA_ERR_INVALID_ARG;
      }
      for (int64_t j = 1; j < n; ++j) {
        if (st[j] <= st[j - 1] || st[j] >= S) {
          set_error(F + ": document starts of row " + std::to_string(b) +
                    " must be strictly increasing and < S");
          return HCA_ERR_INVALID_ARG;
        }
      }
    }
  }
  // B * G rows of H / G heads from here on; the documents of batch row b are
  // repeated for each of its kv heads (internal row b * G + g).
  const int32_t B_caller = B, H_caller = H;
  std::vector<int32_t> starts_rep, counts_rep;
  if (G > 1) {
    if (seg_counts) {
      for (int b = 0; b < B; ++b)
        for (int g = 0; g < G; ++g) {
          starts_rep.insert(starts_rep.end(), seg_starts + seg_off[b], seg_starts + seg_off[b + 1]);
          counts_rep.push_back(seg_counts[b]);
        }
      seg_starts = starts_rep.data();
      seg_counts = counts_rep.data();
    }
    B *= G;
    H /= G;
    seg_off.assign(B + 1, 0);
    if (seg_counts)
      for (int b = 0; b < B; ++b) seg_off[b + 1] = seg_off[b] + seg_counts[b];
  }
  int bq, bkr, bkc;
  default_tiles(dtype, D, H, &bq, &bkr, &bkc);
  int64_t half_min = kHalfItemsMin;
  int64_t comp_chunks_cfg = 0;
  const int kv_keys = kv_tile_keys(dtype, D, tiles ? tiles->kv_keys : 0);
  if (kv_keys == 0) {
    set_error(F + ": kv_keys must be 0, 64 or 128 at head dim 512 bfloat16, else 0 or 32");
    return HCA_ERR_INVALID_ARG;
  }
  if (tiles) {
    if (tiles->bq < 0 || tiles->bk_raw < 0 || tiles->bk_comp < 0 ||
        tiles->comp_item_chunks < 0) {
      set_error(F + ": tile sizes and comp_item_chunks must be >= 0");
      return HCA_ERR_INVALID_ARG;
    }
    if (tiles->bq) bq = tiles->bq;
    if (tiles->bk_raw) bkr = tiles->bk_raw;
    if (tiles->bk_comp) bkc = tiles->bk_comp;
    if (tiles->half_items_min > 0) half_min = tiles->half_items_min;
    if (tiles->half_items_min < 0) half_min = INT64_MAX;
    comp_chunks_cfg = tiles->comp_item_chunks;
  }
  // Work-list entries pack tile indices into 30 bits.
  if (ceil_div(S, bq) >= (1 << 29) || ceil_div(S, bkr) >= (1 << 29)) {
    set_error(F + ": too many tiles");
    return HCA_ERR_INVALID_ARG;
  }

  hca_plan *p = new (std::nothrow) hca_plan();
  if (!p) {
    set_error(F + ": out of host memory");
    return HCA_ERR_NOMEM;
  }
  try {
    const int64_t nqt = ceil_div(S, bq);
    const int64_t nktr = ceil_div(S, bkr);
    const int64_t nktc = ceil_div(S_c, bkc);
    hca_plan_info &in = p->info;
    in.B = B_caller; in.S = S; in.H = H_caller; in.D = D; in.r = r; in.W = W; in.S_c = S_c;
    in.kv_heads = G;
    p->rows_b = B;
    in.dtype = dtype; in.comp_mode = mode;
    in.bq = bq; in.bk_raw = bkr; in.bk_comp = bkc;
    in.nqt = (int32_t)nqt; in.nkt_raw = (int32_t)nktr; in.nkt_comp = (int32_t)nktc;
    p->unsupported = kernel_supports(dtype, D, H, bq, bkr, bkc);
    if (p->unsupported.empty())
      p->unsupported = kernel_sizes_ok(dtype, D, nktr * bkr, nktc * bkc);
    if (p->unsupported.empty() && cmask && !(dtype == HCA_BF16 && D == 512))
      p->unsupported = "plans with a given compressed-key mask run on the head dim 512 "
                       "bfloat16 kernels only";
    // the key-stationary kernel addresses the mask bits with 32-bit byte offsets
    if (p->unsupported.empty() && cmask &&
        (int64_t)B * S * ceil_div(S_c, 128) * 16 >= ((int64_t)1 << 31))
      p->unsupported = "compressed-key mask too large for 32-bit offsets";
    in.comp_masked = cmask ? 1 : 0;
    in.kernel_ok = p->unsupported.empty() ? 1 : 0;
    p->kv_bk = kv_keys;
    in.kv_keys = kv_keys;

    // ---- per-position visible intervals --------------------------------- //
    p->rows.assign((size_t)B * S * 4, 0);
    int64_t pairs_raw = 0, pairs_comp = 0;
    for (int b = 0; b < B; ++b) {
      const int32_t *st = seg_starts ? seg_starts + seg_off[b] : nullptr;
      const int64_t nseg = seg_starts ? seg_off[b + 1] - seg_off[b] : 1;
      int64_t next = 1, a = 0;
      for (int64_t i = 0; i < S; ++i) {
        while (st && next < nseg && st[next] <= i) a = st[next++];
        int64_t rlo = W == 0 ? i + 1 : std::max<int64_t>(i - W + 1, a);
        int64_t chi = std::min<int64_t>((i + 1) / r, S_c);
        int64_t clo = mode == HCA_COMPSEG_STRICT ? ceil_div(a, r) : a / r;
        if (clo > chi) clo = chi;
        if (cmask) {  // the mask decides; the interval spans every entry
          clo = 0;
          chi = S_c;
          const uint8_t *mr = cmask + ((size_t)b * S + i) * S_c;
          for (int64_t c = 0; c < S_c; ++c) pairs_comp += mr[c] != 0;
        } else {
          pairs_comp += chi - clo;
        }
        int32_t *row = &p->rows[((size_t)b * S + i) * 4];
        row[0] = (int32_t)rlo; row[1] = (int32_t)clo; row[2] = (int32_t)chi; row[3] = 0;
        pairs_raw += std::max<int64_t>(0, i - rlo + 1);
      }
    }
    // Every kv head's rows see the same pattern: pairs per caller batch row.
    in.pairs_raw = pairs_raw / G;
    in.pairs_comp = pairs_comp / G;

    // ---- query-tile schedule (CSR) ---------------------------------------- //
    p->qptr.assign((size_t)B * nqt + 1, 0);
    std::vector<int64_t> cost((size_t)B * nqt, 0);
    int64_t full_raw = 0, full_comp = 0;
    for (int b = 0; b < B; ++b) {
      for (int64_t qt = 0; qt < nqt; ++qt) {
        const int64_t i0 = qt * bq, i1 = std::min<int64_t>(S, i0 + bq);
        const bool nominal_q = i0 + bq <= S;
        const int32_t *rw = &p->rows[((size_t)b * S) * 4];
        // raw key tiles
        int64_t lo = INT64_MAX, hi = -1;
        for (int64_t i = i0; i < i1; ++i) {
          if (rw[i * 4] <= i) {
            lo = std::min<int64_t>(lo, rw[i * 4]);
            hi = std::max<int64_t>(hi, i);
          }
        }
        if (hi >= 0) {
          for (int64_t kt = lo / bkr; kt <= hi / bkr; ++kt) {
            const int64_t k0 = kt * bkr, k1 = k0 + bkr, kend = std::min<int64_t>(k1, S);
            bool any = false, all = nominal_q && k1 <= S;
            for (int64_t i = i0; i < i1; ++i) {
              const int64_t rlo = rw[i * 4];
              if (std::max(rlo, k0) <= std::min(i, kend - 1)) any = true;
              if (!(rlo <= k0 && k1 - 1 <= i)) all = false;
            }
            if (!any) continue;
            uint32_t e = (uint32_t)kt | (all ? kEntFull : 0u);
            p->qent.push_back(e);
            full_raw += all;
            cost[(size_t)b * nqt + qt] += bkr;
          }
        }
        // compressed entry tiles
        if (cmask) {
          const uint8_t *m = cmask + (size_t)b * S * S_c;
          for (int64_t kt = 0; kt < nktc; ++kt) {
            const int st = classify_tile_mask(m, S, S_c, qt, bq, kt * bkc, bkc);
            if (st == HCA_TILE_EMPTY) continue;
            p->qent.push_back((uint32_t)kt | kEntComp | (st == HCA_TILE_FULL ? kEntFull : 0u));
            full_comp += st == HCA_TILE_FULL;
            cost[(size_t)b * nqt + qt] += bkc;
          }
          p->qptr[(size_t)b * nqt + qt + 1] = (int32_t)p->qent.size();
          continue;
        }
        lo = INT64_MAX;
        hi = -1;
        for (int64_t i = i0; i < i1; ++i) {
          const int64_t clo = rw[i * 4 + 1], chi = rw[i * 4 + 2];
          if (clo < chi) {
            lo = std::min(lo, clo);
            hi = std::max(hi, chi - 1);
          }
        }
        if (hi >= 0) {
          for (int64_t kt = lo / bkc; kt <= hi / bkc; ++kt) {
            const int64_t k0 = kt * bkc, k1 = k0 + bkc, kend = std::min<int64_t>(k1, S_c);
            bool any = false, all = nominal_q && k1 <= S_c;
            for (int64_t i = i0; i < i1; ++i) {
              const int64_t clo = rw[i * 4 + 1], chi = rw[i * 4 + 2];
              if (std::max(clo, k0) < std::min(chi, kend)) any = true;
              if (!(clo <= k0 && k1 <= chi)) all = false;
            }
            if (!any) continue;
            uint32_t e = (uint32_t)kt | kEntComp | (all ? kEntFull : 0u);
            p->qent.push_back(e);
            full_comp += all;
            cost[(size_t)b * nqt + qt] += bkc;
          }
        }
        p->qptr[(size_t)b * nqt + qt + 1] = (int32_t)p->qent.size();
      }
    }
    if (p->qent.size() >= (size_t)INT32_MAX) throw std::bad_alloc();
    in.full_raw = full_raw;
    in.full_comp = full_comp;
    int64_t ent_comp = 0;
    for (uint32_t e : p->qent) ent_comp += (e & kEntComp) ? 1 : 0;
    in.tiles_raw = (int64_t)p->qent.size() - ent_comp;
    in.tiles_comp = ent_comp;

    // Heaviest query tiles first.
    p->qorder.resize((size_t)B * nqt);
    std::iota(p->qorder.begin(), p->qorder.end(), 0);
    std::stable_sort(p->qorder.begin(), p->qorder.end(),
                     [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
    // Staggered first round: every workgroup loads its query rows before its
    // tile loop and stores its output rows after it.  If the first round of
    // workgroups all cost the same, all of them hit memory at the same time,
    // then all compute, and the rounds stay in lock step.  Taking the first
    // round's tiles from across the heavier half of the list spreads their
    // finishing times; the rest follow heaviest first, so the tail stays light.
    {
      constexpr int64_t kFirstRound = 256;
      const int64_t n = (int64_t)p->qorder.size();
      if (n >= 4 * kFirstRound) {
        std::vector<int32_t> order;
        order.reserve(n);
        std::vector<char> taken(n, 0);
        for (int64_t i = 0; i < kFirstRound; ++i) {
          const int64_t at = i * (n / 2) / kFirstRound;
          order.push_back(p->qorder[at]);
          taken[at] = 1;
        }
        for (int64_t i = 0; i < n; ++i)
          if (!taken[i]) order.push_back(p->qorder[i]);
        p->qorder.swap(order);
      }
    }

    // ---- key-tile work lists for the key-stationary backward ------------ //
    // Library choice of 64-key tiles with stored P and dS: one bq * H x 32
    // block of each per listed (query tile, 32-key tile) pair, O(S (W + S / r))
    // bytes; past kPdsBudget the recomputing 128-key backward is used.
    if (p->kv_bk == 64 && !(tiles && tiles->kv_keys) &&
        (uint64_t)p->qent.size() * 2 * bq * H * 32 * 2 > kPdsBudget) {
      p->kv_bk = 128;
      in.kv_keys = 128;
    }
    // Key tiles of kv_bk keys (64 or 128 at D = 512, wider than the forward's
    // 32); for each, the query tiles that see any of its keys, classified from
    // the same intervals.
    const int64_t kvb = p->kv_bk;
    // 64-key tiles at D = 512: P and dS stored by the dQ pass (see below).
    const bool stored = dtype == HCA_BF16 && D == 512 && kvb == 64;
    const int64_t nkvr = ceil_div(S, kvb), nkvc = ceil_div(S_c, kvb);
    const int64_t nkv = nkvr + nkvc;
    // Query tiles per 64-position chunk.
    const int64_t chunk = std::max<int64_t>(1, kItemPositions / bq);
    std::vector<std::vector<uint32_t>> lists((size_t)B * nkv);
    int64_t total_entries = 0;
    for (int b = 0; b < B; ++b) {
      const int32_t *rw = &p->rows[((size_t)b * S) * 4];
      for (int64_t t = 0; t < nkv; ++t) {
        const int kind = t < nkvr ? 0 : 1;
        const int64_t kt = kind ? t - nkvr : t;
        const int64_t k0 = kt * kvb;
        const int64_t nk = kind ? S_c : S;
        // positions that can see a key of [k0, k0 + kvb)
        int64_t p0, p1;
        if (kind == 0) {
          p0 = k0;
          p1 = W > 0 ? std::min<int64_t>(S - 1, k0 + kvb - 1 + W - 1) : -1;
        } else {
          p0 = cmask ? 0 : (k0 + 1) * r - 1;
          p1 = S - 1;
        }
        std::vector<uint32_t> &list = lists[(size_t)b * nkv + t];
        for (int64_t qt = p0 >= 0 && p0 <= p1 ? p0 / bq : 0; p0 <= p1 && qt <= p1 / bq; ++qt) {
          const int st = kind && cmask
                             ? classify_tile_mask(cmask + (size_t)b * S * S_c, S, S_c, qt, bq,
                                                  k0, kvb)
                             : classify_tile(rw, S, qt, bq, kind, k0, kvb, nk);
          if (st != HCA_TILE_EMPTY)
            list.push_back((uint32_t)qt | (st == HCA_TILE_FULL ? kEntFull : 0u));
        }
        total_entries += (int64_t)list.size();
      }
    }
    // Chunks per compressed-tile item (raw tiles: one chunk per item; their
    // keys are seen by at most W + kv_bk - 1 positions).
    auto count_items = [&](int kind, int64_t run) {  // items of `kind` with runs of `run` qts
      int64_t n = 0;
      for (int b = 0; b < B; ++b)
        for (int64_t t = kind ? nkvr : 0; t < (kind ? nkv : nkvr); ++t) {
          const std::vector<uint32_t> &list = lists[(size_t)b * nkv + t];
          for (size_t e = 0; e < list.size(); ++e)
            if (e == 0 || (list[e] & kEntIdx) / run != (list[e - 1] & kEntIdx) / run) ++n;
        }
      return n;
    };
    int64_t cchunks = comp_chunks_cfg;
    if (cchunks == 0 && stored) {
      // With stored P / dS the workspace already holds 256 x bq x H bytes per
      // listed (query tile, 64-key tile) pair, O(visible pairs); one-chunk
      // items, whose partial blocks (kv_bk x D float32, 128 KiB) number at
      // most the listed pairs over a chunk's query tiles, grow no faster.
      // Longer runs only cost balance: with per-query top-k selections every
      // query tile lists every compressed tile, and eight-chunk runs left the
      // key-stationary pass at 7.7 ms against 5.9 with one-chunk items
      // (S = 16384, H = 64, r = 4, 512 of 4096 entries per query).
      cchunks = 1;
    } else if (cchunks == 0) {
      const int64_t budget = std::max<int64_t>(2 * count_items(0, chunk), 4 * kCuTarget);
      cchunks = 1;
      while (cchunks < ceil_div(nqt, chunk) && count_items(1, chunk * cchunks) > budget)
        cchunks *= 2;
    }
    (void)total_entries;
    const int64_t ngrid = ceil_div(ceil_div(nqt, chunk), cchunks);  // item groups per row
    p->kvtile.assign((size_t)B * nkv * 2, 0);
    std::vector<int64_t> item_group;  // (b, run of cchunks chunks) of each item
    std::vector<int64_t> item_tile;   // b * nkv + t of each item
    for (int b = 0; b < B; ++b) {
      const int32_t *rw = &p->rows[((size_t)b * S) * 4];
      for (int64_t t = 0; t < nkv; ++t) {
        const int kind = t < nkvr ? 0 : 1;
        const int64_t kt = kind ? t - nkvr : t;
        const int64_t k0 = kt * kvb;
        const int64_t nk = kind ? S_c : S;
        const std::vector<uint32_t> &list = lists[(size_t)b * nkv + t];
        const int64_t run = kind ? chunk * cchunks : chunk;  // query tiles per item at most
        // Items break at multiples of `run` query tiles, the same grid for
        // every key tile of a kind, so the items of different key tiles over
        // one stretch of positions stream exactly the same query rows.
        for (size_t s0 = 0; s0 < list.size();) {
          const int64_t ck = (int64_t)(list[s0] & kEntIdx) / run;
          size_t s1 = s0 + 1;
          while (s1 < list.size() && (int64_t)(list[s1] & kEntIdx) / run == ck) ++s1;
          KvItem it{};
          it.b = b;
          it.kind = kind;
          it.kt = (int32_t)kt;
          it.e0 = (int32_t)p->kvent.size();
          p->kvent.insert(p->kvent.end(), list.begin() + s0, list.begin() + s1);
          it.e1 = (int32_t)p->kvent.size();
          it.halves = 3;
          if (kvb == 128 && !stored) {
            // Which 64-key halves of the tile any row of the item sees, from
            // the same per-position intervals as the tile states.
            it.halves = 0;
            const int64_t kmid = std::min<int64_t>(k0 + 64, nk), kend = std::min<int64_t>(k0 + kvb, nk);
            for (size_t e = s0; e < s1; ++e) {
              const int64_t qt = list[e] & kEntIdx;
              for (int64_t i = qt * bq; i < std::min<int64_t>(S, qt * bq + bq); ++i) {
                if (kind && cmask) {
                  const uint8_t *mr = cmask + ((size_t)b * S + i) * S_c;
                  for (int64_t c = k0; c < kend; ++c)
                    if (mr[c]) it.halves |= c < kmid ? 1 : 2;
                  continue;
                }
                const int64_t lo = kind ? rw[i * 4 + 1] : rw[i * 4];
                const int64_t hi = kind ? rw[i * 4 + 2] : i + 1;
                if (std::max(lo, k0) < std::min(hi, kmid)) it.halves |= 1;
                if (std::max(lo, kmid) < std::min(hi, kend)) it.halves |= 2;
              }
            }
            if (it.halves == 0) it.halves = 3;  // (a listed tile always has a visible key)
          }
          p->kvitem.push_back(it);
          const int64_t first_chunk = (int64_t)(list[s0] & kEntIdx) / chunk;
          item_group.push_back((int64_t)b * ngrid + first_chunk / cchunks);
          item_tile.push_back((int64_t)b * nkv + t);
          s0 = s1;
        }
      }
    }
    if (p->kvent.size() >= (size_t)INT32_MAX) throw std::bad_alloc();
    p->nkv_raw = (int32_t)nkvr;
    p->nkv_comp = (int32_t)nkvc;
    in.comp_item_chunks = (int32_t)cchunks;

    // With few items, every item runs over its whole tile (see kHalfItemsMin).
    if ((int64_t)p->kvitem.size() < half_min)
      for (KvItem &it : p->kvitem) it.halves = 3;

    // Partial blocks.  A key tile's items own consecutive [kv_bk][D] float32
    // blocks (the reduction sums them in block order).  Items over the whole
    // tile take a block each; an item over the lower half and one over the
    // upper half of the same tile share a block, each writing its half; a
    // half item left without a partner writes its whole block, zeros in the
    // idle half.
    int64_t nblocks = 0;
    {
      size_t i0 = 0;
      while (i0 < p->kvitem.size()) {
        size_t i1 = i0 + 1;
        while (i1 < p->kvitem.size() && item_tile[i1] == item_tile[i0]) ++i1;
        const int64_t tile = item_tile[i0];
        const int64_t first = nblocks;
        std::vector<size_t> lows, highs;
        for (size_t i = i0; i < i1; ++i) {
          KvItem &it = p->kvitem[i];
          it.shared = 0;
          if (it.halves == 1) lows.push_back(i);
          else if (it.halves == 2) highs.push_back(i);
          else it.part_off = nblocks++ * kvb * D;
        }
        const size_t npair = std::min(lows.size(), highs.size());
        for (size_t k = 0; k < std::max(lows.size(), highs.size()); ++k) {
          const int64_t off = nblocks++ * kvb * D;
          if (k < lows.size()) {
            p->kvitem[lows[k]].part_off = off;
            p->kvitem[lows[k]].shared = k < npair;
          }
          if (k < highs.size()) {
            p->kvitem[highs[k]].part_off = off;
            p->kvitem[highs[k]].shared = k < npair;
          }
        }
        p->kvtile[tile * 2] = (int32_t)first;
        p->kvtile[tile * 2 + 1] = (int32_t)(nblocks - first);
        i0 = i1;
      }
    }
    if (nblocks >= INT32_MAX) throw std::bad_alloc();
    int64_t nhalf = 0;
    for (const KvItem &it : p->kvitem) nhalf += it.halves != 3;
    in.items = (int64_t)p->kvitem.size();
    in.items_half = nhalf;
    in.part_blocks = nblocks;

    // Launch order.  Workgroup i of a launch goes to XCD i % kXcd, and each
    // XCD runs its share in order.  The items of one group (one stretch of
    // positions) read the same query rows at about the same pace, so a group
    // is kept together on one XCD, where its L2 serves the repeated reads.
    // Groups go, heaviest first, to the least-loaded XCD; slots past the end
    // of a short XCD queue hold -1 (no work).
    {
      constexpr int kXcd = 8;
      const int64_t ngroup = (int64_t)B * ngrid;
      auto build_order = [&]() {
        std::vector<int64_t> gwork(ngroup, 0);
        std::vector<std::vector<int32_t>> gitems(ngroup);
        for (size_t i = 0; i < p->kvitem.size(); ++i) {
          gwork[item_group[i]] += p->kvitem[i].e1 - p->kvitem[i].e0;
          gitems[item_group[i]].push_back((int32_t)i);
        }
        std::vector<int64_t> gorder;
        for (int64_t gi = 0; gi < ngroup; ++gi)
          if (!gitems[gi].empty()) gorder.push_back(gi);
        std::stable_sort(gorder.begin(), gorder.end(),
                         [&](int64_t x, int64_t y) { return gwork[x] > gwork[y]; });
        std::vector<std::vector<int32_t>> queue(kXcd);
        std::vector<int64_t> load(kXcd, 0);
        for (int64_t gi : gorder) {
          std::vector<int32_t> &its = gitems[gi];
          std::stable_sort(its.begin(), its.end(), [&](int32_t x, int32_t y) {
            return (p->kvitem[x].e1 - p->kvitem[x].e0) > (p->kvitem[y].e1 - p->kvitem[y].e0);
          });
          const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
          queue[x].insert(queue[x].end(), its.begin(), its.end());
          load[x] += gwork[gi];
        }
        size_t qmax = 0;
        for (const auto &qq : queue) qmax = std::max(qmax, qq.size());
        std::vector<int32_t> order(qmax * kXcd, -1);
        for (int x = 0; x < kXcd; ++x)
          for (size_t k = 0; k < queue[x].size(); ++k) order[k * kXcd + x] = queue[x][k];
        return order;
      };
      p->kvorder = build_order();
    }

    // ---- stored P and dS --------------------------------------------------- //
    // With 64-key tiles at D = 512 the dQ pass stores P and dS (bf16) of every
    // listed (query tile, 32-key tile) pair, and the key-stationary pass reads
    // them instead of recomputing S and dP.  A 64-key tile's entry for query
    // tile qt names the stored blocks of its two 32-key halves: their indices
    // in qt's list (the qent CSR), -1 where qt does not list that half.
    if (stored) {
      p->pds_rows = (int32_t)(bq * H);
      const int64_t nqk = kvb / 32;  // 32-key tiles of the forward per key tile
      p->kvpe.assign(p->kvent.size() * nqk, -1);
      std::vector<std::pair<uint64_t, int32_t>> keyed;  // (qt, kind, tile) -> qent index
      for (int b = 0; b < B; ++b) {
        keyed.clear();
        for (int64_t qt = 0; qt < nqt; ++qt)
          for (int32_t e = p->qptr[b * nqt + qt]; e < p->qptr[b * nqt + qt + 1]; ++e) {
            const uint32_t ent = p->qent[e];
            keyed.emplace_back(((uint64_t)qt << 32) | (ent & (kEntComp | kEntIdx)), e);
          }
        std::sort(keyed.begin(), keyed.end());
        auto find = [&](int64_t qt, uint32_t kind, int64_t tile) -> int32_t {
          const uint64_t key = ((uint64_t)qt << 32) | (kind ? kEntComp : 0u) | (uint32_t)tile;
          auto at = std::lower_bound(keyed.begin(), keyed.end(),
                                     std::make_pair(key, (int32_t)INT32_MIN));
          return at != keyed.end() && at->first == key ? at->second : -1;
        };
        for (const KvItem &it : p->kvitem) {
          if (it.b != b) continue;
          for (int32_t e = it.e0; e < it.e1; ++e) {
            const int64_t qt = p->kvent[e] & kEntIdx;
            for (int64_t h = 0; h < nqk; ++h)
              p->kvpe[nqk * (size_t)e + h] = find(qt, it.kind, nqk * (int64_t)it.kt + h);
          }
        }
      }
    }

    // ---- device image ----------------------------------------------------- //
    DevLayout &L = p->lay;
    uint64_t off = 0;
    auto place = [&](uint64_t bytes) { uint64_t o = off; off = align_up(off + bytes); return o; };
    L.rows = place(p->rows.size() * 4);
    L.qptr = place(p->qptr.size() * 4);
    L.qent = place(std::max<size_t>(1, p->qent.size()) * 4);
    L.qorder = place(p->qorder.size() * 4);
    L.kvitem = place(std::max<size_t>(1, p->kvitem.size()) * sizeof(KvItem));
    L.kvorder = place(std::max<size_t>(1, p->kvorder.size()) * 4);
    L.kvent = place(std::max<size_t>(1, p->kvent.size()) * 4);
    L.kvtile = place(p->kvtile.size() * 4);
    if (cmask) {
      // The mask as bits: per (row, query position) ceil(S_c / 128) * 4 words,
      // bit c % 32 of word c / 32 set when entry c is visible.
      p->cmask_ldw = (int32_t)(ceil_div(S_c, 128) * 4);
      L.cmask = place((uint64_t)B * S * p->cmask_ldw * 4);
    }
    if (stored) L.kvpe = place(std::max<size_t>(1, p->kvpe.size()) * 4);
    L.total = off;
    p->image.assign(L.total, 0);
    auto put = [&](uint64_t o, const void *src, size_t bytes) {
      if (bytes) std::memcpy(p->image.data() + o, src, bytes);
    };
    put(L.rows, p->rows.data(), p->rows.size() * 4);
    put(L.qptr, p->qptr.data(), p->qptr.size() * 4);
    put(L.qent, p->qent.data(), p->qent.size() * 4);
    put(L.qorder, p->qorder.data(), p->qorder.size() * 4);
    put(L.kvitem, p->kvitem.data(), p->kvitem.size() * sizeof(KvItem));
    put(L.kvorder, p->kvorder.data(), p->kvorder.size() * 4);
    put(L.kvent, p->kvent.data(), p->kvent.size() * 4);
    put(L.kvtile, p->kvtile.data(), p->kvtile.size() * 4);
    if (stored) put(L.kvpe, p->kvpe.data(), p->kvpe.size() * 4);
    if (cmask) {
      uint32_t *words = reinterpret_cast<uint32_t *>(p->image.data() + L.cmask);
      for (size_t row = 0; row < (size_t)B * S; ++row) {
        const uint8_t *mr = cmask + row * S_c;
        uint32_t *wr = words + row * p->cmask_ldw;
        for (int64_t c = 0; c < S_c; ++c)
          if (mr[c]) wr[c >> 5] |= 1u << (c & 31);
      }
    }
    in.device_bytes = L.total;

    // ---- workspaces ------------------------------------------------------- //
    WsLayout &w = p->ws;
    off = 0;
    if (dtype == HCA_BF16 && D == 512) {
      // K and K^T of every tile in MFMA fragment order (the tile images).  The
      // D = 64 / 128 kernels stage the row-major tensor itself.
      w.kvt = place(2 * B * D * (nktr * bkr) * 2);
      w.kvct = place(2 * B * D * std::max<int64_t>(1, nktc * bkc) * 2);
    }
    w.fwd_total = off;
    w.delta = place((uint64_t)B * H * S * 4);
    // (the float32 kernels write dKV directly: no key-tile partials)
    if (dtype != HCA_F32) w.part = place((uint64_t)std::max<int64_t>(1, nblocks * kvb * D) * 4);
    if (dtype == HCA_F32 && S_c > 0) {
      // float32 dKV: the visits of a compressed entry (up to S x H rows) are
      // split over f32_split workgroups of about kF32SplitVisits each, whose
      // partial sums a second kernel adds in split order.
      int64_t split = std::min<int64_t>(
          kF32SplitMax, std::max<int64_t>(1, ceil_div((int64_t)S * H, kF32SplitVisits)));
      // ... and at most kF32PartBudget bytes of partial sums in all
      split = std::max<int64_t>(
          1, std::min<int64_t>(split, kF32PartBudget / ((int64_t)B * S_c * D * 4)));
      p->f32_split = (int32_t)split;
      if (split > 1) w.f32_part = place((uint64_t)B * S_c * split * D * 4);
    }
    if (stored) {
      // per qent entry: P and dS of bq * H rows x 32 keys, bf16
      w.pds_bytes = (uint64_t)std::max<size_t>(1, p->qent.size()) * 2 * bq * H * 32 * 2;
      w.pds = place(w.pds_bytes);
      in.ws_pds_bytes = w.pds_bytes;
    }
    w.bwd_total = off;
    in.ws_fwd_bytes = w.fwd_total;
    in.ws_bwd_bytes = w.bwd_total;
  } catch (const std::bad_alloc &) {
    delete p;
    set_error(F + ": out of host memory");
    return HCA_ERR_NOMEM;
  }
  *out = p;
  return HCA_OK;
}

extern "C" hca_status hca_block_mask_build(int32_t B, int32_t S, int32_t r, int32_t W,
                                           int32_t S_c, const int32_t *seg_starts,
                                           const int32_t *seg_counts, int32_t H, int32_t D,
                                           hca_dtype dtype, hca_compseg_mode mode,
                                           const hca_tile_cfg *tiles, hca_plan **out) {
  return build_plan("hca_block_mask_build", B, 1, S, r, W, S_c, seg_starts, seg_counts, H, D,
                    dtype, mode, tiles, out);
}

extern "C" hca_status hca_block_mask_build_gqa(int32_t B, int32_t kv_heads, int32_t S,
                                               int32_t r, int32_t W, int32_t S_c,
                                               const int32_t *seg_starts,
                                               const int32_t *seg_counts, int32_t H, int32_t D,
                                               hca_dtype dtype, hca_compseg_mode mode,
                                               const hca_tile_cfg *tiles, hca_plan **out) {
  return build_plan("hca_block_mask_build_gqa", B, kv_heads, S, r, W, S_c, seg_starts,
                    seg_counts, H, D, dtype, mode, tiles, out);
}

extern "C" hca_status hca_block_mask_build_masked(int32_t B, int32_t S, int32_t W, int32_t S_c,
                                                  const int32_t *seg_starts,
                                                  const int32_t *seg_counts, int32_t H,
                                                  int32_t D, hca_dtype dtype,
                                                  const uint8_t *comp_mask,
                                                  const hca_tile_cfg *tiles, hca_plan **out) {
  if (!comp_mask || S_c < 0) {
    set_error("hca_block_mask_build_masked: comp_mask is NULL or S_c < 0");
    if (out) *out = nullptr;
    return HCA_ERR_INVALID_ARG;
  }
  // r only enters the compressed rule, which the mask replaces.
  return build_plan("hca_block_mask_build_masked", B, 1, S, 1, W, S_c, seg_starts, seg_counts,
                    H, D, dtype, HCA_COMPSEG_STRICT, tiles, out, comp_mask);
}

extern "C" hca_status hca_block_mask_build_topk(int32_t B, int32_t S, int32_t W, int32_t S_c,
                                                const int32_t *seg_starts,
                                                const int32_t *seg_counts, int32_t H, int32_t D,
                                                hca_dtype dtype, const int32_t *idx, int32_t K,
                                                const hca_tile_cfg *tiles, hca_plan **out) {
  if (out) *out = nullptr;
  if (!idx || K < 1 || S_c < 1 || B < 1 || S < 1) {
    set_error("hca_block_mask_build_topk: idx is NULL, or K, S_c, B or S < 1");
    return HCA_ERR_INVALID_ARG;
  }
  std::vector<uint8_t> mask;
  try {
    mask.assign((size_t)B * S * S_c, 0);
  } catch (const std::bad_alloc &) {
    set_error("hca_block_mask_build_topk: out of host memory");
    return HCA_ERR_NOMEM;
  }
  for (size_t row = 0; row < (size_t)B * S; ++row)
    for (int32_t k = 0; k < K; ++k) {
      const int32_t c = idx[row * K + k];
      if (c >= S_c) {
        set_error("hca_block_mask_build_topk: index " + std::to_string(c) + " >= S_c");
        return HCA_ERR_INVALID_ARG;
      }
      if (c >= 0) mask[row * S_c + c] = 1;
    }
  return build_plan("hca_block_mask_build_topk", B, 1, S, 1, W, S_c, seg_starts, seg_counts, H,
                    D, dtype, HCA_COMPSEG_STRICT, tiles, out, mask.data());
}

extern "C" hca_status hca_plan_get_info(const hca_plan *plan, hca_plan_info *out) {
  if (!plan || !out) {
    set_error("hca_plan_get_info: NULL argument");
    return HCA_ERR_INVALID_ARG;
  }
  *out = plan->info;
  return HCA_OK;
}

extern "C" hca_status hca_plan_export_tiles(const hca_plan *plan, uint8_t *raw_states,
                                            uint8_t *comp_states) {
  if (!plan) {
    set_error("hca_plan_export_tiles: plan is NULL");
    return HCA_ERR_INVALID_ARG;
  }
  const hca_plan_info &in = plan->info;
  const size_t nqt = in.nqt, nktr = in.nkt_raw, nktc = in.nkt_comp;
  const int nb = plan->rows_b;  // batch rows x kv heads
  if (raw_states) std::memset(raw_states, HCA_TILE_EMPTY, (size_t)nb * nqt * nktr);
  if (comp_states) std::memset(comp_states, HCA_TILE_EMPTY, (size_t)nb * nqt * nktc);
  for (int b = 0; b < nb; ++b)
    for (size_t qt = 0; qt < nqt; ++qt)
      for (int32_t e = plan->qptr[b * nqt + qt]; e < plan->qptr[b * nqt + qt + 1]; ++e) {
        uint32_t v = plan->qent[e];
        uint8_t st = (v & kEntFull) ? HCA_TILE_FULL : HCA_TILE_PARTIAL;
        size_t kt = v & kEntIdx;
        if (v & kEntComp) {
          if (comp_states) comp_states[((size_t)b * nqt + qt) * nktc + kt] = st;
        } else if (raw_states) {
          raw_states[((size_t)b * nqt + qt) * nktr + kt] = st;
        }
      }
  return HCA_OK;
}

extern "C" hca_status hca_plan_export_rows(const hca_plan *plan, int32_t *rows) {
  if (!plan || !rows) {
    set_error("hca_plan_export_rows: NULL argument");
    return HCA_ERR_INVALID_ARG;
  }
  const size_t n = (size_t)plan->rows_b * plan->info.S;
  for (size_t j = 0; j < n; ++j)
    for (int c = 0; c < 3; ++c) rows[j * 3 + c] = plan->rows[j * 4 + c];
  return HCA_OK;
}

extern "C" hca_status hca_plan_export_items(const hca_plan *plan, int64_t *items,
                                            int64_t capacity, int64_t *count) {
  if (!plan || !count || capacity < 0) {
    set_error("hca_plan_export_items: NULL plan or count, or negative capacity");
    return HCA_ERR_INVALID_ARG;
  }
  const int64_t n = (int64_t)plan->kvitem.size();
  *count = n;
  if (!items) return HCA_OK;
  for (int64_t i = 0; i < std::min(n, capacity); ++i) {
    const KvItem &it = plan->kvitem[i];
    int64_t *o = items + i * 8;
    o[0] = it.b;
    o[1] = it.kind;
    o[2] = (int64_t)it.kt * plan->kv_bk;
    o[3] = plan->kv_bk;
    o[4] = it.e1 > it.e0 ? (int64_t)(plan->kvent[it.e0] & kEntIdx) : -1;
    o[5] = it.e1 > it.e0 ? (int64_t)(plan->kvent[it.e1 - 1] & kEntIdx) : -1;
    o[6] = it.halves | (it.shared ? 4 : 0);
    o[7] = it.part_off;
  }
  return HCA_OK;
}

extern "C" void hca_plan_destroy(hca_plan *plan) { delete plan; }
