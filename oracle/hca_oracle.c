/*
 * hca_oracle.c -- plain CPU oracle for DeepSeek-V4 Heavily Compressed Attention (HCA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the HIP
 * library; it is written from the pages' description of the method alone.
 *
 * What it computes (all arithmetic in fp64):
 *
 *   Masking rule -- "Add HCA Static Compilation for Splash Attention
 *   [Deepseek v4]", Description: each query attends to a local sliding window
 *   of raw keys plus every compression window that has completed before it;
 *   the pattern is deterministic (no indexer, no top-k).  The precise
 *   conventions used here (window bounds, completion boundary, segment rule)
 *   are the ones this library fixes where the pages leave them open:
 *     raw key t is visible to query i   iff  i - W < t <= i  and seg(t) == seg(i)
 *     compressed entry c (covering raw positions [c*r, (c+1)*r)) is visible
 *     to query i  iff  (c+1)*r <= i+1  and  segc(c) == seg(i)
 *   where segc(c) is the entry's document: in STRICT mode the document that
 *   holds the whole window (or none when the window straddles a boundary), in
 *   LAST mode the document of the window's last raw position.  In MASK mode
 *   a given dense mask decides every compressed pair instead (see
 *   hco_vis_comp).
 *   Segment ids isolate packed documents ("document packing boundary
 *   isolation", same page, Description; the segment-equality mask in
 *   "DSV4: Route compressed and sliding train attention onto the splash
 *   kernels", review of build_local_sliding_splash_mask).
 *
 *   Attention -- "[DeepSeek-V4] Implement Compressed Attention Layers",
 *   review suggestions on the einsum form: logits are the scaled dot products
 *   of each query head with a single shared key/value tensor (k = v = kv,
 *   broadcast over heads), one softmax over all visible keys, output = the
 *   softmax-weighted sum of the same kv rows.  Raw and compressed keys form one
 *   concatenated key axis, so there is a single softmax and a single
 *   log-sum-exp per query row.
 *
 *   Gradients -- the standard derivative of softmax attention with K = V
 *   shared: for loss L = sum(O * dO),
 *     dP_k  = <dO_i, kv_k>
 *     delta = sum_k P_k dP_k
 *     dS_k  = P_k (dP_k - delta)
 *     dQ_i  = scale * sum_k dS_k kv_k
 *     dKV_k = sum over (h, i) that see k of  scale * dS_k * q_{h,i} + P_k * dO_{h,i}
 *   (the key-path and value-path gradients add because K and V are one tensor).
 *
 *   Rows with no visible key: O = 0, LSE = -inf, and they contribute nothing
 *   to any gradient.
 *
 *   Tile states -- brute force over the element predicate: a (query-tile,
 *   key-tile) rectangle is EMPTY (0) if no in-range element is visible, FULL
 *   (2) if every element of the nominal rectangle is in range and visible,
 *   PARTIAL (1) otherwise.
 *
 * Inputs are read as float32, bfloat16 bit patterns or float64 and widened
 * to double exactly.  Layouts: q, dout [B][H][S][D]; kv [B][S][D];
 * kvc [B][Sc][D]; seg [B][S] (per-token document id).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t B, S, H, D, r, W, Sc;
  int32_t comp_mode; /* 0 = STRICT, 1 = LAST, 2 = MASK */
  int32_t in_dtype;  /* 0 = float32, 1 = bfloat16 bit patterns, 2 = float64 */
  int32_t pad_;
  double scale;
  const int32_t *seg;        /* [B][S] */
  const uint8_t *comp_mask;  /* [B][S][Sc], MASK mode only: nonzero = visible */
} hco_problem;

/* ---- element access ------------------------------------------------------ */

static double load_val(const void *base, int32_t dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float *)base)[idx];
  if (dtype == 2) return ((const double *)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int32_t seg_of(const hco_problem *p, int32_t b, int64_t t) {
  return p->seg[(int64_t)b * p->S + t];
}

/* ---- the element predicate ---------------------------------------------- */

/* Document that compressed entry c belongs to (-1: none). */
static int32_t comp_segment(const hco_problem *p, int32_t b, int32_t c) {
  int64_t first = (int64_t)c * p->r, last = (int64_t)(c + 1) * p->r - 1;
  if (p->comp_mode == 1) return seg_of(p, b, last);
  int32_t s0 = seg_of(p, b, first);
  for (int64_t t = first; t <= last; ++t)
    if (seg_of(p, b, t) != s0) return -1;
  return s0;
}

int hco_vis_raw(const hco_problem *p, int32_t b, int64_t i, int64_t t) {
  if (i < 0 || i >= p->S || t < 0 || t >= p->S) return 0;
  if (!(i - p->W < t && t <= i)) return 0;
  return seg_of(p, b, t) == seg_of(p, b, i);
}

/*
 * MASK mode: the visibility of every (query, compressed entry) pair is given
 * as a materialised dense mask, the form in which the dynamic path of "Add
 * HCA Static Compilation for Splash Attention [Deepseek v4]" (Description)
 * hands the compressed attention its pattern (a dense (B, 1, S, S_comp) mask
 * in device memory), and in which a per-query selection of entries (a top-k
 * over the compressed keys) is expressed.  The raw window keeps its rule.
 */
int hco_vis_comp(const hco_problem *p, int32_t b, int64_t i, int64_t c) {
  if (i < 0 || i >= p->S || c < 0 || c >= p->Sc) return 0;
  if (p->comp_mode == 2) return p->comp_mask[((int64_t)b * p->S + i) * p->Sc + c] != 0;
  if ((c + 1) * (int64_t)p->r > i + 1) return 0;
  return comp_segment(p, b, (int32_t)c) == seg_of(p, b, i);
}

/* ---- one query row ------------------------------------------------------- */

/* Key handle: kind 0 = raw position, 1 = compressed entry. */
typedef struct {
  int32_t kind;
  int32_t idx;
} keyref;

static const void *key_base(const void *kv, const void *kvc, int32_t kind) {
  return kind == 0 ? kv : kvc;
}

static int64_t key_row_offset(const hco_problem *p, int32_t b, keyref k) {
  if (k.kind == 0) return ((int64_t)b * p->S + k.idx) * p->D;
  return ((int64_t)b * p->Sc + k.idx) * p->D;
}

/* Lists every key visible to query i of batch b by scanning all candidates. */
static int64_t visible_keys(const hco_problem *p, int32_t b, int64_t i, keyref *out) {
  int64_t n = 0;
  for (int64_t t = 0; t < p->S; ++t)
    if (hco_vis_raw(p, b, i, t)) out[n++] = (keyref){0, (int32_t)t};
  for (int64_t c = 0; c < p->Sc; ++c)
    if (hco_vis_comp(p, b, i, c)) out[n++] = (keyref){1, (int32_t)c};
  return n;
}

static double dot_row(const hco_problem *p, const void *x, int64_t xoff, const void *kv,
                      const void *kvc, int32_t b, keyref k) {
  const void *kb = key_base(kv, kvc, k.kind);
  int64_t koff = key_row_offset(p, b, k);
  double acc = 0.0;
  for (int32_t d = 0; d < p->D; ++d)
    acc += load_val(x, p->in_dtype, xoff + d) * load_val(kb, p->in_dtype, koff + d);
  return acc;
}

/*
 * Full row computation for query row (b, h, i): output O (D values), LSE,
 * delta = sum_k P_k dP_k, and dQ (D values).  Any output pointer may be NULL.
 * Work buffers: keys (>= S + Sc entries), s and dp (same length).
 */
static void row_compute(const hco_problem *p, const void *q, const void *kv, const void *kvc,
                        const void *dout, int32_t b, int32_t h, int64_t i, keyref *keys,
                        double *s, double *dp, double *o, double *lse, double *delta,
                        double *dq) {
  const int32_t D = p->D;
  const int64_t qoff = (((int64_t)b * p->H + h) * p->S + i) * D;
  int64_t n = visible_keys(p, b, i, keys);
  if (n == 0) {
    if (o) for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    if (lse) *lse = -INFINITY;
    if (delta) *delta = 0.0;
    if (dq) for (int32_t d = 0; d < D; ++d) dq[d] = 0.0;
    return;
  }
  double m = -INFINITY;
  for (int64_t k = 0; k < n; ++k) {
    s[k] = p->scale * dot_row(p, q, qoff, kv, kvc, b, keys[k]);
    if (s[k] > m) m = s[k];
  }
  double l = 0.0;
  for (int64_t k = 0; k < n; ++k) l += exp(s[k] - m);
  /* s[] now becomes the probabilities P_k. */
  for (int64_t k = 0; k < n; ++k) s[k] = exp(s[k] - m) / l;
  if (lse) *lse = m + log(l);
  if (o) {
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t k = 0; k < n; ++k) {
      const void *kb = key_base(kv, kvc, keys[k].kind);
      int64_t koff = key_row_offset(p, b, keys[k]);
      for (int32_t d = 0; d < D; ++d) o[d] += s[k] * load_val(kb, p->in_dtype, koff + d);
    }
  }
  if (!delta && !dq) return;
  double dl = 0.0;
  for (int64_t k = 0; k < n; ++k) {
    dp[k] = dot_row(p, dout, qoff, kv, kvc, b, keys[k]);
    dl += s[k] * dp[k];
  }
  if (delta) *delta = dl;
  if (dq) {
    for (int32_t d = 0; d < D; ++d) dq[d] = 0.0;
    for (int64_t k = 0; k < n; ++k) {
      double ds = s[k] * (dp[k] - dl);
      const void *kb = key_base(kv, kvc, keys[k].kind);
      int64_t koff = key_row_offset(p, b, keys[k]);
      for (int32_t d = 0; d < D; ++d) dq[d] += p->scale * ds * load_val(kb, p->in_dtype, koff + d);
    }
  }
}

/*
 * Row pass over a list of query rows.  rows[j] is the flat row index
 * (b * H + h) * S + i.  Outputs: o, dq are [nrows][D]; lse, delta [nrows].
 * dout may be NULL (then delta and dq must be NULL too).
 */
void hco_rows(const hco_problem *p, const void *q, const void *kv, const void *kvc,
              const void *dout, int64_t nrows, const int64_t *rows, double *o, double *lse,
              double *delta, double *dq) {
  const int64_t nk = (int64_t)p->S + p->Sc + 1;
#pragma omp parallel
  {
    keyref *keys = (keyref *)malloc(sizeof(keyref) * nk);
    double *s = (double *)malloc(sizeof(double) * nk);
    double *dp = (double *)malloc(sizeof(double) * nk);
#pragma omp for schedule(dynamic, 16)
    for (int64_t j = 0; j < nrows; ++j) {
      int64_t flat = rows[j];
      int64_t i = flat % p->S;
      int64_t bh = flat / p->S;
      int32_t h = (int32_t)(bh % p->H), b = (int32_t)(bh / p->H);
      row_compute(p, q, kv, kvc, dout, b, h, i, keys, s, dp, o ? o + j * p->D : NULL,
                  lse ? lse + j : NULL, delta ? delta + j : NULL, dq ? dq + j * p->D : NULL);
    }
    free(keys);
    free(s);
    free(dp);
  }
}

/*
 * Key pass: gradient of the shared key/value row for each listed key.
 * kinds[j] = 0 (raw position) or 1 (compressed entry), bs[j] = batch, idx[j] =
 * position or entry.  lse_all / delta_all are [B][H][S] arrays from a row pass
 * over every row, or NULL: then each row that sees the key is recomputed here.
 * dkv is [nkeys][D].
 */
void hco_keys(const hco_problem *p, const void *q, const void *kv, const void *kvc,
              const void *dout, const double *lse_all, const double *delta_all, int64_t nkeys,
              const int32_t *kinds, const int32_t *bs, const int32_t *idx, double *dkv) {
  const int32_t D = p->D;
  const int64_t nk = (int64_t)p->S + p->Sc + 1;
  const int64_t nrow = (int64_t)p->H * p->S;
  /* The rows are summed in fixed blocks of kRowBlock (rows in order inside a
   * block, then the blocks in order), so the result does not depend on the
   * thread count or on which thread took which block. */
  enum { kRowBlock = 64 };
  const int64_t nblk = (nrow + kRowBlock - 1) / kRowBlock;
  double *bpart = (double *)malloc(sizeof(double) * (size_t)(nblk > 0 ? nblk : 1) * D);
  unsigned char *bused = (unsigned char *)malloc((size_t)(nblk > 0 ? nblk : 1));
  for (int64_t j = 0; j < nkeys; ++j) {
    keyref key = {kinds[j], idx[j]};
    int32_t b = bs[j];
    double *out = dkv + j * D;
    for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
#pragma omp parallel
    {
      keyref *keys = NULL;
      double *s = NULL, *dp = NULL;
      if (!lse_all) {
        keys = (keyref *)malloc(sizeof(keyref) * nk);
        s = (double *)malloc(sizeof(double) * nk);
        dp = (double *)malloc(sizeof(double) * nk);
      }
#pragma omp for schedule(dynamic, 1)
      for (int64_t blk = 0; blk < nblk; ++blk) {
        double *acc = bpart + blk * D;
        for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
        bused[blk] = 0;
        const int64_t hi_end = (blk + 1) * kRowBlock < nrow ? (blk + 1) * kRowBlock : nrow;
        for (int64_t hi = blk * kRowBlock; hi < hi_end; ++hi) {
          int32_t h = (int32_t)(hi / p->S);
          int64_t i = hi % p->S;
          int vis = key.kind == 0 ? hco_vis_raw(p, b, i, key.idx) : hco_vis_comp(p, b, i, key.idx);
          if (!vis) continue;
          bused[blk] = 1;
          int64_t qoff = (((int64_t)b * p->H + h) * p->S + i) * D;
          double lse, delta;
          if (lse_all) {
            lse = lse_all[((int64_t)b * p->H + h) * p->S + i];
            delta = delta_all[((int64_t)b * p->H + h) * p->S + i];
          } else {
            row_compute(p, q, kv, kvc, dout, b, h, i, keys, s, dp, NULL, &lse, &delta, NULL);
          }
          double sk = p->scale * dot_row(p, q, qoff, kv, kvc, b, key);
          double pk = exp(sk - lse);
          double dpk = dot_row(p, dout, qoff, kv, kvc, b, key);
          double dsk = pk * (dpk - delta);
          for (int32_t d = 0; d < D; ++d)
            acc[d] += p->scale * dsk * load_val(q, p->in_dtype, qoff + d) +
                      pk * load_val(dout, p->in_dtype, qoff + d);
        }
      }
      free(keys);
      free(s);
      free(dp);
    }
    /* blocks without a visible row hold zeros and are skipped */
    for (int64_t blk = 0; blk < nblk; ++blk)
      if (bused[blk])
        for (int32_t d = 0; d < D; ++d) out[d] += bpart[blk * D + d];
  }
  free(bused);
  free(bpart);
}

/* ---- tile states, brute force --------------------------------------------- */

/* State of one (query tile qt, key tile kt) rectangle of kind 0 (raw) or 1 (compressed). */
uint8_t hco_tile_state(const hco_problem *p, int32_t kind, int32_t b, int64_t qt, int64_t kt,
                       int32_t bq, int32_t bk) {
  const int64_t nkeys = kind == 0 ? p->S : p->Sc;
  int any = 0;
  int all = ((qt + 1) * bq <= p->S) && ((kt + 1) * bk <= nkeys);
  for (int64_t i = qt * bq; i < (qt + 1) * bq; ++i) {
    for (int64_t k = kt * bk; k < (kt + 1) * bk; ++k) {
      int v = 0;
      if (i < p->S && k < nkeys)
        v = kind == 0 ? hco_vis_raw(p, b, i, k) : hco_vis_comp(p, b, i, k);
      any |= v;
      all &= v;
    }
  }
  if (!any) return 0;
  return all ? 2 : 1;
}

/* Whole table: out[b][qt][kt] for qt < ceil(S/bq), kt < ceil(nkeys/bk). */
void hco_tile_states(const hco_problem *p, int32_t kind, int32_t bq, int32_t bk, uint8_t *out) {
  const int64_t nkeys = kind == 0 ? p->S : p->Sc;
  const int64_t nqt = (p->S + bq - 1) / bq;
  const int64_t nkt = (nkeys + bk - 1) / bk;
  const int64_t total = (int64_t)p->B * nqt * nkt;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t e = 0; e < total; ++e) {
    int64_t kt = e % nkt;
    int64_t qt = (e / nkt) % nqt;
    int32_t b = (int32_t)(e / (nkt * nqt));
    out[e] = hco_tile_state(p, kind, b, qt, kt, bq, bk);
  }
}

/* Selected tiles: tiles[j] = flat (b * nqt + qt) * nkt + kt. */
void hco_tile_states_at(const hco_problem *p, int32_t kind, int32_t bq, int32_t bk, int64_t n,
                        const int64_t *tiles, uint8_t *out) {
  const int64_t nkeys = kind == 0 ? p->S : p->Sc;
  const int64_t nqt = (p->S + bq - 1) / bq;
  const int64_t nkt = (nkeys + bk - 1) / bk;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t j = 0; j < n; ++j) {
    int64_t e = tiles[j];
    int64_t kt = e % nkt;
    int64_t qt = (e / nkt) % nqt;
    int32_t b = (int32_t)(e / (nkt * nqt));
    out[j] = hco_tile_state(p, kind, b, qt, kt, bq, bk);
  }
}

/* Number of visible (query position, key) pairs per batch row, summed over the batch. */
int64_t hco_count_pairs(const hco_problem *p, int32_t kind) {
  int64_t total = 0;
  const int64_t nkeys = kind == 0 ? p->S : p->Sc;
#pragma omp parallel for reduction(+ : total) schedule(dynamic, 64)
  for (int64_t bi = 0; bi < (int64_t)p->B * p->S; ++bi) {
    int32_t b = (int32_t)(bi / p->S);
    int64_t i = bi % p->S;
    for (int64_t k = 0; k < nkeys; ++k)
      total += kind == 0 ? hco_vis_raw(p, b, i, k) : hco_vis_comp(p, b, i, k);
  }
  return total;
}

int hco_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
