/* Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * CPU oracle (hca_oracle.c): runs the row pass, key pass, tile classifier
 * and pair counts over small problems in every mode and input type. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
  int32_t B, S, H, D, r, W, Sc;
  int32_t comp_mode, in_dtype, pad_;
  double scale;
  const int32_t *seg;
  const uint8_t *comp_mask;
} hco_problem;

void hco_rows(const hco_problem *, const void *, const void *, const void *, const void *,
              int64_t, const int64_t *, double *, double *, double *, double *);
void hco_keys(const hco_problem *, const void *, const void *, const void *, const void *,
              const double *, const double *, int64_t, const int32_t *, const int32_t *,
              const int32_t *, double *);
void hco_tile_states(const hco_problem *, int32_t, int32_t, int32_t, uint8_t *);
int64_t hco_count_pairs(const hco_problem *, int32_t);

static double frand(void) { return rand() / (double)RAND_MAX - 0.5; }

int main(void) {
  srand(3);
  int runs = 0;
  for (int t = 0; t < 24; ++t) {
    const int B = 1 + t % 2, S = 1 + rand() % 60, H = 1 + rand() % 3, D = 8, r = 1 + rand() % 9;
    const int W = rand() % 20, mode = t % 3, dt = t % 3 == 2 ? 2 : (t % 2);
    const int Sc = mode == 2 ? 1 + rand() % 20 : S / r;
    const size_t es = dt == 0 ? 4 : (dt == 1 ? 2 : 8);
    int32_t *seg = malloc(sizeof(int32_t) * B * S);
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < S; ++i) seg[b * S + i] = i / (1 + S / 3);
    uint8_t *mask = malloc((size_t)B * S * (Sc ? Sc : 1));
    for (int k = 0; k < B * S * Sc; ++k) mask[k] = rand() % 3 == 0;
    hco_problem p = {B, S, H, D, r, W, Sc, mode, dt, 0, 0.35, seg, mode == 2 ? mask : NULL};
    const size_t nq = (size_t)B * H * S * D, nk = (size_t)B * S * D, nc = (size_t)B * (Sc ? Sc : 1) * D;
    void *q = malloc(nq * es), *kv = malloc(nk * es), *kvc = malloc(nc * es), *dout = malloc(nq * es);
    for (size_t k = 0; k < nq * es; ++k) ((uint8_t *)q)[k] = rand();
    for (size_t k = 0; k < nq * es; ++k) ((uint8_t *)dout)[k] = rand();
    for (size_t k = 0; k < nk * es; ++k) ((uint8_t *)kv)[k] = rand();
    for (size_t k = 0; k < nc * es; ++k) ((uint8_t *)kvc)[k] = rand();
    if (dt != 1) { /* keep float inputs finite */
      for (size_t k = 0; k < nq; ++k) {
        if (dt == 0) { ((float *)q)[k] = frand(); ((float *)dout)[k] = frand(); }
        else { ((double *)q)[k] = frand(); ((double *)dout)[k] = frand(); }
      }
      for (size_t k = 0; k < nk; ++k) { if (dt == 0) ((float *)kv)[k] = frand(); else ((double *)kv)[k] = frand(); }
      for (size_t k = 0; k < nc; ++k) { if (dt == 0) ((float *)kvc)[k] = frand(); else ((double *)kvc)[k] = frand(); }
    } else { /* bf16: clear exponents that would make inf / nan */
      for (size_t k = 0; k < nq; ++k) { ((uint16_t *)q)[k] &= 0xbfff; ((uint16_t *)dout)[k] &= 0xbfff; }
      for (size_t k = 0; k < nk; ++k) ((uint16_t *)kv)[k] &= 0xbfff;
      for (size_t k = 0; k < nc; ++k) ((uint16_t *)kvc)[k] &= 0xbfff;
    }
    const int64_t nrow = (int64_t)B * H * S;
    int64_t *rows = malloc(sizeof(int64_t) * nrow);
    for (int64_t k = 0; k < nrow; ++k) rows[k] = k;
    double *o = malloc(sizeof(double) * nrow * D), *lse = malloc(sizeof(double) * nrow);
    double *delta = malloc(sizeof(double) * nrow), *dq = malloc(sizeof(double) * nrow * D);
    hco_rows(&p, q, kv, kvc, dout, nrow, rows, o, lse, delta, dq);
    const int64_t nkeys = (int64_t)B * (S + Sc);
    int32_t *kinds = malloc(4 * nkeys), *bs = malloc(4 * nkeys), *idx = malloc(4 * nkeys);
    int64_t j = 0;
    for (int b = 0; b < B; ++b) {
      for (int i = 0; i < S; ++i) { kinds[j] = 0; bs[j] = b; idx[j++] = i; }
      for (int c = 0; c < Sc; ++c) { kinds[j] = 1; bs[j] = b; idx[j++] = c; }
    }
    double *dkv = malloc(sizeof(double) * nkeys * D);
    hco_keys(&p, q, kv, kvc, dout, lse, delta, nkeys, kinds, bs, idx, dkv);
    hco_keys(&p, q, kv, kvc, dout, NULL, NULL, nkeys < 4 ? nkeys : 4, kinds, bs, idx, dkv);
    for (int kind = 0; kind < 2; ++kind) {
      const int bq = 1 + rand() % 8, bk = 1 + rand() % 8, nkk = kind ? Sc : S;
      uint8_t *st = malloc((size_t)B * ((S + bq - 1) / bq) * ((nkk + bk - 1) / bk) + 1);
      hco_tile_states(&p, kind, bq, bk, st);
      free(st);
      (void)hco_count_pairs(&p, kind);
    }
    free(seg); free(mask); free(q); free(kv); free(kvc); free(dout); free(rows); free(o);
    free(lse); free(delta); free(dq); free(kinds); free(bs); free(idx); free(dkv);
    ++runs;
  }
  printf("oracle problems %d\n", runs);
  return 0;
}
