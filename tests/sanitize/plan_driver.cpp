// Host-only driver for the AddressSanitizer / UndefinedBehaviorSanitizer
// build of the planner (hca_plan.cpp): builds plans over edge cases and
// random configurations and reads every export back.  Any out-of-bounds
// access, leak or undefined behaviour aborts the run.  The planner's only
// outside dependency, set_error, is defined here.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "hca_internal.h"

namespace hca {
void set_error(const std::string &) {}
}  // namespace hca

static int fails = 0;

static void exercise(hca_plan *p) {
  hca_plan_info in{};
  if (hca_plan_get_info(p, &in) != HCA_OK) { ++fails; return; }
  const size_t nb = (size_t)in.B * in.kv_heads;
  std::vector<uint8_t> raw(nb * in.nqt * in.nkt_raw + 1), comp(nb * in.nqt * in.nkt_comp + 1);
  if (hca_plan_export_tiles(p, raw.data(), comp.data()) != HCA_OK) ++fails;
  std::vector<int32_t> rows(nb * in.S * 3);
  if (hca_plan_export_rows(p, rows.data()) != HCA_OK) ++fails;
  int64_t n = 0;
  if (hca_plan_export_items(p, nullptr, 0, &n) != HCA_OK) ++fails;
  std::vector<int64_t> items(n * 8 + 8);
  if (hca_plan_export_items(p, items.data(), n, &n) != HCA_OK) ++fails;
  hca_plan_destroy(p);
}

int main() {
  std::mt19937 rng(7);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int built = 0;
  // random configurations: every dtype / head dim, documents, modes, knobs
  for (int t = 0; t < 300; ++t) {
    const int B = uni(1, 3), S = uni(1, 1500), r = uni(1, 200), W = uni(0, 300);
    const int Hs[] = {1, 2, 4, 8, 16, 64, 128}, Ds[] = {64, 128, 512};
    const int H = Hs[uni(0, 6)], D = Ds[uni(0, 2)];
    const hca_dtype dt = uni(0, 1) ? HCA_BF16 : HCA_F32;
    const hca_compseg_mode mode = uni(0, 1) ? HCA_COMPSEG_LAST : HCA_COMPSEG_STRICT;
    std::vector<int32_t> starts, counts;
    const bool docs = uni(0, 1);
    for (int b = 0; b < B && docs; ++b) {
      int pos = 0, c = 0;
      while (pos < S) {
        starts.push_back(pos);
        ++c;
        pos += uni(1, S);
      }
      counts.push_back(c);
    }
    hca_tile_cfg cfg{0, 0, 0, uni(-1, 3), uni(0, 5)};
    hca_plan *p = nullptr;
    const int G = (H % 2 == 0 && uni(0, 1)) ? 2 : 1;
    hca_status s = G == 1 ? hca_block_mask_build(B, S, r, W, S / r, docs ? starts.data() : nullptr,
                                                 docs ? counts.data() : nullptr, H, D, dt, mode,
                                                 uni(0, 1) ? &cfg : nullptr, &p)
                          : hca_block_mask_build_gqa(B, G, S, r, W, S / r,
                                                     docs ? starts.data() : nullptr,
                                                     docs ? counts.data() : nullptr, H, D, dt,
                                                     mode, &cfg, &p);
    if (s != HCA_OK) { ++fails; continue; }
    exercise(p);
    ++built;
    // the same documents with a random compressed-key mask, and a top-k selection
    const int Sc = uni(1, 300);
    std::vector<uint8_t> mask((size_t)B * S * Sc);
    for (auto &m : mask) m = uni(0, 9) == 0;
    if (hca_block_mask_build_masked(B, S, W, Sc, docs ? starts.data() : nullptr,
                                    docs ? counts.data() : nullptr, H, D, dt, mask.data(), &cfg,
                                    &p) == HCA_OK) {
      exercise(p);
      ++built;
    } else {
      ++fails;
    }
    const int K = uni(1, 12);
    std::vector<int32_t> idx((size_t)B * S * K);
    for (auto &x : idx) x = uni(-2, Sc - 1);
    if (hca_block_mask_build_topk(B, S, W, Sc, docs ? starts.data() : nullptr,
                                  docs ? counts.data() : nullptr, H, D, dt, idx.data(), K, nullptr,
                                  &p) == HCA_OK) {
      exercise(p);
      ++built;
    } else {
      ++fails;
    }
  }
  // rejected arguments must not touch memory they do not own
  hca_plan *p = nullptr;
  int32_t bad_starts[] = {0, 5, 5}, bad_counts[] = {3};
  if (hca_block_mask_build(1, 10, 2, 3, 5, bad_starts, bad_counts, 4, 64, HCA_BF16,
                           HCA_COMPSEG_STRICT, nullptr, &p) != HCA_ERR_INVALID_ARG || p)
    ++fails;
  if (hca_block_mask_build(1, 0, 2, 3, 0, nullptr, nullptr, 4, 64, HCA_BF16, HCA_COMPSEG_STRICT,
                           nullptr, &p) != HCA_ERR_INVALID_ARG)
    ++fails;
  hca_plan_destroy(nullptr);
  std::printf("plans %d failures %d\n", built, fails);
  return fails ? 1 : 0;
}
