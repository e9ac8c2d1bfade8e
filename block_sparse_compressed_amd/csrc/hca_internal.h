// hca_internal.h -- host-side plan structure and kernel launcher declarations
// shared by the planner, the C-ABI shim and the HIP kernels.  Not installed.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "hca.h"

namespace hca {

// Query-tile schedule entry (one per non-empty (query tile, key tile) pair):
//   bit 31: key kind (0 raw, 1 compressed)   bit 30: tile is FULL
//   bits 0..29: key tile index
constexpr uint32_t kEntComp = 1u << 31;
constexpr uint32_t kEntFull = 1u << 30;
constexpr uint32_t kEntIdx = (1u << 30) - 1;

// Key-tile work item for the key-stationary backward kernel: the query tiles
// kv_ent[e0, e1) that see key tile `kt` (kv_bk keys) of kind `kind` in batch
// row `b`; the item's float32 partial gradient [kv_bk][D] is written at
// `part_off` floats into the partial area of the backward workspace.  An item
// that runs over one 64-key half of its tile (halves 1 or 2) writes that half
// of its block only when `shared` is set (another half item of the same tile
// writes the other half of the same block), and the whole block otherwise
// (zeros for the idle half).
struct KvItem {
  int32_t b, kind, kt, e0, e1;
  // 128-key items: bit 0 / bit 1 set when some row of the item sees a key of
  // the lower / upper 64 (3 for other key-tile widths, and whenever the
  // item runs over all keys of its tile).
  int16_t halves;
  int16_t shared;
  int64_t part_off;
};
static_assert(sizeof(KvItem) == 32, "KvItem layout");

// Byte offsets of the sections of the plan's device image (256-B aligned).
struct DevLayout {
  uint64_t rows = 0;     // int4 [B][S]: raw_lo, comp_lo, comp_hi, 0
  uint64_t qptr = 0;     // int32 [B*nqt + 1]
  uint64_t qent = 0;     // uint32 [n_qent]
  uint64_t qorder = 0;   // int32 [B*nqt]: query-tile launch order
  uint64_t kvitem = 0;   // KvItem [n_items] (tile-major)
  uint64_t kvorder = 0;  // int32 [n_items]: launch slot -> item, -1 = none
  uint64_t kvent = 0;    // uint32 [n_kvent]: bit 30 FULL, bits 0..29 query tile
  uint64_t kvtile = 0;   // int32 [B][nkv_raw + nkv_comp][2]: first partial block, block count
  uint64_t cmask = 0;    // uint32 [B][S][cmask_ldw]: compressed-key visibility bits (masked
                         // plans only)
  uint64_t kvpe = 0;     // int32 [n_kvent][2]: stored-P/dS blocks of the two 32-key halves
                         // of each key-tile entry (qent index, -1 = not listed; 64-key
                         // tiles at D = 512 only)
  uint64_t total = 0;
};

// Byte offsets inside the caller's workspaces.
struct WsLayout {
  uint64_t kvt = 0;     // raw kv tile images (bf16, D = 512 only): [B][S_pad/32][K | K^T
                        // fragments, 64 KiB]
  uint64_t kvct = 0;    // the same for compressed kv, Sc_pad entries
  uint64_t delta = 0;   // float32 [B][H][S] (backward)
  uint64_t part = 0;    // float32 partial key gradients (backward)
  uint64_t pds = 0;     // bf16 P and dS per query-tile entry e: [e][P | dS][bq * H rows]
                        // [32 keys], chunks swizzled (64-key tiles at D = 512 only)
  uint64_t pds_bytes = 0;
  uint64_t f32_part = 0;  // float32 plans: partial dKV of the compressed entries'
                          // split workgroups, [B][Sc][f32_split][D]
  uint64_t fwd_total = 0;
  uint64_t bwd_total = 0;
};

// Parameters every kernel receives (by value).
struct Dims {
  int32_t B, S, H, D, r, W, Sc;
  int32_t bq, bk_raw, bk_comp, nqt, nkt_raw, nkt_comp;
  int32_t S_pad, Sc_pad;  // nkt_raw * bk_raw, nkt_comp * bk_comp
  int32_t n_items;       // launch slots of the key-stationary backward
  int32_t kv_bk, nkv_raw, nkv_comp;  // key tiles of the key-stationary backward
  int32_t cmask_ldw;  // words per position of the compressed-key mask; 0: interval rule
  int32_t pds_rows;   // rows per stored P/dS block (bq * H); 0: dKV recomputes S and dP
  int32_t f32_split;  // float32 dKV: workgroups per compressed entry (1: one)
};

struct DevPlan {
  const int32_t *rows;  // int4 per position
  const int32_t *qptr;
  const uint32_t *qent;
  const int32_t *qorder;
  const KvItem *kvitem;
  const int32_t *kvorder;
  const uint32_t *kvent;
  const int32_t *kvtile;
  const uint32_t *cmask;  // masked plans: visibility bits of compressed keys
  const int32_t *kvpe;    // stored-P/dS plans: qent index of each kvent's two halves
};

// Launchers (defined in the .hip files).  Each returns a hipError_t as int.
// launch_transpose_kv writes the D = 512 tile images (other head dims: an
// error; their kernels stage the row-major tensor).
int launch_transpose_kv(const void *kv, void *kvt, int N, int N_pad, const void *kvc,
                        void *kvct, int Nc, int Nc_pad, int B, int D, void *stream);
int launch_fwd_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kv,
                    const void *kvc, const void *kvt, const void *kvct, float scale, void *o,
                    float *lse, void *stream);
int launch_bwd_dq_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kv,
                       const void *kvc, const void *kvt, const void *kvct, const void *o,
                       const float *lse, const void *dout, float scale, void *dq, float *delta,
                       void *pds, void *stream);
// Stored-P plans: the P / dS pass (launch_bwd_dq_bf16 then runs the streaming
// dQ pass from the stored dS).
int launch_bwd_pds_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kvt,
                        const void *kvct, const void *o, const float *lse, const void *dout,
                        float scale, float *delta, void *pds, void *stream);
int launch_bwd_dkv_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kv,
                        const void *kvc, const float *lse, const float *delta,
                        const void *dout, float scale, const void *pds, float *part,
                        void *stream);
int launch_dkv_reduce(const Dims &d, const DevPlan &p, const float *part, int dtype, void *dkv,
                      void *dkvc, void *stream);
int launch_fwd_f32(const Dims &d, const DevPlan &p, const float *q, const float *kv,
                   const float *kvc, float scale, float *o, float *lse, void *stream);
// f32_part: the workspace section of that name (used when d.f32_split > 1).
int launch_bwd_f32(const Dims &d, const DevPlan &p, const float *q, const float *kv,
                   const float *kvc, const float *o, const float *lse, const float *dout,
                   float scale, float *dq, float *dkv, float *dkvc, float *delta,
                   float *f32_part, void *stream);

// Scratch of the allocation-free forward: a file-scope device array in
// hca_fwd.hip of this many bytes (the limit hca.h states).
constexpr uint64_t kNoAllocScratchBytes = HCA_NOALLOC_SCRATCH_BYTES;
void *noalloc_scratch(int *err);

// Tile shapes the GPU kernels are built for ("" = supported, else the reason).
std::string kernel_supports(int dtype, int D, int H, int bq, int bk_raw, int bk_comp);
// Sizes the kernels' 32-bit offsets can address ("" = fine, else the reason).
std::string kernel_sizes_ok(int dtype, int D, int64_t S_pad, int64_t Sc_pad);
void default_tiles(int dtype, int D, int H, int *bq, int *bk_raw, int *bk_comp);

void set_error(const std::string &msg);

}  // namespace hca

struct hca_plan {
  hca_plan_info info{};
  std::vector<int32_t> rows;  // [B][S][4]
  std::vector<int32_t> qptr;
  std::vector<uint32_t> qent;
  std::vector<int32_t> qorder;
  std::vector<hca::KvItem> kvitem;
  std::vector<int32_t> kvorder;  // launch slots (-1 = none)
  std::vector<uint32_t> kvent;
  std::vector<int32_t> kvtile;
  std::vector<int32_t> kvpe;  // stored-P/dS plans: [n_kvent][2]
  int32_t kv_bk = 32, nkv_raw = 0, nkv_comp = 0;  // key-stationary backward tiling
  int32_t rows_b = 0;  // rows of the plan's tables: batch rows x kv heads
  int32_t cmask_ldw = 0;  // masked plans: words per position of the device mask
  int32_t pds_rows = 0;   // stored-P/dS plans: rows per stored block (bq * H)
  int32_t f32_split = 1;  // float32 plans: dKV workgroups per compressed entry
  hca::DevLayout lay;
  hca::WsLayout ws;
  std::string unsupported;     // why kernel_ok is 0 ("" when it is 1)
  std::vector<uint8_t> image;  // the device image, built once
  void *dev = nullptr;         // caller's device buffer after upload
};
