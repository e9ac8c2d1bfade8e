// hca_stage.h -- asynchronous staging of 32-key K/V tiles (D = 512) into LDS.
//
// Tiles move global -> LDS with buffer_load_dwordx4 ... lds: each wave
// instruction deposits 64 lanes x 16 B = 1 KiB contiguously at its LDS base
// (lane l at base + 16 l), bypassing VGPRs; the buffer range check returns
// zeros for rows past the end of the tensor.  Each lane chooses which global
// 16-byte chunk it fetches, so the tiles land in LDS in MFMA fragment order:
// every 1 KiB block is one A operand of v_mfma_f32_16x16x32_bf16, lane l's 8
// values at byte 16 l, and each operand read is a flat, conflict-free
// ds_read_b128 of 64 consecutive 16-byte pieces.
//
//   K tile   block 2 ks + h (k-step ks = 0..15, key half h = 0..1) holds, for
//            lane l = 16 g + j, key 8 (j >> 2) + (j & 3) + 4 h of the tile and
//            columns 32 ks + 8 g .. 32 ks + 8 g + 7.  With this key order the
//            S^T product leaves lane group g holding keys 8 g .. 8 g + 7 of its
//            query row, the B operand layout of the PV product.
//   K^T tile block db (16 d-rows) holds, for lane l = 16 g + j, d-row
//            16 db + j and keys 8 g .. 8 g + 7.
// Both orders are laid out in HBM by a small image kernel at the start of
// each call (gathering them per lane straight from the row-major tensor made
// every copy instruction touch 16 rows and ran far slower), so every copy
// instruction reads one contiguous KiB.
#pragma once

#include "hca_device.h"

namespace hca {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

constexpr int kTileBytes512 = 32 * 1024;  // one K tile or one K^T tile at D = 512

// 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4, SGPR base +
// per-lane byte offset; lane l lands at LDS byte address lds + 16 l).  Issued
// from inline assembly on purpose: the compiler's wait-count pass treats an
// LDS-DMA in flight as aliasing every LDS read and would wait for it before
// each of them (and at every barrier), serialising the copy with the math it
// is meant to overlap.  Callers wait for these copies themselves with
// wait_all_loads() before the barrier that publishes the buffer.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(lds_void_t *)p;
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, not for its global loads (an ordinary __syncthreads() would also
// drain the tile copies in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer resource (4 dwords: base, stride 0, size in bytes, format word) over
// `bytes` bytes at `base`; loads at offsets past `bytes` return zeros.
typedef unsigned int rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return rsrc_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16-byte-per-lane buffer -> LDS copy (buffer_load_dwordx4 ... offen lds; lane
// l lands at LDS byte address lds + 16 l).  The whole offset is the per-lane
// operand (scalar offset 0), so the range check covers all of it.  Issued
// from inline assembly for the same reason as dma16 below.
__device__ __forceinline__ void buf_load16(rsrc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff),
               "s"(r), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Tile images at D = 512: per 32-key tile 64 KiB, the K tile in fragment order
// (32 KiB) followed by the K^T tile in fragment order (32 KiB), written by the
// image kernel at the start of each forward / backward call; tiles of the
// padding are zero.
constexpr int kImageBytes512 = 2 * kTileBytes512;

// Stages one half of the image of key tile k0 .. k0+31 (`part` 0: K, 1: K^T)
// into `buf` (32 KiB): each instruction copies one contiguous KiB, lane l's
// 16 bytes landing at buf + 1024 blk + 16 l.
template <int NW>
__device__ __forceinline__ void stage_img512(rsrc_t r, int k0, int part, char *buf, int wave,
                                             int lane) {
  static_assert(32 % NW == 0, "waves must divide the tile blocks");
  const int voff = (k0 / 32) * kImageBytes512 + part * kTileBytes512 + 16 * lane;
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int blk = wave * (32 / NW) + i;
    buf_load16(r, lds_addr(buf + blk * 1024), voff + blk * 1024);
  }
}

// Stores a wave's 16 output rows of 512 as bf16.  acc[db] is the transposed
// MFMA layout: lane (g, j) holds elements 16 db + 4 g + v (v = 0..3) of row j.
// The rows go through `buf` (16 KiB of LDS used by this wave only), with the
// 16-byte chunks of row r stored at chunk index c ^ r so both the scattered
// writes and the row reads are free of bank conflicts, and then leave as one
// fully coalesced 1 KiB store per row instead of 32 partial-line writes.
// row_ptr(r) gives the destination of row r, or nullptr to skip it; it must be
// wave-uniform.
template <typename RowPtr>
__device__ __forceinline__ void store_rows512(const floatx4 (&acc)[32], float mul, char *buf,
                                              int lane, RowPtr row_ptr) {
  const int g = lane >> 4, j = lane & 15;
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    ushort4 w;
    w.x = f2bf(acc[db][0] * mul);
    w.y = f2bf(acc[db][1] * mul);
    w.z = f2bf(acc[db][2] * mul);
    w.w = f2bf(acc[db][3] * mul);
    const int c = 2 * db + (g >> 1);
    *reinterpret_cast<ushort4 *>(buf + j * 1024 + ((c ^ j) << 4) + 8 * (g & 1)) = w;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // Rows in batches of four: four reads (one wait), then four stores.
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += 4) {
    const uint4 v0 = *reinterpret_cast<const uint4 *>(buf + (r0 + 0) * 1024 + ((lane ^ (r0 + 0)) << 4));
    const uint4 v1 = *reinterpret_cast<const uint4 *>(buf + (r0 + 1) * 1024 + ((lane ^ (r0 + 1)) << 4));
    const uint4 v2 = *reinterpret_cast<const uint4 *>(buf + (r0 + 2) * 1024 + ((lane ^ (r0 + 2)) << 4));
    const uint4 v3 = *reinterpret_cast<const uint4 *>(buf + (r0 + 3) * 1024 + ((lane ^ (r0 + 3)) << 4));
    bf16raw *d0 = row_ptr(r0 + 0), *d1 = row_ptr(r0 + 1), *d2 = row_ptr(r0 + 2),
            *d3 = row_ptr(r0 + 3);
    if (d0) *reinterpret_cast<uint4 *>(d0 + 8 * lane) = v0;
    if (d1) *reinterpret_cast<uint4 *>(d1 + 8 * lane) = v1;
    if (d2) *reinterpret_cast<uint4 *>(d2 + 8 * lane) = v2;
    if (d3) *reinterpret_cast<uint4 *>(d3 + 8 * lane) = v3;
  }
}

typedef short shortx4 __attribute__((ext_vector_type(4)));

// Transposed A operand of an MFMA from two ds_read_b64_tr_b16 reads: the
// second read is `four_rows` bytes after the first (four rows further down a
// row-major LDS tile).
__device__ __forceinline__ bf16x8 tr_frag_rows(const char *p, int four_rows) {
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4 *)(p));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4 *)(p + four_rows));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A 32-key tile of the row-major K = V tensor at head dim D (64 or 128) in
// LDS, for kernels of NT threads: rows unpadded, the 16-byte chunk c of row r
// at slot c ^ sw(r), sw(r) = (r & 3) | ((r >> 3) & 3) << 2 (within the row's
// D / 8 chunks).  Both MFMA operands come from this one copy: the K
// A-operand of S^T = K Q^T as flat 16-byte reads (the eight rows a read
// instruction touches fall in distinct bank groups), and the K^T A-operand of
// a product over keys (O^T += K^T P^T, dQ^T += K^T dS^T) as two transpose
// reads, so no transposed copy of K is staged.
template <int D, int NT>
struct KTile {
  static constexpr int NCH = D / 8;  // 16-byte chunks per row
  static constexpr int KCH = 32 * NCH;
  static constexpr int KPT = (KCH + NT - 1) / NT;
  __device__ __forceinline__ static int sw(int r) { return ((r & 3) | (((r >> 3) & 3) << 2)) & (NCH - 1); }
  // Rows k0 .. k0 + 31 of src (nk rows; zero past the end) into registers.
  __device__ __forceinline__ static void load(uint4 (&pk)[KPT], int tid, const bf16raw *src,
                                              int nk, int k0) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / NCH, col = c % NCH;
        const int key = k0 + row;
        pk[u] = key < nk ? *reinterpret_cast<const uint4 *>(src + (size_t)key * D + col * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ static void store(const uint4 (&pk)[KPT], int tid, bf16raw *k_lds) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / NCH, col = c % NCH;
        *reinterpret_cast<uint4 *>(k_lds + row * D + (col ^ sw(row)) * 8) = pk[u];
      }
    }
  }
  // K A-operand for k-step ks: row `row` (16 keys of the tile: rows r0 and
  // r0 + 4 of lane (g, j)), columns 32 ks + 8 g .. + 7.
  __device__ __forceinline__ static bf16x8 kfrag(const bf16raw *k_lds, int row, int ks, int g) {
    return *reinterpret_cast<const bf16x8 *>(k_lds + row * D + ((4 * ks + g) ^ sw(row)) * 8);
  }
  // K^T A-operand of column block db: lane (g, j) gets column 16 db + j of
  // keys 8 g .. 8 g + 7.
  __device__ __forceinline__ static bf16x8 tfrag(const bf16raw *k_lds, int db, int g, int j) {
    const int tr_row = 8 * g + (j >> 2);  // rows tr_row + 4 share its swizzle
    const int off = tr_row * D * 2 + (((2 * db + ((j & 3) >> 1)) ^ sw(tr_row)) << 4) + (j & 1) * 8;
    return tr_frag_rows(reinterpret_cast<const char *>(k_lds) + off, 4 * D * 2);
  }
};

__device__ __forceinline__ bf16x8 lds_frag(const char *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// Cross-lane max / sum over lanes i ^ 16 and i ^ 32 (the four lane groups of a
// 16x16 MFMA output column) with the gfx950 permlane swaps.
__device__ __forceinline__ float group_max(float v) {
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  u = __float_as_uint(v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float group_sum(float v) {
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  u = __float_as_uint(v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace hca
