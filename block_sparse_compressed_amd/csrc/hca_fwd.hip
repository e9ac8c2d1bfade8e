// hca_fwd.hip -- HCA attention forward on gfx950 (bf16 MFMA, fp32 accumulation).
//
// A query tile is bq positions x all H heads (single KV head, so every head of
// a position sees the same keys; the shared-KV einsum form of "[DeepSeek-V4]
// Implement Compressed Attention Layers", review suggestions); a workgroup
// owns the tile (D = 64 / 128: 128 rows) or a slice of it (D = 512: 64 rows of
// a 16-position x 64-head tile).  It walks the tile's list of non-empty key
// tiles from the host-built block table (EMPTY tiles never appear; "Add HCA
// Static Compilation for Splash Attention [Deepseek v4]", Description), stages
// each 32-key tile of the shared K = V tensor in LDS once for all heads, and
// runs
//   S^T = K Q^T      (v_mfma_f32_16x16x32_bf16, Q fragments held in VGPRs)
//   online softmax   (PARTIAL tiles masked in registers from per-row intervals)
//   O^T += K^T P^T   (P rounded to bf16, K^T read from a transposed LDS copy)
// Computing S transposed leaves each lane holding one query row and 8
// consecutive keys, which is exactly the B operand layout the PV product
// needs, so P never goes through LDS.
#include <climits>
#include <mutex>

#include "hca_device.h"
#include "hca_internal.h"
#include "hca_stage.h"

namespace hca {

constexpr int kBK = 32;  // keys per tile (raw and compressed)

#ifndef HCA_FWD_NW
#define HCA_FWD_NW 4  // waves of the D = 512 forward: 4 (two workgroups per CU) or 8
#endif
#ifndef HCA_FWD_MB
#define HCA_FWD_MB 1  // 16-row blocks per wave of the D = 512 forward
#endif
#ifndef HCA_FWD_QK_PF
#define HCA_FWD_QK_PF 3  // k-steps of K fragments in flight ahead of the S^T MFMAs
#endif
#ifndef HCA_FWD_PV_PF
#define HCA_FWD_PV_PF 4  // column blocks of K^T fragments in flight ahead of the PV MFMAs
#endif


// K tile chunks: BK rows x D; transposed tile chunks: D rows x BK.  16 B each.
template <int D, int NT>
struct Stage {
  static constexpr int KROW = D + 8;    // padded LDS row of the K tile (bf16)
  static constexpr int TROW = kBK + 8;  // padded LDS row of the transposed tile
  static constexpr int KCH = kBK * D / 8;
  static constexpr int TCH = D * kBK / 8;
  static constexpr int KPT = (KCH + NT - 1) / NT;
  static constexpr int TPT = (TCH + NT - 1) / NT;

  __device__ __forceinline__ static void load(uint4 (&pk)[KPT], uint4 (&pt)[TPT], int tid,
                                              const bf16raw *src, int nk, const bf16raw *srct,
                                              int ts, int k0) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / (D / 8), col = c % (D / 8);
        const int key = k0 + row;
        pk[u] = key < nk ? *reinterpret_cast<const uint4 *>(src + (size_t)key * D + col * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int c = tid + u * NT;
      if (TCH % NT == 0 || c < TCH) {
        const int dd = c / (kBK / 8), col = c % (kBK / 8);
        pt[u] = *reinterpret_cast<const uint4 *>(srct + (size_t)k0 * D + dd * kBK + col * 8);
      }
    }
  }

  __device__ __forceinline__ static void store(const uint4 (&pk)[KPT], const uint4 (&pt)[TPT],
                                               int tid, bf16raw *k_lds, bf16raw *t_lds) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / (D / 8), col = c % (D / 8);
        *reinterpret_cast<uint4 *>(k_lds + row * KROW + col * 8) = pk[u];
      }
    }
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int c = tid + u * NT;
      if (TCH % NT == 0 || c < TCH) {
        const int dd = c / (kBK / 8), col = c % (kBK / 8);
        *reinterpret_cast<uint4 *>(t_lds + dd * TROW + col * 8) = pt[u];
      }
    }
  }
};

template <int D, int NW, int MB>
__global__ void __launch_bounds__(NW * 64, 1)
    hca_fwd_bf16_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                        const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                        const bf16raw *__restrict__ kvt, const bf16raw *__restrict__ kvct,
                        float scale_log2, bf16raw *__restrict__ o, float *__restrict__ lse) {
  constexpr int NT = NW * 64;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  using St = Stage<D, NT>;
  __shared__ __attribute__((aligned(16))) bf16raw k_lds[kBK * St::KROW];
  __shared__ __attribute__((aligned(16))) bf16raw t_lds[D * St::TROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int nitems = d.B * d.nqt;
  const int item = p.qorder[xcd_remap(blockIdx.x, nitems)];
  const int b = item / d.nqt, qt = item - b * d.nqt;

  int pos[MB], hh[MB], rlo[MB], clo[MB], chi[MB];
  bool valid[MB];
  bf16x8 qf[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rho = (wave * MB + mb) * 16 + j;
    pos[mb] = qt * d.bq + rho / d.H;
    hh[mb] = rho % d.H;
    valid[mb] = pos[mb] < d.S;
    if (valid[mb]) {
      const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pos[mb]];
      rlo[mb] = rw.x;
      clo[mb] = rw.y;
      chi[mb] = rw.z;
    } else {
      rlo[mb] = INT_MAX;
      clo[mb] = 0;
      chi[mb] = 0;
    }
    const bf16raw *qrow = q + (((size_t)b * d.H + hh[mb]) * d.S + pos[mb]) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[mb][ks] = valid[mb] ? as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * g))
                             : as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  float m_run[MB], l_run[MB];
  floatx4 oacc[MB][DB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = -INFINITY;
    l_run[mb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[mb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int e_begin = p.qptr[item], e_end = p.qptr[item + 1];
  const bf16raw *kv_b = kv + (size_t)b * d.S * D;
  const bf16raw *kvc_b = kvc + (size_t)b * d.Sc * D;
  const bf16raw *kvt_b = kvt + (size_t)b * D * d.S_pad;
  const bf16raw *kvct_b = kvct + (size_t)b * D * d.Sc_pad;

  uint4 pk[St::KPT], pt[St::TPT];
  auto issue = [&](int e) {
    const uint32_t ent = p.qent[e];
    const bool comp = ent & kEntComp;
    const int k0 = (int)(ent & kEntIdx) * kBK;
    St::load(pk, pt, tid, comp ? kvc_b : kv_b, comp ? d.Sc : d.S, comp ? kvct_b : kvt_b,
             comp ? d.Sc_pad : d.S_pad, k0);
  };
  if (e_begin < e_end) issue(e_begin);

  // A-operand rows of the two 16-key halves: lane group g ends up holding
  // keys 8g .. 8g+7 of the 32-key tile for its query row.
  const int r0 = 8 * (j >> 2) + (j & 3), r1 = r0 + 4;

  for (int e = e_begin; e < e_end; ++e) {
    const uint32_t ent = p.qent[e];
    const bool comp = ent & kEntComp;
    const bool full = ent & kEntFull;
    const int k0 = (int)(ent & kEntIdx) * kBK;
    __syncthreads();
    St::store(pk, pt, tid, k_lds, t_lds);
    __syncthreads();
    if (e + 1 < e_end) issue(e + 1);

    floatx4 s0[MB], s1[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s0[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      s1[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a0 = as_bf16x8(lds_load16(k_lds + r0 * St::KROW + 32 * ks + 8 * g));
      const bf16x8 a1 = as_bf16x8(lds_load16(k_lds + r1 * St::KROW + 32 * ks + 8 * g));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s0[mb] = mfma16x16x32(a0, qf[mb][ks], s0[mb]);
        s1[mb] = mfma16x16x32(a1, qf[mb][ks], s1[mb]);
      }
    }

    bf16x8 pb[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float x[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[v] = s0[mb][v] * scale_log2;
        x[4 + v] = s1[mb][v] * scale_log2;
      }
      if (!full) {
        const int kb = k0 + 8 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int key = kb + t;
          const bool vis = comp ? (key >= clo[mb] && key < chi[mb])
                                : (key >= rlo[mb] && key <= pos[mb]);
          if (!vis) x[t] = -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int t = 1; t < 8; ++t) mx = fmaxf(mx, x[t]);
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const float m_new = fmaxf(m_run[mb], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[mb] - m_use);
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[t] = fast_exp2(x[t] - m_use);
        ps += x[t];
      }
      l_run[mb] = l_run[mb] * alpha + ps;
      m_run[mb] = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[mb][db] *= alpha;
      pb[mb] = pack8(x);
    }

#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = as_bf16x8(lds_load16(t_lds + (16 * db + j) * St::TROW + 8 * g));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][db] = mfma16x16x32(a, pb[mb], oacc[mb][db]);
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float l = l_run[mb];
    l = xor_sum(l, 16);
    l = xor_sum(l, 32);
    if (valid[mb]) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      bf16raw *orow = o + (((size_t)b * d.H + hh[mb]) * d.S + pos[mb]) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        ushort4 w;
        w.x = f2bf(oacc[mb][db][0] * inv);
        w.y = f2bf(oacc[mb][db][1] * inv);
        w.z = f2bf(oacc[mb][db][2] * inv);
        w.w = f2bf(oacc[mb][db][3] * inv);
        *reinterpret_cast<ushort4 *>(orow + 16 * db + 4 * g) = w;
      }
      if (g == 0)
        lse[((size_t)b * d.H + hh[mb]) * d.S + pos[mb]] =
            l > 0.f ? (m_run[mb] + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// D = 512 forward: NW waves x 16 rows per workgroup (one wave = 16 consecutive
// positions of one head).
//
// NW = 4 (the default): 64 rows, two workgroups per CU, K and K^T tiles
// single-buffered (32 KiB each).  Per tile: softmax and O^T += K^T P^T of tile
// t (K of tile t+1 arriving meanwhile), barrier, copy K^T of tile t+1 while
// S^T = K Q^T of tile t+1 runs, barrier, copy K of tile t+2.  The second
// workgroup on the CU fills this one's waits and its row loads.
// NW = 8: 128 rows, one workgroup per CU, K and K^T double-buffered and one
// tile apart (4 x 32 KiB), one barrier per tile, the S^T MFMAs of tile t+1
// issued before the softmax and PV of tile t.
// Tiles go global -> LDS directly (no VGPR staging) from the tile images, in
// MFMA fragment order, so every operand read is a flat ds_read_b128.
// ---------------------------------------------------------------------------
// Lazy rescaling: a row's reference max m_run only moves when the tile max
// exceeds it by more than kLazy (log2 units), so P = 2^(x - m_run) stays below
// 2^kLazy and the O rescale (a wave-uniform branch) is rare.
constexpr float kLazy = 8.f;

// NW = 8: one workgroup per CU, K and K^T double-buffered (128 KiB of LDS).
// NW = 4: two workgroups per CU, K and K^T single-buffered (64 KiB each), so
// one workgroup's row loads, barriers and tile waits overlap the other's math.
// MASKED: compressed visibility from the plan's mask bits (masked plans);
// otherwise from the per-position intervals.  Separate instantiations, so the
// interval kernel carries none of the mask code.
template <int NW, int MB, bool MASKED>
__global__ void __launch_bounds__(NW * 64, 8 / NW)
    hca_fwd512_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                      const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                      const bf16raw *__restrict__ kvt, const bf16raw *__restrict__ kvct,
                      float scale_log2, bf16raw *__restrict__ o, float *__restrict__ lse) {
  constexpr int D = 512, KS = D / 32, DB = D / 16;
  constexpr int M = NW * MB * 16;  // rows per workgroup
  // [K buffer 0][K buffer 1][K^T buffer 0][K^T buffer 1]
  constexpr bool kSingle = NW == 4;
  constexpr int kBufs = kSingle ? 1 : 2;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufs * kTileBytes512];
  char *const kbase = smem;
  char *const tbase = smem + kBufs * kTileBytes512;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  // A query tile is bq positions x H heads, rows ordered position-fastest
  // (row rho = position rho % bq, head rho / bq), cut into slices of M rows;
  // one wave's 16 rows are 16 consecutive positions of one head.  The slices
  // of two neighbouring tiles run back to back on one XCD.
  const int nslices = d.bq * d.H / M;
  const int lbq = __builtin_ctz(d.bq);
  const int u = xcd_remap(blockIdx.x, d.B * d.nqt * nslices, 2 * nslices);
  const int li = u / nslices, sl = u - li * nslices;
  const int item = p.qorder[li];
  const int b = item / d.nqt, qt = item - b * d.nqt;

  int pos[MB], hh[MB], rlo[MB], clo[MB], chi[MB];
  bool valid[MB];
  bf16x8 qf[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rho = sl * M + (wave * MB + mb) * 16 + j;
    pos[mb] = qt * d.bq + (rho & (d.bq - 1));
    hh[mb] = rho >> lbq;
    valid[mb] = pos[mb] < d.S;
    rlo[mb] = INT_MAX;
    clo[mb] = chi[mb] = 0;
  }

  const int e_begin = p.qptr[item], nent = p.qptr[item + 1] - e_begin;
  // The tile's list, one entry per lane: entries are fetched with readlane,
  // not with a dependent memory load per tile (lists longer than 64 fall back
  // to memory for the tail).  They are needed for the first tile copies: load
  // them first and wait for them once, before any copy is in flight.
  const uint32_t ent_lane = lane < nent ? p.qent[e_begin + lane] : 0u;
  __builtin_amdgcn_s_waitcnt(0);
  auto entry = [&](int t) -> uint32_t {
    return t < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)ent_lane, t)
                  : uniform_load(p.qent, e_begin + t);
  };
  // K and K^T tiles come from the tile images (kvt, kvct) that the image
  // kernel wrote at the start of the call.
  const rsrc_t r_img =
      make_rsrc(kvt + (size_t)b * 2 * D * d.S_pad, (uint32_t)d.S_pad * D * 4);
  const rsrc_t r_imgc =
      make_rsrc(kvct + (size_t)b * 2 * D * d.Sc_pad, (uint32_t)d.Sc_pad * D * 4);
  auto stage_k = [&](int t) {  // K of list entry t
    if (t >= nent) return;
    const uint32_t ent = entry(t);
    stage_img512<NW>((ent & kEntComp) ? r_imgc : r_img, (int)(ent & kEntIdx) * kBK, 0,
                     kbase + (t & (kBufs - 1)) * kTileBytes512, wave, lane);
  };
  auto stage_t = [&](int t) {  // K^T of list entry t
    if (t >= nent) return;
    const uint32_t ent = entry(t);
    stage_img512<NW>((ent & kEntComp) ? r_imgc : r_img, (int)(ent & kEntIdx) * kBK, 1,
                     tbase + (t & (kBufs - 1)) * kTileBytes512, wave, lane);
  };

  // Operand reads are flat: lane l reads bytes 16 l .. 16 l + 15 of a block.
  const int frag_off = 16 * lane;

  // S^T of tile t for every row block: two 16-key halves per block.
  // Operand fragments are read QK_PF k-steps ahead of their MFMAs (the
  // group barriers keep the compiler from collapsing the distance), so each
  // MFMA finds its operand landed instead of waiting out an LDS round trip.
  auto qk = [&](int t, floatx4 (&s)[MB][2]) {
    constexpr int PF = HCA_FWD_QK_PF;
    const char *kb = kbase + (t & (kBufs - 1)) * kTileBytes512 + frag_off;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) s[mb][0] = s[mb][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 a0[KS], a1[KS];
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) {
      a0[ks] = lds_frag(kb + 2048 * ks);
      a1[ks] = lds_frag(kb + 2048 * ks + 1024);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) {
        a0[ks + PF] = lds_frag(kb + 2048 * (ks + PF));
        a1[ks + PF] = lds_frag(kb + 2048 * (ks + PF) + 1024);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb][0] = mfma16x16x32(a0[ks], qf[mb][ks], s[mb][0]);
        s[mb][1] = mfma16x16x32(a1[ks], qf[mb][ks], s[mb][1]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * MB, 0);
    }
  };

  float m_run[MB], l_run[MB];
  floatx4 oacc[MB][DB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = -INFINITY;
    l_run[mb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[mb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // Query rows and their key intervals.  All loads are unconditional (a padded
  // row, pos >= S, reads the last row): issued back to back, waited for once.
  // A padded row's interval is empty and a tile holding it is never FULL, so
  // it contributes nothing, and it is never stored.
  auto load_q = [&]() {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int pc = min(pos[mb], d.S - 1);
      const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pc];
      rlo[mb] = valid[mb] ? rw.x : INT_MAX;
      clo[mb] = valid[mb] ? rw.y : 0;
      chi[mb] = valid[mb] ? rw.z : 0;
      const bf16raw *qrow = q + (((size_t)b * d.H + hh[mb]) * d.S + pc) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[mb][ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * g));
    }
  };
  // Masked plans (compressed visibility from a given mask): the 32 visibility
  // bits of each row for the compressed tile of entry `ent`, loaded when the
  // entry becomes current, one tile ahead of their use (0 otherwise).
  uint32_t mword[MB];
  auto load_mask = [&](uint32_t ent) {
    if constexpr (MASKED) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        mword[mb] = 0u;
        if ((ent & kEntComp) && !(ent & kEntFull) && valid[mb])
          mword[mb] = p.cmask[((size_t)b * d.S + pos[mb]) * d.cmask_ldw + (ent & kEntIdx)];
      }
    }
  };
  // Online softmax of tile `it` (scores sc, list entry ent) and O^T += K^T P^T.
  auto soft_pv = [&](int it, const floatx4 (&sc)[MB][2], uint32_t ent) {
    const bool comp = ent & kEntComp;
    const int k0 = (int)(ent & kEntIdx) * kBK;
    bf16x8 pb[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float x[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[v] = sc[mb][0][v] * scale_log2;
        x[4 + v] = sc[mb][1][v] * scale_log2;
      }
      if (!(ent & kEntFull)) {
        if (MASKED && comp) {
          // this lane's 8 keys: bits 8 g .. 8 g + 7 of the row's tile word
          const uint32_t bits = mword[mb] >> (8 * g);
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = ((bits >> t) & 1u) ? x[t] : -INFINITY;
        } else {
          // visible keys of this row: [lo, hi) relative to this lane's 8 keys
          const int lo = (comp ? clo[mb] : rlo[mb]) - (k0 + 8 * g);
          const int hi = (comp ? chi[mb] : pos[mb] + 1) - (k0 + 8 * g);
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = (t >= lo && t < hi) ? x[t] : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = group_max(mx);
      const bool up = mx > m_run[mb] + kLazy;
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float m_new = up ? mx : m_run[mb];
        const float alpha = fast_exp2(m_run[mb] - (m_new == -INFINITY ? 0.f : m_new));
        l_run[mb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[mb][db] *= alpha;
        m_run[mb] = m_new;
      }
      const float m_use = m_run[mb] == -INFINITY ? 0.f : m_run[mb];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[t] = fast_exp2(x[t] - m_use);
        l_run[mb] += x[t];
      }
      pb[mb] = pack8(x);
    }
    // K^T fragments read PV_PF column blocks ahead of their MFMAs.
    constexpr int PV = HCA_FWD_PV_PF;
    const char *tb = tbase + (it & (kBufs - 1)) * kTileBytes512 + frag_off;
    bf16x8 kt[DB];
#pragma unroll
    for (int db = 0; db < PV; ++db) kt[db] = lds_frag(tb + db * 1024);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db + PV < DB) kt[db + PV] = lds_frag(tb + (db + PV) * 1024);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][db] = mfma16x16x32(kt[db], pb[mb], oacc[mb][db]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, PV, 0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db + PV < DB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MB, 0);
    }
  };

  if constexpr (!kSingle) {
    // Double-buffered: K runs two tiles ahead, K^T one; S of tile t+1 is
    // issued before the softmax and PV of tile t; one barrier per tile.
    // First tile copies go out before the query-row loads, so the two
    // latencies overlap.
    stage_k(0);
    stage_k(1);
    stage_t(0);
    load_q();
    wait_all_loads();
    __syncthreads();
    floatx4 sc[MB][2];
    if (nent > 0) qk(0, sc);
    __syncthreads();
    stage_k(2);
    stage_t(1);

    // List entries are read only right after the barrier (where a wait for a
    // scalar load costs nothing): ent holds the entry of the current tile.
    uint32_t ent = nent > 0 ? entry(0) : 0u;
    load_mask(ent);
    for (int it = 0; it < nent; ++it) {
      floatx4 sn[MB][2];
      if (it + 1 < nent) qk(it + 1, sn);
      soft_pv(it, sc, ent);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        sc[mb][0] = sn[mb][0];
        sc[mb][1] = sn[mb][1];
      }
      wait_all_loads();
      __syncthreads();
      if (it + 1 < nent) {
        ent = entry(it + 1);
        load_mask(ent);
      }
      stage_k(it + 3);
      stage_t(it + 2);
    }
  } else {
    // Single-buffered: the copy of K for tile t+1 overlaps the softmax and PV
    // of tile t, the copy of K^T for tile t+1 overlaps S of tile t+1; two
    // barriers per tile.  The second workgroup on the CU covers the rest.
    stage_k(0);
    stage_t(0);
    load_q();
    wait_all_loads();
    __syncthreads();
    floatx4 sc[MB][2];
    if (nent > 0) qk(0, sc);
    __syncthreads();  // K buffer free
    stage_k(1);
    uint32_t ent = nent > 0 ? entry(0) : 0u;
    load_mask(ent);
    for (int it = 0; it < nent; ++it) {
      soft_pv(it, sc, ent);
      wait_all_loads();  // K of tile it + 1
      __syncthreads();   // K^T buffer free, K of tile it + 1 visible
      if (it + 1 < nent) {
        ent = entry(it + 1);
        load_mask(ent);
        stage_t(it + 1);
        qk(it + 1, sc);
        wait_all_loads();  // K^T of tile it + 1
        __syncthreads();   // K buffer free, K^T of tile it + 1 visible
        stage_k(it + 2);
      }
    }
  }

  // The tile buffers are free (the loop ended on a barrier with no copy in
  // flight): each 16-row block is staged there and stored as whole rows.
  static_assert(NW * MB * 16384 <= 2 * kBufs * kTileBytes512, "row staging fits the tiles");
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float l = group_sum(l_run[mb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    store_rows512(oacc[mb], inv, smem + (wave * MB + mb) * 16384, lane, [&](int r) -> bf16raw * {
      const int rr = sl * M + (wave * MB + mb) * 16 + r;
      const int pr = qt * d.bq + (rr & (d.bq - 1)), hr = rr >> lbq;
      return pr < d.S ? o + (((size_t)b * d.H + hr) * d.S + pr) * D : nullptr;
    });
    if (valid[mb] && g == 0)
      lse[((size_t)b * d.H + hh[mb]) * d.S + pos[mb]] =
          l > 0.f ? (m_run[mb] + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// One key tensor and its workspace copy (raw kv or compressed kv): N keys,
// N_pad after padding to whole tiles.
struct KvCopy {
  const bf16raw *src;
  bf16raw *dst;
  int N, N_pad;
};

// Tile-major transpose: dst[b][t / 32][d][t % 32] = src[b][t][d] for t < N, 0 for
// N <= t < N_pad (N_pad a multiple of 32).  Each 32-key tile's transpose is one
// contiguous D x 32 block, so a kernel stages it with contiguous copies.  One
// launch covers the raw keys (blockIdx.x < ceil(raw.N_pad / 64)), then the
// compressed ones.
__global__ void __launch_bounds__(256) hca_transpose_kernel(KvCopy raw, KvCopy cmp, int D) {
  __shared__ bf16raw tile[64][66];
  const int nraw = (raw.N_pad + 63) / 64;
  const bool second = (int)blockIdx.x >= nraw;
  const KvCopy k = second ? cmp : raw;
  const int N = k.N, N_pad = k.N_pad;
  const int b = blockIdx.z, t0 = (second ? blockIdx.x - nraw : blockIdx.x) * 64,
            d0 = blockIdx.y * 64;
  const bf16raw *s = k.src + (size_t)b * N * D;
  bf16raw *o = k.dst + (size_t)b * D * N_pad;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int tt = i / 64, dd = i % 64, t = t0 + tt, dx = d0 + dd;
    tile[tt][dd] = (t < N && dx < D) ? s[(size_t)t * D + dx] : (bf16raw)0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int dd = i / 64, tt = i % 64, t = t0 + tt, dx = d0 + dd;
    if (dx < D && t < N_pad) o[(size_t)(t / kBK) * D * kBK + (size_t)dx * kBK + t % kBK] = tile[tt][dd];
  }
}

// Tile images at D = 512: dst[b][t] (64 KiB) = the K tile t (keys 32 t ..
// 32 t + 31, zero past N) in MFMA fragment order, then its transpose in
// fragment order (block and lane layout as the D = 512 kernels read them).
// One workgroup per tile: the tile goes through LDS once, both orders are
// written as contiguous 16-byte pieces.  One launch covers the raw tiles
// (blockIdx.x < raw.N_pad / 32) and then the compressed ones.
__global__ void __launch_bounds__(256) hca_image512_kernel(KvCopy raw, KvCopy cmp) {
  constexpr int D = 512, PITCH = D + 8;
  __shared__ __attribute__((aligned(16))) bf16raw tile[32 * PITCH];
  const int nraw = raw.N_pad / 32;
  const bool second = (int)blockIdx.x >= nraw;
  const KvCopy k = second ? cmp : raw;
  const int b = blockIdx.y, t = second ? blockIdx.x - nraw : blockIdx.x;
  const int N = k.N;
  const bf16raw *s = k.src + (size_t)b * N * D;
  uint4 *out =
      reinterpret_cast<uint4 *>(k.dst + ((size_t)b * k.N_pad + (size_t)t * 32) * 2 * D);
  for (int c = threadIdx.x; c < 32 * D / 8; c += 256) {
    const int key = c / (D / 8), col = (c % (D / 8)) * 8, gk = t * 32 + key;
    *reinterpret_cast<uint4 *>(tile + key * PITCH + col) =
        gk < N ? *reinterpret_cast<const uint4 *>(s + (size_t)gk * D + col)
               : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  // Block blk, lane l = 16 g + j.  K: k-step blk / 2, key half blk % 2, key
  // 8 (j / 4) + j % 4 + 4 (blk % 2), columns 32 (blk / 2) + 8 g ...; K^T:
  // d-row 16 blk + j, keys 8 g ... 8 g + 7.
  for (int c = threadIdx.x; c < 2048; c += 256) {
    const int blk = c >> 6, l = c & 63, j = l & 15, g = l >> 4;
    const int key = 8 * (j >> 2) + (j & 3) + 4 * (blk & 1);
    out[c] = *reinterpret_cast<const uint4 *>(tile + key * PITCH + 32 * (blk >> 1) + 8 * g);
    const int dc = 16 * blk + j;
    ushort4 lo, hi;
    lo.x = tile[(8 * g + 0) * PITCH + dc];
    lo.y = tile[(8 * g + 1) * PITCH + dc];
    lo.z = tile[(8 * g + 2) * PITCH + dc];
    lo.w = tile[(8 * g + 3) * PITCH + dc];
    hi.x = tile[(8 * g + 4) * PITCH + dc];
    hi.y = tile[(8 * g + 5) * PITCH + dc];
    hi.z = tile[(8 * g + 6) * PITCH + dc];
    hi.w = tile[(8 * g + 7) * PITCH + dc];
    out[2048 + c] = make_uint4(lo.x | ((unsigned)lo.y << 16), lo.z | ((unsigned)lo.w << 16),
                               hi.x | ((unsigned)hi.y << 16), hi.z | ((unsigned)hi.w << 16));
  }
}

int launch_transpose_kv(const void *kv, void *kvt, int N, int N_pad, const void *kvc,
                        void *kvct, int Nc, int Nc_pad, int B, int D, void *stream) {
  const KvCopy raw{(const bf16raw *)kv, (bf16raw *)kvt, N, N_pad};
  const KvCopy cmp{(const bf16raw *)kvc, (bf16raw *)kvct, Nc, kvc ? Nc_pad : 0};
  hipStream_t s = (hipStream_t)stream;
  if (D == 512) {
    if (raw.N_pad % 32 || cmp.N_pad % 32) return (int)hipErrorInvalidValue;
    const int tiles = raw.N_pad / 32 + cmp.N_pad / 32;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(hca_image512_kernel, dim3(tiles, B), dim3(256), 0, s, raw, cmp);
    return (int)hipGetLastError();
  }
  const int blocks = (raw.N_pad + 63) / 64 + (cmp.N_pad + 63) / 64;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(hca_transpose_kernel, dim3(blocks, (D + 63) / 64, B), dim3(256), 0, s, raw,
                     cmp, D);
  return (int)hipGetLastError();
}

int launch_fwd_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kv,
                    const void *kvc, const void *kvt, const void *kvct, float scale, void *o,
                    float *lse, void *stream) {
  const dim3 grid(d.B * d.nqt);
  const float sl2 = scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  auto args = [&](auto kernel, int nw) {
    hipLaunchKernelGGL(kernel, grid, dim3(nw * 64), 0, s, d, p, (const bf16raw *)q,
                       (const bf16raw *)kv, (const bf16raw *)kvc, (const bf16raw *)kvt,
                       (const bf16raw *)kvct, sl2, (bf16raw *)o, lse);
  };
  switch (d.D) {
    case 512: {
      constexpr int NW = HCA_FWD_NW, MB = HCA_FWD_MB;
      const dim3 g512(d.B * d.nqt * (d.bq * d.H / (NW * MB * 16)));
      auto go512 = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, g512, dim3(NW * 64), 0, s, d, p, (const bf16raw *)q,
                           (const bf16raw *)kv, (const bf16raw *)kvc, (const bf16raw *)kvt,
                           (const bf16raw *)kvct, sl2, (bf16raw *)o, lse);
      };
      if (d.cmask_ldw)
        go512(hca_fwd512_kernel<NW, MB, true>);
      else
        go512(hca_fwd512_kernel<NW, MB, false>);
      break;
    }
    case 128: args(hca_fwd_bf16_kernel<128, 8, 1>, 8); break;
    case 64: args(hca_fwd_bf16_kernel<64, 8, 1>, 8); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Library-held scratch of the allocation-free forward (hca_attn_fwd_noalloc):
// the tile images of the call's kv and kv_comp.  Each device the library runs
// on holds one copy until the process ends.  In host code `scratch` is only a
// stand-in for the symbol, never a device address: kernels receive the
// address hipGetSymbolAddress returns for the current device.
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, resolved once per device
// (nullptr and *err set if the device or the symbol cannot be queried).
void *noalloc_scratch(int *err) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void *addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  *err = 0;
  return addr[dev];
}

}  // namespace hca
