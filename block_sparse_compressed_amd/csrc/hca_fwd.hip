// hca_fwd.hip -- HCA attention forward on gfx950 (bf16 MFMA, fp32 accumulation).
//
// A query tile is bq positions x all H heads (single KV head, so every head of
// a position sees the same keys; the shared-KV einsum form of "[DeepSeek-V4]
// Implement Compressed Attention Layers", review suggestions); a workgroup
// owns the tile (D = 64 / 128: 128 rows) or a slice of it (D = 512: 128 rows
// of a 16-position x 64-head tile).  It walks the tile's list of non-empty key
// tiles from the host-built block table (EMPTY tiles never appear; "Add HCA
// Static Compilation for Splash Attention [Deepseek v4]", Description), stages
// each 32-key tile of the shared K = V tensor in LDS once for all heads, and
// runs
//   S^T = K Q^T      (v_mfma_f32_16x16x32_bf16, Q fragments held in VGPRs)
//   online softmax   (PARTIAL tiles masked in registers from per-row intervals)
//   O^T += K^T P^T   (P rounded to bf16; K^T fragments: at D = 512 from a
//                     transposed copy staged from the tile images, at D = 64 /
//                     128 by transpose reads of the one staged K tile)
// Computing S transposed leaves each lane holding one query row and 8
// consecutive keys, which is exactly the B operand layout the PV product
// needs: at D = 64 / 128 P stays in registers; at D = 512 each wave's P
// fragment goes through LDS once so that the PV product can be split over D
// (see hca_fwd512s_kernel).
#include <climits>
#include <mutex>

#include "hca_device.h"
#include "hca_internal.h"
#include "hca_stage.h"

namespace hca {

constexpr int kBK = 32;  // keys per tile (raw and compressed)
constexpr float kLazyF = 8.f;  // lazy-rescale margin of the D = 64 / 128 forward (log2 units)

#ifndef HCA_FWD_NW
#define HCA_FWD_NW 4  // waves of the D = 512 forward: 4 (two workgroups per CU) or 8 (one)
#endif
#ifndef HCA_FWD_QK_PF
#define HCA_FWD_QK_PF 3  // k-steps of K fragments in flight ahead of the S^T MFMAs
#endif


template <int D, int NW, int MB>
__global__ void __launch_bounds__(NW * 64, 1)
    hca_fwd_bf16_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                        const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                        const bf16raw *__restrict__ kvt, const bf16raw *__restrict__ kvct,
                        float scale_log2, bf16raw *__restrict__ o, float *__restrict__ lse) {
  constexpr int NT = NW * 64;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  using St = KTile<D, NT>;
  __shared__ __attribute__((aligned(16))) bf16raw k_lds[kBK * D];

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

  uint4 pk[St::KPT];
  // The query tile's list entries: the first 64 held one per lane (read with
  // readlane, no memory round trip per tile), later ones loaded.
  const uint32_t ent_lane = lane < e_end - e_begin ? p.qent[e_begin + lane] : 0u;
  auto entry = [&](int e) -> uint32_t {
    const int t = e - e_begin;
    return t < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)ent_lane, t)
                  : uniform_load(p.qent, e);
  };
  auto issue = [&](int e) {
    const uint32_t ent = entry(e);
    const bool comp = ent & kEntComp;
    const int k0 = (int)(ent & kEntIdx) * kBK;
    St::load(pk, tid, comp ? kvc_b : kv_b, comp ? d.Sc : d.S, k0);
  };
  if (e_begin < e_end) issue(e_begin);

  // A-operand rows of the two 16-key halves: lane group g ends up holding
  // keys 8g .. 8g+7 of the 32-key tile for its query row.
  const int r0 = 8 * (j >> 2) + (j & 3), r1 = r0 + 4;

  for (int e = e_begin; e < e_end; ++e) {
    const uint32_t ent = entry(e);
    const bool comp = ent & kEntComp;
    const bool full = ent & kEntFull;
    const int k0 = (int)(ent & kEntIdx) * kBK;
    __syncthreads();
    St::store(pk, tid, k_lds);
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
      const bf16x8 a0 = St::kfrag(k_lds, r0, ks, g);
      const bf16x8 a1 = St::kfrag(k_lds, r1, ks, g);
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
        // The row's visible keys of this tile's kind, [lo, hi] (selects, no
        // branches).
        const int lo = comp ? clo[mb] : rlo[mb], hi = comp ? chi[mb] - 1 : pos[mb];
        const int kb = k0 + 8 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bool vis = (kb + t >= lo) & (kb + t <= hi);
          x[t] = vis ? x[t] : -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int t = 1; t < 8; ++t) mx = fmaxf(mx, x[t]);
      mx = group_max(mx);
      // Lazy rescaling (as at D = 512): the reference max m_run only moves when
      // the tile max passes it by more than kLazyF log2 units.
      const bool up = mx > m_run[mb] + kLazyF;
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float m_new = up ? mx : m_run[mb];
        const float alpha = fast_exp2(m_run[mb] - (m_new == -INFINITY ? 0.f : m_new));
        l_run[mb] *= alpha;
        m_run[mb] = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[mb][db] *= alpha;
      }
      const float m_use = m_run[mb] == -INFINITY ? 0.f : m_run[mb];
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[t] = fast_exp2(x[t] - m_use);
        ps += x[t];
      }
      l_run[mb] += ps;
      pb[mb] = pack8(x);
    }

#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = St::tfrag(k_lds, db, g, j);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][db] = mfma16x16x32(a, pb[mb], oacc[mb][db]);
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float l = group_sum(l_run[mb]);
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

// Lazy rescaling: a row's reference max m_run only moves when the tile max
// exceeds it by more than kLazy (log2 units), so P = 2^(x - m_run) stays below
// 2^kLazy and the O rescale (a wave-uniform branch) is rare.
constexpr float kLazy = 8.f;

// ---------------------------------------------------------------------------
// D = 512 forward with the PV product split over the head dimension.
// ---------------------------------------------------------------------------
// NW waves, 16 NW rows per workgroup.  NW = 4 (the default): two workgroups
// per CU, K and K^T single-buffered (64 KiB), so one workgroup's copies and
// barriers run under the other's math; NW = 8: one workgroup per CU, K and
// K^T double-buffered (128 KiB), one barrier per tile.  The scores stay
// row-blocked: wave w holds the Q fragments of rows 16 w .. 16 w + 15 and
// forms their S^T and softmax.  The PV product is split over D instead: wave
// w accumulates O^T for columns (512 / NW) w .. of all the workgroup's rows,
// so each K^T fragment it reads from LDS feeds NW MFMAs (one per row block)
// instead of one.  P goes through LDS (one 1 KiB fragment per wave and tile,
// double-buffered), with each row's lazy-rescale factor.  Per wave and tile
// the LDS reads fall from 64 KiB (32 K and 32 K^T fragments) to 44 KiB
// (NW = 8: 32 K, 4 K^T, 8 P fragments; NW = 4: 32 K, 8 K^T, 4 P).
template <int NW, bool MASKED>
__global__ void __launch_bounds__(NW * 64, 8 / NW)
    hca_fwd512s_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                       const bf16raw *__restrict__ kvt, const bf16raw *__restrict__ kvct,
                       float scale_log2, bf16raw *__restrict__ o, float *__restrict__ lse) {
  constexpr int D = 512, KS = D / 32, M = NW * 16, RB = M / 16, CB = D / 16 / NW;
  // NW = 8: [K 0][K 1][K^T 0][K^T 1], NW = 4: [K][K^T]; after the tile walk,
  // the output rows.
  constexpr int kBufs = NW == 8 ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufs * kTileBytes512];
  __shared__ __attribute__((aligned(1024))) char pbuf[2][RB * 1024];  // P fragments per row block
  __shared__ float alpha_s[2][M];  // per row: O rescale factor of the tile
  __shared__ int resc_s[2][RB];    // per row block: any row rescaled in the tile
  __shared__ float inv_s[M];       // per row: 1 / l
  char *const kbase = smem;
  char *const tbase = smem + kBufs * kTileBytes512;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int nslices = d.bq * d.H / M;
  const int lbq = __builtin_ctz(d.bq);
  const int u = xcd_remap(blockIdx.x, d.B * d.nqt * nslices, 2 * nslices);
  const int li = u / nslices, sl = u - li * nslices;
  const int item = p.qorder[li];
  const int b = item / d.nqt, qt = item - b * d.nqt;

  // This lane's score row: row 16 wave + j of the slice.
  const int rho = sl * M + wave * 16 + j;
  const int pos = qt * d.bq + (rho & (d.bq - 1)), hh = rho >> lbq;
  const bool valid = pos < d.S;

  const int e_begin = p.qptr[item], nent = p.qptr[item + 1] - e_begin;
  const uint32_t ent_lane = lane < nent ? p.qent[e_begin + lane] : 0u;
  __builtin_amdgcn_s_waitcnt(0);
  auto entry = [&](int t) -> uint32_t {
    return t < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)ent_lane, t)
                  : uniform_load(p.qent, e_begin + t);
  };
  const rsrc_t r_img =
      make_rsrc(kvt + (size_t)b * 2 * D * d.S_pad, (uint32_t)d.S_pad * D * 4);
  const rsrc_t r_imgc =
      make_rsrc(kvct + (size_t)b * 2 * D * d.Sc_pad, (uint32_t)d.Sc_pad * D * 4);
  auto stage_k = [&](int t) {
    if (t >= nent) return;
    const uint32_t ent = entry(t);
    stage_img512<NW>((ent & kEntComp) ? r_imgc : r_img, (int)(ent & kEntIdx) * kBK, 0,
                     kbase + (t & (kBufs - 1)) * kTileBytes512, wave, lane);
  };
  auto stage_t = [&](int t) {
    if (t >= nent) return;
    const uint32_t ent = entry(t);
    stage_img512<NW>((ent & kEntComp) ? r_imgc : r_img, (int)(ent & kEntIdx) * kBK, 1,
                     tbase + (t & (kBufs - 1)) * kTileBytes512, wave, lane);
  };
  const int frag_off = 16 * lane;

  // Q fragments and the row's key intervals (padded rows read the last row
  // and get empty intervals).
  bf16x8 qf[KS];
  int rlo, clo, chi;
  auto load_q = [&]() {
    const int pc = min(pos, d.S - 1);
    const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pc];
    rlo = valid ? rw.x : INT_MAX;
    clo = valid ? rw.y : 0;
    chi = valid ? rw.z : 0;
    const bf16raw *qrow = q + (((size_t)b * d.H + hh) * d.S + pc) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * g));
  };

  // S^T of tile t for this wave's rows: two 16-key halves, K fragments read
  // QK_PF k-steps ahead of their MFMAs.
  auto qk = [&](int t, floatx4 (&s)[2]) {
    constexpr int PF = HCA_FWD_QK_PF;
    const char *kb = kbase + (t & (kBufs - 1)) * kTileBytes512 + frag_off;
    s[0] = s[1] = floatx4{0.f, 0.f, 0.f, 0.f};
    mfma_phase_begin();
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
      s[0] = mfma16x16x32(a0[ks], qf[ks], s[0]);
      s[1] = mfma16x16x32(a1[ks], qf[ks], s[1]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    mfma_phase_end();
  };

  // Masked plans: the row's 32 visibility bits for the compressed tile of
  // entry `ent` (0 for raw, FULL and padded).
  auto load_mask = [&](uint32_t ent) -> uint32_t {
    if constexpr (MASKED) {
      if ((ent & kEntComp) && !(ent & kEntFull) && valid)
        return p.cmask[((size_t)b * d.S + pos) * d.cmask_ldw + (ent & kEntIdx)];
    }
    return 0u;
  };

  // Online softmax of tile t (owner of the rows): P to the exchange buffer
  // t & 1, with the rows' rescale factors.
  float m_run = -INFINITY, l_run = 0.f;
  auto softmax = [&](int t, const floatx4 (&sc)[2], uint32_t ent, uint32_t mword) {
    const bool comp = ent & kEntComp;
    const int k0 = (int)(ent & kEntIdx) * kBK;
    float x[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x[v] = sc[0][v] * scale_log2;
      x[4 + v] = sc[1][v] * scale_log2;
    }
    if (!(ent & kEntFull)) {
      if (MASKED && comp) {
        const uint32_t bits = mword >> (8 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = ((bits >> i) & 1u) ? x[i] : -INFINITY;
      } else {
        const int lo = (comp ? clo : rlo) - (k0 + 8 * g);
        const int hi = (comp ? chi : pos + 1) - (k0 + 8 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (i >= lo && i < hi) ? x[i] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = group_max(mx);
    const bool up = mx > m_run + kLazy;
    const bool any = __builtin_amdgcn_ballot_w64(up) != 0;
    float alpha = 1.f;
    if (any) {
      const float m_new = up ? mx : m_run;
      alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = fast_exp2(x[i] - m_use);
      l_run += x[i];
    }
    *reinterpret_cast<bf16x8 *>(pbuf[t & 1] + wave * 1024 + frag_off) = pack8(x);
    if (g == 0) alpha_s[t & 1][wave * 16 + j] = alpha;
    if (lane == 0) resc_s[t & 1][wave] = any ? 1 : 0;
  };

  // O^T[64 w .. 64 w + 63][all rows] += K^T P^T of tile t: the wave's four
  // K^T fragments are held while the eight P fragments stream through.
  floatx4 oacc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < CB; ++c) oacc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto pv = [&](int t) {
    const int bf = t & 1;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (__builtin_amdgcn_readfirstlane(resc_s[bf][rb])) {
        const float a = alpha_s[bf][rb * 16 + j];
#pragma unroll
        for (int c = 0; c < CB; ++c) oacc[rb][c] *= a;
      }
    }
    mfma_phase_begin();
    const char *tb = tbase + (t & (kBufs - 1)) * kTileBytes512 + wave * CB * 1024 + frag_off;
    const char *pb = pbuf[bf] + frag_off;
    bf16x8 kt[CB], pf[RB];
#pragma unroll
    for (int c = 0; c < CB; ++c) kt[c] = lds_frag(tb + c * 1024);
    pf[0] = lds_frag(pb);
    pf[1] = lds_frag(pb + 1024);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb + 2 < RB) pf[rb + 2] = lds_frag(pb + (rb + 2) * 1024);
#pragma unroll
      for (int c = 0; c < CB; ++c) oacc[rb][c] = mfma16x16x32(kt[c], pf[rb], oacc[rb][c]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, CB + 2, 0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb + 2 < RB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, CB, 0);
    }
    mfma_phase_end();
  };

  floatx4 sc[2];
  if constexpr (NW == 8) {
    // K runs two tiles ahead, K^T one; the S^T of tile t + 1 is issued before
    // the PV of tile t, its softmax after; one barrier per tile.
    stage_k(0);
    stage_k(1);
    stage_t(0);
    load_q();
    wait_all_loads();
    __syncthreads();
    if (nent > 0) {
      const uint32_t e0 = entry(0);
      const uint32_t mw = load_mask(e0);
      qk(0, sc);
      softmax(0, sc, e0, mw);
    }
    __syncthreads();  // P of tile 0 visible; K buffer 0 free
    stage_k(2);
    stage_t(1);
    for (int it = 0; it < nent; ++it) {
      const bool more = it + 1 < nent;
      const uint32_t en = more ? entry(it + 1) : 0u;
      const uint32_t mw = load_mask(en);
      if (more) qk(it + 1, sc);
      pv(it);
      if (more) softmax(it + 1, sc, en, mw);
      wait_all_loads();
      __syncthreads();
      stage_k(it + 3);
      stage_t(it + 2);
    }
  } else {
    // Single-buffered, two workgroups per CU: the K copy of tile t + 1 runs
    // under the PV of tile t, the K^T copy of tile t + 1 under its scores and
    // softmax; two barriers per tile.  The other workgroup covers the waits.
    stage_k(0);
    stage_t(0);
    load_q();
    wait_all_loads();
    __syncthreads();
    if (nent > 0) {
      const uint32_t e0 = entry(0);
      const uint32_t mw = load_mask(e0);
      qk(0, sc);
      softmax(0, sc, e0, mw);
    }
    __syncthreads();  // P of tile 0 visible; K buffer free
    stage_k(1);
    for (int it = 0; it < nent; ++it) {
      pv(it);
      wait_all_loads();  // K of tile it + 1
      __syncthreads();   // K^T buffer free, K of tile it + 1 visible
      if (it + 1 < nent) {
        const uint32_t en = entry(it + 1);
        const uint32_t mw = load_mask(en);
        stage_t(it + 1);
        qk(it + 1, sc);
        softmax(it + 1, sc, en, mw);
        wait_all_loads();  // K^T of tile it + 1
        __syncthreads();   // K buffer free, K^T and P of tile it + 1 visible
        stage_k(it + 2);
      }
    }
  }

  // Row statistics: 1 / l to LDS for every wave, LSE by the owner.
  {
    const float l = group_sum(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (g == 0) inv_s[wave * 16 + j] = inv;
    if (valid && g == 0)
      lse[((size_t)b * d.H + hh) * d.S + pos] =
          l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
  }
  __syncthreads();  // inv_s visible (the tile buffers are idle: no copy in flight)
  // Normalised O as bf16 into the tile buffers, row r at r * 1024 with its
  // 16-byte chunk c at (c ^ (r & 15)), then every wave stores 16 whole rows.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + j;
    const float inv = inv_s[r];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      ushort4 w;
      w.x = f2bf(oacc[rb][c][0] * inv);
      w.y = f2bf(oacc[rb][c][1] * inv);
      w.z = f2bf(oacc[rb][c][2] * inv);
      w.w = f2bf(oacc[rb][c][3] * inv);
      const int chunk = 2 * (CB * wave + c) + (g >> 1);
      *reinterpret_cast<ushort4 *>(smem + r * 1024 + ((chunk ^ j) << 4) + ((g & 1) << 3)) = w;
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int r = wave * 16 + i;
    const int rr = sl * M + r;
    const int pr = qt * d.bq + (rr & (d.bq - 1)), hr = rr >> lbq;
    if (pr < d.S) {
      const uint4 v = *reinterpret_cast<const uint4 *>(smem + r * 1024 + ((lane ^ (r & 15)) << 4));
      *reinterpret_cast<uint4 *>(o + (((size_t)b * d.H + hr) * d.S + pr) * D + 8 * lane) = v;
    }
  }
}

// One key tensor and its workspace copy (raw kv or compressed kv): N keys,
// N_pad after padding to whole tiles.
struct KvCopy {
  const bf16raw *src;
  bf16raw *dst;
  int N, N_pad;
};

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
  // (Only the D = 512 kernels read staged copies of K.)
  return (int)hipErrorInvalidValue;
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
      // 16 NW rows per workgroup (bq * H is a power of two >= 128).
      constexpr int NW = HCA_FWD_NW;
      const dim3 gs(d.B * d.nqt * (d.bq * d.H / (16 * NW)));
      auto gos = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, gs, dim3(NW * 64), 0, s, d, p, (const bf16raw *)q,
                           (const bf16raw *)kvt, (const bf16raw *)kvct, sl2, (bf16raw *)o, lse);
      };
      if (d.cmask_ldw)
        gos(hca_fwd512s_kernel<NW, true>);
      else
        gos(hca_fwd512s_kernel<NW, false>);
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
