// hca_bwd.hip -- HCA attention backward on gfx950 (bf16 MFMA, fp32 accumulation).
//
// Gradients of softmax attention with one shared key/value tensor ("[DeepSeek-V4]
// Implement Compressed Attention Layers", review suggestions: k = kv, v = kv,
// broadcast over heads), so each key's gradient is the sum of its key path and
// its value path over every head:
//   P = exp(scale <q, kv> - LSE),  dP = <dO, kv>,  delta = <dO, O>,
//   dS = P (dP - delta),  dQ = scale sum_k dS kv_k,
//   dKV_k = sum_rows scale dS q + P dO.
//
// Three kernels, all driven by the host-built block table:
//  1. query-stationary dQ: same tiling and key-tile walk as the forward; the
//     row's Q and dO fragments stay in VGPRs, delta is computed from O and dO
//     before the tile walk, and dQ is accumulated in registers and written
//     once -- no atomics (the page on the static mask compiles the backward with
//     an on-chip dQ reduction; here the whole dQ row stays on chip).
//  2. key-stationary dKV: a workgroup owns one work item -- a key tile (raw
//     or compressed; 128 keys at D = 512, 32 otherwise) and the query tiles
//     of one 64-position chunk that see it -- recomputing S and dP with the
//     tile's K fragments held in VGPRs.  At D = 512, items whose rows see only
//     one 64-key half of their tile run as a second launch over that half.
//     Each item writes a float32 partial.
//  3. a fixed-order reduction of the partials into dKV and dKV_comp, so the
//     result is bitwise reproducible.
#include <atomic>
#include <climits>

#include "hca_device.h"
#include "hca_internal.h"
#include "hca_stage.h"

namespace hca {

namespace {

constexpr int kBK = 32;

template <int D, int NT>
struct StageB {
  static constexpr int KROW = D + 8;
  static constexpr int TROW = kBK + 8;
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

__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  const bf16raw *x = reinterpret_cast<const bf16raw *>(&a);
  const bf16raw *y = reinterpret_cast<const bf16raw *>(&b);
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) s += bf2f(x[t]) * bf2f(y[t]);
  return s;
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. dQ (+ delta), query-stationary.
// ---------------------------------------------------------------------------
template <int D, int NW, int MB>
__global__ void __launch_bounds__(NW * 64, 1)
    hca_bwd_dq_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                      const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                      const bf16raw *__restrict__ kvt, const bf16raw *__restrict__ kvct,
                      const bf16raw *__restrict__ o, const float *__restrict__ lse,
                      const bf16raw *__restrict__ dout, float scale_log2, float scale,
                      bf16raw *__restrict__ dq, float *__restrict__ delta) {
  constexpr int NT = NW * 64;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr int M = NW * MB * 16;
  using St = StageB<D, NT>;
  __shared__ __attribute__((aligned(16))) bf16raw k_lds[kBK * St::KROW];
  __shared__ __attribute__((aligned(16))) bf16raw t_lds[D * St::TROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int nslices = d.bq * d.H / M;
  const int nitems = d.B * d.nqt;
  const int li = blockIdx.x / nslices, sl = blockIdx.x - li * nslices;
  const int item = p.qorder[xcd_remap(li, nitems)];
  const int b = item / d.nqt, qt = item - b * d.nqt;

  int pos[MB], hh[MB], rlo[MB], clo[MB], chi[MB];
  bool valid[MB];
  float lse2[MB], dl[MB];
  bf16x8 qf[MB][KS], dof[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rho = sl * M + (wave * MB + mb) * 16 + j;
    pos[mb] = qt * d.bq + rho / d.H;
    hh[mb] = rho % d.H;
    valid[mb] = pos[mb] < d.S;
    const size_t row = ((size_t)b * d.H + hh[mb]) * d.S + pos[mb];
    if (valid[mb]) {
      const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pos[mb]];
      rlo[mb] = rw.x;
      clo[mb] = rw.y;
      chi[mb] = rw.z;
      lse2[mb] = lse[row] * kLog2e;
    } else {
      rlo[mb] = INT_MAX;
      clo[mb] = 0;
      chi[mb] = 0;
      lse2[mb] = -INFINITY;
    }
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 qv = make_uint4(0, 0, 0, 0), dv = qv, ov = qv;
      if (valid[mb]) {
        qv = *reinterpret_cast<const uint4 *>(q + row * D + 32 * ks + 8 * g);
        dv = *reinterpret_cast<const uint4 *>(dout + row * D + 32 * ks + 8 * g);
        ov = *reinterpret_cast<const uint4 *>(o + row * D + 32 * ks + 8 * g);
      }
      qf[mb][ks] = as_bf16x8(qv);
      dof[mb][ks] = as_bf16x8(dv);
      part += dot8(dv, ov);
    }
    part = xor_sum(part, 16);
    part = xor_sum(part, 32);
    dl[mb] = part;
    if (valid[mb] && g == 0) delta[row] = part;
  }

  floatx4 acc[MB][DB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[mb][db] = floatx4{0.f, 0.f, 0.f, 0.f};

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

    floatx4 s0[MB], s1[MB], p0[MB], p1[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s0[mb] = s1[mb] = p0[mb] = p1[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a0 = as_bf16x8(lds_load16(k_lds + r0 * St::KROW + 32 * ks + 8 * g));
      const bf16x8 a1 = as_bf16x8(lds_load16(k_lds + r1 * St::KROW + 32 * ks + 8 * g));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s0[mb] = mfma16x16x32(a0, qf[mb][ks], s0[mb]);
        s1[mb] = mfma16x16x32(a1, qf[mb][ks], s1[mb]);
        p0[mb] = mfma16x16x32(a0, dof[mb][ks], p0[mb]);
        p1[mb] = mfma16x16x32(a1, dof[mb][ks], p1[mb]);
      }
    }
    bf16x8 dsb[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float x[8], dp[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[v] = s0[mb][v] * scale_log2;
        x[4 + v] = s1[mb][v] * scale_log2;
        dp[v] = p0[mb][v];
        dp[4 + v] = p1[mb][v];
      }
      const int kb = k0 + 8 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        bool vis = true;
        if (!full) {
          const int key = kb + t;
          vis = comp ? (key >= clo[mb] && key < chi[mb]) : (key >= rlo[mb] && key <= pos[mb]);
        }
        const float pr = vis ? fast_exp2(x[t] - lse2[mb]) : 0.f;
        x[t] = pr * (dp[t] - dl[mb]);
      }
      dsb[mb] = pack8(x);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = as_bf16x8(lds_load16(t_lds + (16 * db + j) * St::TROW + 8 * g));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][db] = mfma16x16x32(a, dsb[mb], acc[mb][db]);
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (!valid[mb]) continue;
    bf16raw *drow = dq + (((size_t)b * d.H + hh[mb]) * d.S + pos[mb]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      ushort4 w;
      w.x = f2bf(acc[mb][db][0] * scale);
      w.y = f2bf(acc[mb][db][1] * scale);
      w.z = f2bf(acc[mb][db][2] * scale);
      w.w = f2bf(acc[mb][db][3] * scale);
      *reinterpret_cast<ushort4 *>(drow + 16 * db + 4 * g) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// 1b. dQ (+ delta) at D = 512: NW waves x 16 rows, one wave per SIMD (Q, dO
//     and the dQ accumulator take ~260 registers), persistent: one workgroup
//     per compute unit walks 64-row slices, loading the next slice's list
//     entries and rows under its current slice's last two tiles.  K and K^T
//     tiles double-buffered in LDS one tile apart, copied from the tile images
//     by buffer-to-LDS loads in MFMA fragment order, one barrier per tile.
//     The S^T and dP^T products of tile t+1 share their K A-operands and are
//     issued before dS and the dQ product of tile t, so VALU work overlaps
//     matrix-core work.
// ---------------------------------------------------------------------------
template <int NW>
__global__ void __launch_bounds__(NW * 64, 1)
    hca_bwd_dq512_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                         const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                         const bf16raw *__restrict__ kvt, const bf16raw *__restrict__ kvct,
                         const bf16raw *__restrict__ o, const float *__restrict__ lse,
                         const bf16raw *__restrict__ dout, float scale_log2, float scale,
                         bf16raw *__restrict__ dq, float *__restrict__ delta) {
  constexpr int D = 512, KS = D / 32, DB = D / 16;
  constexpr int M = NW * 16;
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileBytes512];
  char *const kbase = smem;
  char *const tbase = smem + 2 * kTileBytes512;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  // Query tile = bq positions x H heads, rows position-fastest, in slices of
  // M rows (one wave = 16 consecutive positions of one head); the slices of
  // two neighbouring tiles run back to back on one XCD.
  const int nslices = d.bq * d.H / M;
  const int lbq = __builtin_ctz(d.bq);
  const int nunits = d.B * d.nqt * nslices;
  // Operand reads are flat: lane l reads bytes 16 l .. 16 l + 15 of a block.
  const int frag_off = 16 * lane;

  // Persistent: workgroup w takes units w, w + G, w + 2G, ... (G = grid size, a
  // multiple of 8, so all of them run on w's XCD), each one slice of M rows of
  // a query tile.  While a unit works on its last key tile its Q and dO rows
  // are dead, so the next unit's list entries and rows are loaded then.
  int sl = 0, item = 0, e_begin = 0, nent = 0;
  uint32_t ent_lane = 0u;
  int4 rw;
  float lv;
  uint4 qv[KS], dv[KS], ov[KS];
  // Unit v's slice, query tile and list extent, from scalar loads.
  auto locate = [&](int v, int &sl_, int &item_, int &e_begin_, int &nent_) {
    const int u = xcd_remap(v, nunits, 2 * nslices);
    const int li = u / nslices;
    sl_ = u - li * nslices;
    item_ = (int)uniform_load((const uint32_t *)p.qorder, li);
    e_begin_ = (int)uniform_load((const uint32_t *)p.qptr, item_);
    nent_ = (int)uniform_load((const uint32_t *)p.qptr, item_ + 1) - e_begin_;
  };
  // Issues the loads of a unit's list entries and rows (entries first); no wait.
  // A wave's 16 rows are 16 consecutive positions of one head (bq >= 16), so
  // each tensor is addressed from one wave-uniform row base plus a small
  // per-lane offset.  Padded rows (pos >= S) read row S - 1 and are zeroed /
  // masked later, so every load is unconditional.
  // fetch() ends with these vector-memory loads (Q, dO and O row fragments);
  // the wait in the last tile below counts on them being the last ones issued.
  constexpr int kRowLoads = 3 * KS;
  static_assert(kRowLoads <= 63, "the vmcnt field holds at most 63 outstanding loads");
  auto fetch = [&](int sl_, int item_, int e_begin_, int nent_) {
    e_begin = e_begin_;
    nent = nent_;
    ent_lane = lane < nent ? p.qent[e_begin + lane] : 0u;
    const int b_ = item_ / d.nqt, qt_ = item_ - b_ * d.nqt;
    const int rho0 = sl_ * M + wave * 16;
    const int pos0 = qt_ * d.bq + (rho0 & (d.bq - 1)), hh_ = rho0 >> lbq;
    // this lane's row relative to pos0, clamped to row S - 1 (negative when
    // the whole 16-row block lies past S, as in the last tile when bq = 32)
    const int jr = min(j, d.S - 1 - pos0);
    const size_t r0 = ((size_t)b_ * d.H + hh_) * d.S + pos0;
    rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b_ * d.S + pos0 + jr];
    lv = lse[r0 + jr];
    const bf16raw *qb = q + r0 * D, *db_ = dout + r0 * D, *ob = o + r0 * D;
    const int loff = jr * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qv[ks] = *reinterpret_cast<const uint4 *>(qb + loff + 32 * ks);
      dv[ks] = *reinterpret_cast<const uint4 *>(db_ + loff + 32 * ks);
      ov[ks] = *reinterpret_cast<const uint4 *>(ob + loff + 32 * ks);
    }
  };

  int v = blockIdx.x;
  {
    int e0, n0;
    locate(v, sl, item, e0, n0);
    fetch(sl, item, e0, n0);
  }
  for (;;) {
    const int b = item / d.nqt, qt = item - b * d.nqt;
    const int rho = sl * M + wave * 16 + j;
    const int pos = qt * d.bq + (rho & (d.bq - 1)), hh = rho >> lbq;
    const bool valid = pos < d.S;
    const size_t row = ((size_t)b * d.H + hh) * d.S + pos;
    const int vn = v + (int)gridDim.x;
    const bool more = vn < nunits;

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
                       kbase + (t & 1) * kTileBytes512, wave, lane);
    };
    auto stage_t = [&](int t) {  // K^T of list entry t
      if (t >= nent) return;
      const uint32_t ent = entry(t);
      stage_img512<NW>((ent & kEntComp) ? r_imgc : r_img, (int)(ent & kEntIdx) * kBK, 1,
                       tbase + (t & 1) * kTileBytes512, wave, lane);
    };

    // S^T and dP^T of tile t (shared K A-operands): [0] keys 0-15, [1] keys 16-31.
    // Operand fragments are read PF k-steps ahead of their MFMAs.
    auto sdp = [&](int t, floatx4 (&s)[2], floatx4 (&dp)[2]) {
      constexpr int PF = 3;
      const char *kb = kbase + (t & 1) * kTileBytes512;
      s[0] = s[1] = dp[0] = dp[1] = floatx4{0.f, 0.f, 0.f, 0.f};
      bf16x8 a0[KS], a1[KS];
      auto at = [&](int ks) { return kb + 2048 * ks + frag_off; };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) {
        a0[ks] = lds_frag(at(ks));
        a1[ks] = lds_frag(at(ks) + 1024);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) {
          a0[ks + PF] = lds_frag(at(ks + PF));
          a1[ks + PF] = lds_frag(at(ks + PF) + 1024);
        }
        s[0] = mfma16x16x32(a0[ks], as_bf16x8(qv[ks]), s[0]);
        s[1] = mfma16x16x32(a1[ks], as_bf16x8(qv[ks]), s[1]);
        dp[0] = mfma16x16x32(a0[ks], as_bf16x8(dv[ks]), dp[0]);
        dp[1] = mfma16x16x32(a1[ks], as_bf16x8(dv[ks]), dp[1]);
      }
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    };

    // The first tile copies need only the list entries (loaded before the rows).
    stage_k(0);
    stage_k(1);
    stage_t(0);
    // Past the last unit the current one is fetched again (unused), so the
    // row registers are always reloaded and never kept live across a unit.
    int sl_n = sl, item_n = item, e_begin_n = e_begin, nent_n = nent;
    if (more) locate(vn, sl_n, item_n, e_begin_n, nent_n);
    wait_all_loads();
    // A padded row keeps the clamped row's data: its key interval is empty
    // (and a tile holding it is never FULL), so its P and dS are zero, and its
    // dQ and delta are never stored.
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) part += dot8(dv[ks], ov[ks]);
    const float dl = group_sum(part);
    const int rlo = valid ? rw.x : INT_MAX;
    const int clo = valid ? rw.y : 0;
    const int chi = valid ? rw.z : 0;
    const float lse2 = valid ? lv * kLog2e : -INFINITY;
    if (valid && g == 0) delta[row] = dl;
    __syncthreads();

    floatx4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    floatx4 sc[2], pc[2];
    if (nent > 0) sdp(0, sc, pc);
    __syncthreads();
    stage_k(2);
    stage_t(1);

    // dS of tile it from its scores, then dQ^T += K^T dS^T.
    auto grad = [&](int it, uint32_t ent) {
      const bool comp = ent & kEntComp;
      const int k0 = (int)(ent & kEntIdx) * kBK;
      float x[8];
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        x[v4] = sc[0][v4] * scale_log2 - lse2;
        x[4 + v4] = sc[1][v4] * scale_log2 - lse2;
      }
      if (!(ent & kEntFull)) {
        const int lo = (comp ? clo : rlo) - (k0 + 8 * g);
        const int hi = (comp ? chi : pos + 1) - (k0 + 8 * g);
#pragma unroll
        for (int t = 0; t < 8; ++t) x[t] = (t >= lo && t < hi) ? x[t] : -INFINITY;
      }
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        x[v4] = fast_exp2(x[v4]) * (pc[0][v4] - dl);
        x[4 + v4] = fast_exp2(x[4 + v4]) * (pc[1][v4] - dl);
      }
      const bf16x8 dsb = pack8(x);
      __builtin_amdgcn_sched_barrier(0);
      {
        // Fragments read PV column blocks ahead.
        constexpr int PV = 8;
        const char *tb = tbase + (it & 1) * kTileBytes512 + frag_off;
        bf16x8 kt[DB];
#pragma unroll
        for (int db = 0; db < PV; ++db) kt[db] = lds_frag(tb + db * 1024);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          if (db + PV < DB) kt[db + PV] = lds_frag(tb + (db + PV) * 1024);
          acc[db] = mfma16x16x32(kt[db], dsb, acc[db]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, PV, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          if (db + PV < DB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // List entries are read only right after the barrier (where a wait for a
    // scalar load costs nothing): ent holds the entry of the current tile.
    uint32_t ent = nent > 0 ? entry(0) : 0u;
    const int last = nent - 1;
    for (int it = 0; it + 1 < last; ++it) {
      floatx4 sn[2], pn[2];
      sdp(it + 1, sn, pn);
      grad(it, ent);
      sc[0] = sn[0];
      sc[1] = sn[1];
      pc[0] = pn[0];
      pc[1] = pn[1];
      wait_all_loads();
      __syncthreads();
      ent = entry(it + 1);
      stage_k(it + 3);
      stage_t(it + 2);
    }
    // Once the last tile's scores are taken this unit's Q and dO rows are
    // dead: the next unit's entries and rows load from there on, under the
    // last two tiles and the store (one fetch site, so the loaded registers
    // need no copies that would wait for them).
    floatx4 sn[2], pn[2];
    uint32_t ent_last = 0u;
    if (last >= 1) {
      ent_last = entry(last);  // before the fetch replaces the entries
      sdp(last, sn, pn);
    }
    fetch(sl_n, item_n, e_begin_n, nent_n);
    // Nothing is scheduled across this point, so every load of fetch() is
    // issued before the wait below.
    __builtin_amdgcn_sched_barrier(0);
    if (last >= 1) {
      grad(last - 1, ent);
      sc[0] = sn[0];
      sc[1] = sn[1];
      pc[0] = pn[0];
      pc[1] = pn[1];
      // The last K^T copy was issued before the fetch, and fetch() issues at
      // least kRowLoads vector-memory loads after it (its list, row-interval
      // and LSE loads, then the row fragments).  Loads complete in issue
      // order, so leaving kRowLoads outstanding still waits for the copy while
      // the row loads stay in flight.  The barrier orders LDS only.
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kRowLoads) : "memory");
      lds_barrier();
      ent = ent_last;
    }
    if (last >= 0) grad(last, ent);

    // No copy is in flight and no wave reads the K buffers any more (the last
    // tile reads only its K^T buffer): each wave stages its 16 rows of dQ there
    // and stores whole rows.
    // The store's LDS addresses depend on the lane only; an opaque copy of the
    // lane keeps the compiler from hoisting all 32 of them out of the unit loop
    // (they would be spilled, and every reload waits for the rows in flight).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    store_rows512(acc, scale, smem + wave * 16384, ln, [&](int r) -> bf16raw * {
      const int rr = sl * M + wave * 16 + r;
      const int pr = qt * d.bq + (rr & (d.bq - 1)), hr = rr >> lbq;
      return pr < d.S ? dq + (((size_t)b * d.H + hr) * d.S + pr) * D : nullptr;
    });
    if (!more) {
      wait_all_loads();
      break;
    }
    // Every wave's staged rows are read before the next unit's copies land.
    lds_barrier();
    v = vn;
    sl = sl_n;
    item = item_n;
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

// ---------------------------------------------------------------------------
// 2. dKV, key-stationary.  4 waves: wave & 1 selects 16 of the tile's 32 keys,
//    wave >> 1 selects one 32-row half of each 64-row step.  Staged rows are
//    unpadded with their 16-byte chunks XOR-swizzled (chunk c of row r at
//    slot c ^ rsw(r)), so the score-phase fragment reads touch distinct bank
//    groups and the gradient's transposed operands come from two
//    ds_read_b64_tr_b16 reads each (sixteen 2-byte reads before).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256, 1)
    hca_bwd_dkv_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                       const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                       const float *__restrict__ lse, const float *__restrict__ delta,
                       const bf16raw *__restrict__ dout, float scale_log2, float scale,
                       float *__restrict__ part) {
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr int STEP = 64;           // query rows staged per step
  constexpr int QROW = D;            // LDS row (bf16), chunks swizzled
  constexpr int NCH = D / 8;         // 16-B chunks per row
  constexpr int RCH = STEP * NCH;    // 16-B chunks per staged tensor
  static_assert(STEP * QROW * 2 >= 2 * D * 16 * 4, "reduction scratch fits in q_lds");
  auto rsw = [](int r) { return ((r & 3) | (((r >> 3) & 3) << 2)) & (NCH - 1); };
  __shared__ __attribute__((aligned(16))) bf16raw q_lds[STEP * QROW];
  __shared__ __attribute__((aligned(16))) bf16raw o_lds[STEP * QROW];  // dO rows
  __shared__ float lse_lds[STEP], dl_lds[STEP];
  __shared__ int4 info_lds[STEP];  // rlo, clo, chi, pos (pos = INT_MAX if padded)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int kh = wave & 1, rh = wave >> 1;
  const int item = p.kvorder[blockIdx.x];
  if (item < 0) return;  // padding slot of the launch order
  const KvItem it = p.kvitem[item];
  const int b = it.b;
  const bool comp = it.kind != 0;
  const int k0 = it.kt * kBK;
  const int nk = comp ? d.Sc : d.S;
  const bf16raw *src = (comp ? kvc + (size_t)b * d.Sc * D : kv + (size_t)b * d.S * D);
  const int mykey = k0 + kh * 16 + j;  // this lane's key (B-operand column)

  // Stationary K fragments: B[k = d][n = key].
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kf[ks] = as_bf16x8(mykey < nk ? *reinterpret_cast<const uint4 *>(src + (size_t)mykey * D +
                                                                        32 * ks + 8 * g)
                                  : make_uint4(0, 0, 0, 0));
  floatx4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int rows_per_qt = d.bq * d.H;
  const int r0 = 8 * (j >> 2) + (j & 3);  // A-operand row for the first 16-row block
  for (int e = it.e0; e < it.e1; ++e) {
    const uint32_t ent = p.kvent[e];
    const int qt = (int)(ent & kEntIdx);
    const bool full = ent & kEntFull;
    for (int base = 0; base < rows_per_qt; base += STEP) {
      __syncthreads();
      // Stage rows base .. base+STEP-1 of query tile qt.
      for (int c = tid; c < RCH; c += 256) {
        const int r = c / (D / 8), col = c % (D / 8);
        const int rho = base + r;
        const int pos = qt * d.bq + rho / d.H, h = rho % d.H;
        uint4 qv = make_uint4(0, 0, 0, 0), dv = qv;
        if (pos < d.S) {
          const size_t row = ((size_t)b * d.H + h) * d.S + pos;
          qv = *reinterpret_cast<const uint4 *>(q + row * D + col * 8);
          dv = *reinterpret_cast<const uint4 *>(dout + row * D + col * 8);
        }
        *reinterpret_cast<uint4 *>(q_lds + r * QROW + (col ^ rsw(r)) * 8) = qv;
        *reinterpret_cast<uint4 *>(o_lds + r * QROW + (col ^ rsw(r)) * 8) = dv;
      }
      if (tid < STEP) {
        const int rho = base + tid;
        const int pos = qt * d.bq + rho / d.H, h = rho % d.H;
        if (pos < d.S) {
          const size_t row = ((size_t)b * d.H + h) * d.S + pos;
          const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pos];
          info_lds[tid] = make_int4(rw.x, rw.y, rw.z, pos);
          lse_lds[tid] = lse[row] * kLog2e;
          dl_lds[tid] = delta[row];
        } else {
          info_lds[tid] = make_int4(INT_MAX, 0, 0, INT_MAX);
          lse_lds[tid] = -INFINITY;
          dl_lds[tid] = 0.f;
        }
      }
      __syncthreads();

      // S and dP for this wave's 32 rows x 16 keys.
      const int wr = rh * 32;  // first staged row of this wave
      floatx4 s[2], t[2];
      s[0] = s[1] = t[0] = t[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int arow = wr + r0 + 4 * rb;
          const int slot = ((4 * ks + g) ^ rsw(arow)) * 8;
          const bf16x8 aq = as_bf16x8(lds_load16(q_lds + arow * QROW + slot));
          const bf16x8 ad = as_bf16x8(lds_load16(o_lds + arow * QROW + slot));
          s[rb] = mfma16x16x32(aq, kf[ks], s[rb]);
          t[rb] = mfma16x16x32(ad, kf[ks], t[rb]);
        }
      }
      // Lane holds rows wr + 8g + {0..3} (rb 0) and wr + 8g + 4 + {0..3} (rb 1)
      // for key `mykey`.
      float pv[8], dsv[8];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rr = wr + 8 * g + 4 * rb + v;
          const int4 inf = info_lds[rr];
          bool vis = true;
          if (!full)
            vis = comp ? (mykey >= inf.y && mykey < inf.z) : (mykey >= inf.x && mykey <= inf.w);
          const float pr = vis ? fast_exp2(s[rb][v] * scale_log2 - lse_lds[rr]) : 0.f;
          pv[4 * rb + v] = pr;
          dsv[4 * rb + v] = pr * (t[rb][v] - dl_lds[rr]) * scale;
        }
      const bf16x8 pb = pack8(pv), dsb = pack8(dsv);
      // dKV^T[d][key] += Q^T[d][rows] dS[rows][key] + dO^T[d][rows] P[rows][key].
      // Transposed A operand of column block db (d-row j, rows 8 g .. 8 g + 7
      // of this wave's half): lane reads 8 bytes of row wr + 8 g + (j >> 2),
      // logical chunk 2 db + ((j & 3) >> 1), half j & 1, and the same 4 rows
      // further down; the two transpose reads leave lane j with column j.
      {
        const int tr_row = wr + 8 * g + (j >> 2);  // rows tr_row + 4 share its swizzle
        const int c0 = (j & 3) >> 1, hb = (j & 1) * 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = tr_row * QROW * 2 + (((2 * db + c0) ^ rsw(tr_row)) << 4) + hb;
          const bf16x8 aq = tr_frag_rows(reinterpret_cast<const char *>(q_lds) + off, 4 * QROW * 2);
          const bf16x8 ad = tr_frag_rows(reinterpret_cast<const char *>(o_lds) + off, 4 * QROW * 2);
          acc[db] = mfma16x16x32(aq, dsb, acc[db]);
          acc[db] = mfma16x16x32(ad, pb, acc[db]);
        }
      }
    }
  }

  // Sum the two row-half partials of each key half, then write the item's
  // float32 partial [32 keys][D].
  __syncthreads();
  float *red = reinterpret_cast<float *>(q_lds);  // [2 key halves][D][16 keys]
  if (rh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(kh * D + 16 * db + 4 * g + v) * 16 + j] = acc[db][v];
  }
  __syncthreads();
  if (rh == 0) {
    float *out = part + it.part_off + (size_t)(kh * 16 + j) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      float4 w;
      w.x = acc[db][0] + red[(kh * D + 16 * db + 4 * g + 0) * 16 + j];
      w.y = acc[db][1] + red[(kh * D + 16 * db + 4 * g + 1) * 16 + j];
      w.z = acc[db][2] + red[(kh * D + 16 * db + 4 * g + 2) * 16 + j];
      w.w = acc[db][3] + red[(kh * D + 16 * db + 4 * g + 3) * 16 + j];
      *reinterpret_cast<float4 *>(out + 16 * db + 4 * g) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// 2b. dKV at D = 512, key-stationary.  A work item is a 128-key tile and a run
//     of query tiles that see it.  Query rows stream through LDS in 32-row
//     steps (Q and dO, 64 KiB, double-buffered, direct global->LDS copies,
//     swizzled rows).  Each step has two phases:
//       scores    wave w forms S = Q K^T and dP = dO K^T for all 32 rows and
//                 its 32 keys (K fragments of those keys held in VGPRs); then
//                 P = 2^(S log2e scale - LSE log2e), dS = scale P (dP - delta),
//                 stored as bf16 in exchange tiles in LDS (fragment order);
//       gradient  wave w accumulates dKV^T[d][key] += Q^T dS + dO^T P over the
//                 step's rows for its quarter of the columns, d in
//                 [128 w, 128 w + 128), and all 128 keys: A operands are
//                 ds_read_b64_tr_b16 reads of the row-major Q / dO tiles, B
//                 operands come from the exchange tile, and the fp32 sums
//                 (256 per lane) stay in accumulation registers for the item.
//     128 keys per item give each 64 KiB row copy 2 x 256 MFMAs per wave of
//     work, long enough to hide the copy of the next step behind it.
// ---------------------------------------------------------------------------
// Transposed A operand (d-row j of a 16-wide column block, rows 8g..8g+7 of
// the step) from a swizzled row-major [rows][512] tile: two transpose reads.
__device__ __forceinline__ bf16x8 tr_frag(const char *p) { return tr_frag_rows(p, 4096); }


template <int NW, int HALF>
__global__ void __launch_bounds__(NW * 64, 1)
    hca_bwd_dkv512_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                          const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                          const float *__restrict__ lse, const float *__restrict__ delta,
                          const bf16raw *__restrict__ dout, float scale_log2, float scale,
                          float *__restrict__ part, int slot0) {
  constexpr int D = 512, KS = D / 32;
  constexpr int KEYS = 128, STEP = 32, STEP_BYTES = STEP * 1024, XBYTES = KEYS * STEP * 2;
  static_assert(NW == 4, "4 waves: 32 score keys and one column quarter each");
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * STEP_BYTES];  // [buf][Q | dO]
  __shared__ __attribute__((aligned(16))) char xs[2 * XBYTES];             // [P | dS]
  // Row table per step slot: lse log2e, delta, first and one-past-last key.
  __shared__ float4 ri_s[2][STEP];

  // The wave index is made visibly wave-uniform so that the row bookkeeping
  // below runs on the scalar unit.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int item = p.kvorder[slot0 + blockIdx.x];
  if (item < 0) return;  // padding slot of the launch order
  const KvItem it = p.kvitem[item];
  const int b = it.b;
  const bool comp = it.kind != 0;
  const int nk = comp ? d.Sc : d.S;
  const int k0 = it.kt * KEYS;   // first key of the item
  const bf16raw *src = comp ? kvc + (size_t)b * d.Sc * D : kv + (size_t)b * d.S * D;

  const int nq = it.e1 - it.e0;
  // A query tile is bq positions x H heads (bq a power of two, bq * H a
  // multiple of 128), rows ordered position-fastest: row rho is position
  // qt * bq + (rho & (bq - 1)), head rho >> lbq.  SPQ steps of 32 rows each.
  const int lbq = __builtin_ctz(d.bq);
  const int SPQ = d.bq * d.H / STEP, lspq = __builtin_ctz(SPQ);
  const int nsteps = nq * SPQ;
  // Lane e holds list entry e; the entries past the first 64 (long
  // compressed-tile items) are read through the scalar cache.
  const uint32_t ent_lane = lane < nq ? p.kvent[it.e0 + lane] : 0u;
  auto entry = [&](int e) -> uint32_t {
    return e < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)ent_lane, e)
                  : uniform_load(p.kvent, it.e0 + e);
  };
  const size_t bat = (size_t)b * d.H * d.S * D;
  // Byte offset of this lane's 16-byte chunk in a staged row: row r = 8 wave + i
  // is stored with swizzle (i & 3) | (wave << 2).
  uint32_t lane_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lane_off[i] = (uint32_t)((lane ^ (i | (wave << 2))) << 4);
  // Step s covers rows u*32 .. u*32+31 of query tile entry e = s / SPQ.
  auto stage = [&](int s) {
    const int e = s >> lspq, u = s & (SPQ - 1);
    const int qt = (int)(entry(e) & kEntIdx);
    const uint32_t qb = lds_addr(smem + (s & 1) * 2 * STEP_BYTES);
#pragma unroll
    for (int i = 0; i < STEP / NW; ++i) {
      const int r = wave * (STEP / NW) + i;
      const int rho = u * STEP + r;
      const int pos = min(qt * d.bq + (rho & (d.bq - 1)), d.S - 1), h = rho >> lbq;
      const size_t rowoff = bat + ((size_t)h * d.S + pos) * D;  // wave-uniform
      dma16(q + rowoff, lane_off[i & 3], qb + r * 1024);
      dma16(dout + rowoff, lane_off[i & 3], qb + STEP_BYTES + r * 1024);
    }
  };
  // Row table of the next step (lse log2e, delta, key interval), loaded by
  // every wave while the current step computes and written to LDS by wave 0
  // at its end.  The loads are unconditional (clamped position) and their
  // values are not touched until then, so no wait for them lands mid-step.
  int4 nrw = make_int4(0, 0, 0, 0);
  float nl = 0.f, nd = 0.f;
  int npos = 0;
  auto rowinfo = [&](int s) {  // row (lane & 31) of step s
    const int e = s >> lspq, u = s & (SPQ - 1);
    const int qt = (int)(entry(e) & kEntIdx);
    const int rho = u * STEP + (lane & (STEP - 1));
    npos = qt * d.bq + (rho & (d.bq - 1));
    const int h = rho >> lbq, pc = min(npos, d.S - 1);
    const size_t row = ((size_t)b * d.H + h) * d.S + pc;
    nrw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pc];
    nl = lse[row];
    nd = delta[row];
  };
  auto put_rowinfo = [&](int slot) {
    if (wave == 0 && lane < STEP) {
      const bool ok = npos < d.S;
      float4 w;
      w.x = ok ? nl * kLog2e : 0.f;
      w.y = ok ? nd : 0.f;
      w.z = __int_as_float(ok ? (comp ? nrw.y : nrw.x) : INT_MAX);
      w.w = __int_as_float(ok ? (comp ? nrw.z : npos + 1) : 0);
      ri_s[slot][lane] = w;
    }
  };

  // Score-phase A operands: row i of row block rb maps to step row
  // 8 (i >> 2) + 4 rb + (i & 3), so lane (g, j) ends up holding rows
  // 8 g .. 8 g + 7 of key j of each 16-key block (4 rb + v for block rb).
  int qk_off[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
    qk_off[n] = (8 * (j >> 2) + (j & 3)) * 1024 + 16 * (4 * (n ^ (j >> 2)) + (g ^ (j & 3)));
  // Transpose-read offsets for the column blocks 8 wave + dl of this quarter.
  int tr_off[8];
  {
    const int u = j >> 2, c0 = (j & 3) >> 1;
#pragma unroll
    for (int dl = 0; dl < 8; ++dl)
      tr_off[dl] = (8 * g + u) * 1024 + (((2 * dl + c0) ^ (u + 4 * g)) << 4) + ((j & 1) << 3) +
                   256 * wave;
  }
  // Exchange tiles (P and dS, up to 8 key blocks of 1 KiB) in fragment order:
  // block kb holds keys 16 kb + j of the item's active keys, rows 8 g .. 8 g + 7
  // at byte 16 l of lane l = 16 g + j, both as the score phase produces them
  // and as the gradient reads them as B operands, so writes and reads are flat.
  const int xr0 = 16 * lane;

  // HALF = 0: the item runs over all 128 keys of its tile.  HALF = 1 (a
  // launch of its own, so its register allocation stays apart): items of
  // which no row sees one 64-key half of the tile (the planner marks them:
  // the first and last items of a sliding-window tile) run over the other
  // half only; each wave scores 16 keys, the gradient covers 4 key blocks,
  // and the idle half's partial is written as zeros.
  constexpr int KPW = HALF ? 1 : 2;  // 16-key score blocks per wave
  constexpr int NKB = 4 * KPW;       // active 16-key blocks of the item
  const int hh = HALF ? (it.halves == 2 ? 1 : 0) : 0;  // active half
  const int kbase = k0 + 64 * hh;
  const int kw = kbase + 16 * KPW * wave;  // first of this wave's score keys
  const int xw0 = 16 * lane + 1024 * KPW * wave;

  // K fragments of this wave's score keys, B[k = d][n = key] of S = Q K^T.
  // (Unconditional loads of a clamped key, zeroed past the end, so that all
  // the loads are in flight together.)
  bf16x8 kf[KPW][KS];
#pragma unroll
  for (int kb = 0; kb < KPW; ++kb) {
    const int key = kw + 16 * kb + j;
    const bf16raw *krow = src + (size_t)min(key, nk - 1) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4 *>(krow + 32 * ks + 8 * g);
      kf[kb][ks] = as_bf16x8(key < nk ? v : make_uint4(0, 0, 0, 0));
    }
  }
  floatx4 acc[NKB][8];  // [active 16-key block][16-column block of this wave's quarter]
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int dl = 0; dl < 8; ++dl) acc[kb][dl] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (nsteps > 0) {
    stage(0);
    rowinfo(0);
    put_rowinfo(0);
  }
  wait_all_loads();
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) rowinfo(s + 1);
    // Rows of the next step (on the last step: this step's rows again, into
    // the idle buffer), copied one instruction per score k-step below so the
    // wave never stalls issuing a burst of 16 copies.
    const int sn = min(s + 1, nsteps - 1);
    const int qt_n = (int)(entry(sn >> lspq) & kEntIdx), u_n = sn & (SPQ - 1);
    const uint32_t qb_n = lds_addr(smem + ((s + 1) & 1) * 2 * STEP_BYTES);
    auto copy_one = [&](int ks) {  // row ks >> 1 of this wave's 8, Q (even) or dO (odd)
      const int i = ks >> 1, r = wave * (STEP / NW) + i, rho = u_n * STEP + r;
      const int pos = min(qt_n * d.bq + (rho & (d.bq - 1)), d.S - 1), h = rho >> lbq;
      const size_t rowoff = bat + ((size_t)h * d.S + pos) * D;  // wave-uniform
      if (ks & 1)
        dma16(dout + rowoff, lane_off[i & 3], qb_n + STEP_BYTES + r * 1024);
      else
        dma16(q + rowoff, lane_off[i & 3], qb_n + r * 1024);
    };
    const int slot = s & 1;
    const bool full = entry(s >> lspq) & kEntFull;
    const char *qb = smem + slot * 2 * STEP_BYTES;
    const char *ob = qb + STEP_BYTES;
    __builtin_amdgcn_sched_barrier(0);

    // Scores: operand fragments are read PF k-steps ahead of their MFMAs.
    constexpr int PF = 1;
    floatx4 sv[2][KPW], pv[2][KPW];  // [row block][key block]
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < KPW; ++kb) sv[rb][kb] = pv[rb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
      bf16x8 fq[2][KS], fo[2][KS];
      auto qk_at = [&](int ks) { return qk_off[ks & 3] + 256 * (ks >> 2); };
      auto fetch = [&](int ks) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          fq[rb][ks] = lds_frag(qb + qk_at(ks) + 4096 * rb);
          fo[rb][ks] = lds_frag(ob + qk_at(ks) + 4096 * rb);
        }
      };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) fetch(ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        copy_one(ks);
        if (ks + PF < KS) fetch(ks + PF);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int kb = 0; kb < KPW; ++kb) {
            sv[rb][kb] = mfma16x16x32(fq[rb][ks], kf[kb][ks], sv[rb][kb]);
            pv[rb][kb] = mfma16x16x32(fo[rb][ks], kf[kb][ks], pv[rb][kb]);
          }
      }
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * KPW, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // P and dS of rows 8 g .. 8 g + 7 for this wave's keys -> exchange tile.
    {
      float4 ri[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) ri[r] = ri_s[slot][8 * g + r];
#pragma unroll
      for (int kb = 0; kb < KPW; ++kb) {
        const int key = kw + 16 * kb + j;
        float pr[8], ds[8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float4 rr = ri[4 * rb + v];
            // Branch-free: exp2 always, then a select (a branch per value would
            // cost more than the exp2 it skips).
            const bool vis =
                full | ((key >= __float_as_int(rr.z)) & (key < __float_as_int(rr.w)));
            const float ex = fast_exp2(sv[rb][kb][v] * scale_log2 - rr.x);
            const float e = vis ? ex : 0.f;
            pr[4 * rb + v] = e;
            ds[4 * rb + v] = e * (pv[rb][kb][v] - rr.y) * scale;
          }
        *reinterpret_cast<bf16x8 *>(xs + xw0 + 1024 * kb) = pack8(pr);
        *reinterpret_cast<bf16x8 *>(xs + XBYTES + xw0 + 1024 * kb) = pack8(ds);
      }
    }
    lds_barrier();  // exchange tile complete; the next step's copies stay in flight

    // Gradient, in two passes of four column blocks: the pass's transpose-read
    // fragments are held, the exchange fragments stream through (read one
    // key block ahead).
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      bf16x8 tq[4], to[4], xp[NKB], xd[NKB];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        tq[c] = tr_frag(qb + tr_off[4 * ps + c]);
        to[c] = tr_frag(ob + tr_off[4 * ps + c]);
      }
      xd[0] = lds_frag(xs + XBYTES + xr0);
      xp[0] = lds_frag(xs + xr0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb + 1 < NKB) {
          xd[kb + 1] = lds_frag(xs + XBYTES + xr0 + 1024 * (kb + 1));
          xp[kb + 1] = lds_frag(xs + xr0 + 1024 * (kb + 1));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[kb][4 * ps + c] = mfma16x16x32(tq[c], xd[kb], acc[kb][4 * ps + c]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[kb][4 * ps + c] = mfma16x16x32(to[c], xp[kb], acc[kb][4 * ps + c]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 16 + 2, 0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb + 1 < NKB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nsteps) put_rowinfo((s + 1) & 1);
    wait_all_loads();
    __syncthreads();
  }

  // Partial [128 keys][512] of this item: this wave's 128 columns of every key.
  // A half item writes zeros for its idle half, unless another half item of
  // the tile shares the block and writes that half itself.
  const bool shared = HALF && it.shared;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    float *out = part + it.part_off + (size_t)(16 * kb + j) * D + 128 * wave;
    const bool act = HALF ? (kb >> 2) == hh : true;
    if (shared && !act) continue;
    const int ka = HALF ? (kb & 3) : kb;  // active block of key block kb
#pragma unroll
    for (int dl = 0; dl < 8; ++dl) {
      float4 w;
      w.x = act ? acc[ka][dl][0] : 0.f;
      w.y = act ? acc[ka][dl][1] : 0.f;
      w.z = act ? acc[ka][dl][2] : 0.f;
      w.w = act ? acc[ka][dl][3] : 0.f;
      *reinterpret_cast<float4 *>(out + 16 * dl + 4 * g) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. Fixed-order sum of the partials of every key tile -> dKV / dKV_comp.
// ---------------------------------------------------------------------------
// One launch for the raw key tiles, one for the compressed ones; a workgroup
// takes one (key tile, chunk of the tile's [kv_bk][D] block).  Thread (g, c)
// sums the float4 column c of the tile's partial blocks i = g, g + G, g + 2 G,
// ... in increasing order (eight loads in flight), and the G group sums are
// added in group order.  The grouping is fixed, so the result is bitwise
// reproducible.  Raw tiles have a few blocks each (G = 1, 1024-element
// chunks); a compressed tile has tens to hundreds, streamed by G = 8 groups
// over 128-element chunks.
template <int G>
__global__ void __launch_bounds__(256)
    hca_dkv_reduce_kernel(Dims d, DevPlan p, const float *__restrict__ part, int dtype,
                          void *__restrict__ dkv, void *__restrict__ dkvc, int comp) {
  constexpr int C = 256 / G, CHUNK = 4 * C;  // float4 columns per group, elements per workgroup
  __shared__ float4 red[G][C];
  const int nkt = d.nkv_raw + d.nkv_comp;
  const int ntl = comp ? d.nkv_comp : d.nkv_raw;  // tiles of this launch per batch row
  const int per_tile = d.kv_bk * d.D / CHUNK;
  const int tile = blockIdx.x / per_tile, chunk = blockIdx.x - tile * per_tile;
  const int b = tile / ntl, kt = tile - b * ntl;
  const int t = comp ? d.nkv_raw + kt : kt;
  const int nk = comp ? d.Sc : d.S;
  // The tile's partial blocks: n consecutive [kv_bk][D] blocks from block `first`.
  const int first = p.kvtile[2 * (b * nkt + t)], n = p.kvtile[2 * (b * nkt + t) + 1];
  const int D = d.D;
  const int g = threadIdx.x / C, c = threadIdx.x % C;
  const int e = chunk * CHUNK + c * 4;
  const int key = kt * d.kv_bk + e / D, col = e % D;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](const float4 v) {
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  };
  if (n > g) {
    // Block i of the tile sits i blocks after the first (no per-item table load).
    const size_t blk = (size_t)d.kv_bk * D;
    const float *src = part + (size_t)first * blk + e;
    int i = g;
    for (; i + 7 * G < n; i += 8 * G) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4 *>(src + (i + u * G) * blk);
#pragma unroll
      for (int u = 0; u < 8; ++u) add(v[u]);
    }
    for (; i < n; i += G) add(*reinterpret_cast<const float4 *>(src + i * blk));
  }
  if constexpr (G > 1) {
    red[g][c] = a;
    __syncthreads();
    if (g != 0) return;
    a = red[0][c];
#pragma unroll
    for (int h = 1; h < G; ++h) add(red[h][c]);
  }
  if (key >= nk) return;
  const size_t off = ((size_t)b * nk + key) * D + col;
  if (dtype == HCA_BF16) {
    ushort4 w;
    w.x = f2bf(a.x);
    w.y = f2bf(a.y);
    w.z = f2bf(a.z);
    w.w = f2bf(a.w);
    *reinterpret_cast<ushort4 *>((bf16raw *)(comp ? dkvc : dkv) + off) = w;
  } else {
    *reinterpret_cast<float4 *>((float *)(comp ? dkvc : dkv) + off) = a;
  }
}

// Compute units of the current device rounded down to a multiple of 8 (the
// XCD count), cached per device (threads that race store the same value); 0
// if the device cannot be queried.
static int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    n = n >= 8 ? n / 8 * 8 : 8;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int launch_bwd_dq_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kv,
                       const void *kvc, const void *kvt, const void *kvct, const void *o,
                       const float *lse, const void *dout, float scale, void *dq, float *delta,
                       void *stream) {
  hipStream_t s = (hipStream_t)stream;
  const float sl2 = scale * kLog2e;
  auto go = [&](auto kernel, int nw, int groups) {
    hipLaunchKernelGGL(kernel, dim3(groups), dim3(nw * 64), 0, s, d, p, (const bf16raw *)q,
                       (const bf16raw *)kv, (const bf16raw *)kvc, (const bf16raw *)kvt,
                       (const bf16raw *)kvct, (const bf16raw *)o, lse, (const bf16raw *)dout, sl2,
                       scale, (bf16raw *)dq, delta);
  };
  switch (d.D) {
    case 512: {
      // Persistent: one workgroup per compute unit (each takes 128 KiB of
      // LDS), a multiple of 8 of them so every workgroup stays on one XCD.
      const int units = d.B * d.nqt * (d.bq * d.H / 64);
      const int cus = compute_units();
      if (cus <= 0) return (int)hipErrorInvalidDevice;
      go(hca_bwd_dq512_kernel<4>, 4, units < cus ? units : cus);
      break;
    }
    case 128: go(hca_bwd_dq_kernel<128, 8, 1>, 8, d.B * d.nqt * (d.bq * d.H / 128)); break;
    case 64: go(hca_bwd_dq_kernel<64, 8, 1>, 8, d.B * d.nqt * (d.bq * d.H / 128)); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_bwd_dkv_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kv,
                        const void *kvc, const float *lse, const float *delta,
                        const void *dout, float scale, float *part, void *stream) {
  if (d.n_items == 0) return hipSuccess;
  hipStream_t s = (hipStream_t)stream;
  const float sl2 = scale * kLog2e;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(d.n_items), dim3(256), 0, s, d, p, (const bf16raw *)q,
                       (const bf16raw *)kv, (const bf16raw *)kvc, lse, delta,
                       (const bf16raw *)dout, sl2, scale, part);
  };
  switch (d.D) {
    case 512:
      // Full-tile items, then the half-tile items (see the kernel).
      if (d.n_items_full > 0)
        hipLaunchKernelGGL((hca_bwd_dkv512_kernel<4, 0>), dim3(d.n_items_full), dim3(256), 0, s,
                           d, p, (const bf16raw *)q, (const bf16raw *)kv, (const bf16raw *)kvc,
                           lse, delta, (const bf16raw *)dout, sl2, scale, part, 0);
      if (d.n_items > d.n_items_full)
        hipLaunchKernelGGL((hca_bwd_dkv512_kernel<4, 1>), dim3(d.n_items - d.n_items_full),
                           dim3(256), 0, s, d, p, (const bf16raw *)q, (const bf16raw *)kv,
                           (const bf16raw *)kvc, lse, delta, (const bf16raw *)dout, sl2, scale,
                           part, d.n_items_full);
      break;
    case 128: go(hca_bwd_dkv_kernel<128>); break;
    case 64: go(hca_bwd_dkv_kernel<64>); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_dkv_reduce(const Dims &d, const DevPlan &p, const float *part, int dtype, void *dkv,
                      void *dkvc, void *stream) {
  // kv_bk * D is a multiple of 1024 for every kernel configuration (kv_bk >= 32, D >= 64).
  hipStream_t s = (hipStream_t)stream;
  const int raw_blk = d.B * d.nkv_raw * (d.kv_bk * d.D / 1024);
  const int comp_blk = d.B * d.nkv_comp * (d.kv_bk * d.D / 128);
  if (raw_blk > 0)
    hipLaunchKernelGGL(hca_dkv_reduce_kernel<1>, dim3(raw_blk), dim3(256), 0, s, d, p, part,
                       dtype, dkv, dkvc, 0);
  if (comp_blk > 0)
    hipLaunchKernelGGL(hca_dkv_reduce_kernel<8>, dim3(comp_blk), dim3(256), 0, s, d, p, part,
                       dtype, dkv, dkvc, 1);
  return (int)hipGetLastError();
}

}  // namespace hca
