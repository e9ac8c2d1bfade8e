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
//     or compressed; 64 or 128 keys at D = 512, 32 otherwise) and the query
//     tiles of a run of 64-position chunks that see it.  With 64-key tiles at
//     D = 512 the dQ kernel also stores P and scale dS (bf16) of every tile
//     it walks, and this kernel only forms Q^T dS + dO^T P from them; with
//     128-key tiles (and at D = 64 / 128) it recomputes S and dP with the
//     tile's K fragments held in VGPRs, and items whose rows see only one
//     64-key half of a 128-key tile run over that half.  Each item writes a
//     float32 partial.
//  3. a fixed-order reduction of the partials into dKV and dKV_comp, so the
//     result is bitwise reproducible.
#include <atomic>
#include <type_traits>
#include <climits>

#include "hca_device.h"
#include "hca_internal.h"
#include "hca_stage.h"

// Stored-P backward at D = 512: waves of the P / dS pass and of the streaming
// dQ pass, and the streaming pass's stages in flight.
#ifndef HCA_PDS_NW
#define HCA_PDS_NW 4
#endif
#ifndef HCA_DQS_NW
#define HCA_DQS_NW 8
#endif
#ifndef HCA_DQS_STAGES
#define HCA_DQS_STAGES 3
#endif

namespace hca {

namespace {

constexpr int kBK = 32;

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
  using St = KTile<D, NT>;
  __shared__ __attribute__((aligned(16))) bf16raw k_lds[kBK * D];

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

    floatx4 s0[MB], s1[MB], p0[MB], p1[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s0[mb] = s1[mb] = p0[mb] = p1[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a0 = St::kfrag(k_lds, r0, ks, g);
      const bf16x8 a1 = St::kfrag(k_lds, r1, ks, g);
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
      // The row's visible keys of this tile's kind, [lo, hi]; invisible keys
      // are dropped by selects.
      const int lo = comp ? clo[mb] : rlo[mb], hi = comp ? chi[mb] - 1 : pos[mb];
      const int kb = k0 + 8 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bool vis = full | ((kb + t >= lo) & (kb + t <= hi));
        const float pr = fast_exp2(x[t] - lse2[mb]);
        x[t] = vis ? pr * (dp[t] - dl[mb]) : 0.f;
      }
      dsb[mb] = pack8(x);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = St::tfrag(k_lds, db, g, j);
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
// MASKED: compressed visibility from the plan's mask bits (separate
// instantiation, as for the forward).  Used by plans whose key-stationary
// pass recomputes S and dP (128-key tiles); with stored P and dS the two
// passes 1c and 1d replace it.
template <int NW, bool MASKED>
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

    // Masked plans: the 32 visibility bits of this row for the compressed
    // tile of entry `e`, loaded when the entry becomes current (0 otherwise).
    auto mask_word = [&](uint32_t e) -> uint32_t {
      if constexpr (MASKED) {
        if ((e & kEntComp) && !(e & kEntFull) && valid)
          return p.cmask[((size_t)b * d.S + pos) * d.cmask_ldw + (e & kEntIdx)];
      }
      return 0u;
    };
    // dS of tile it from its scores, then dQ^T += K^T dS^T.
    auto grad = [&](int it, uint32_t ent, uint32_t mw) {
      const bool comp = ent & kEntComp;
      const int k0 = (int)(ent & kEntIdx) * kBK;
      float x[8];
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        x[v4] = sc[0][v4] * scale_log2 - lse2;
        x[4 + v4] = sc[1][v4] * scale_log2 - lse2;
      }
      if (!(ent & kEntFull)) {
        if (MASKED && comp) {
          const uint32_t bits = mw >> (8 * g);
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = ((bits >> t) & 1u) ? x[t] : -INFINITY;
        } else {
          const int lo = (comp ? clo : rlo) - (k0 + 8 * g);
          const int hi = (comp ? chi : pos + 1) - (k0 + 8 * g);
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = (t >= lo && t < hi) ? x[t] : -INFINITY;
        }
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
    uint32_t mw = mask_word(ent);
    const int last = nent - 1;
    for (int it = 0; it + 1 < last; ++it) {
      floatx4 sn[2], pn[2];
      sdp(it + 1, sn, pn);
      grad(it, ent, mw);
      sc[0] = sn[0];
      sc[1] = sn[1];
      pc[0] = pn[0];
      pc[1] = pn[1];
      wait_all_loads();
      __syncthreads();
      ent = entry(it + 1);
      mw = mask_word(ent);
      stage_k(it + 3);
      stage_t(it + 2);
    }
    // Once the last tile's scores are taken this unit's Q and dO rows are
    // dead: the next unit's entries and rows load from there on, under the
    // last two tiles and the store (one fetch site, so the loaded registers
    // need no copies that would wait for them).
    floatx4 sn[2], pn[2];
    uint32_t ent_last = 0u, mw_last = 0u;
    if (last >= 1) {
      ent_last = entry(last);  // before the fetch replaces the entries
      // (its mask word before the row loads too, so they stay the last ones issued)
      mw_last = mask_word(ent_last);
      sdp(last, sn, pn);
    }
    fetch(sl_n, item_n, e_begin_n, nent_n);
    // Nothing is scheduled across this point, so every load of fetch() is
    // issued before the wait below.
    __builtin_amdgcn_sched_barrier(0);
    if (last >= 1) {
      grad(last - 1, ent, mw);
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
      mw = mw_last;
    }
    if (last >= 0) grad(last, ent, mw);

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

// ---------------------------------------------------------------------------
// 1c. Stored-P backward at D = 512, first pass: P and dS only.  With 64-key
//     key tiles the key-stationary pass reads P and dS from the backward
//     workspace, and dQ = scale sum_k dS kv_k is formed by a second streaming
//     pass (1d) from the same stored dS, so this pass carries no dQ
//     accumulator: Q and dO fragments (128 registers) and the scores fit in
//     256 registers and two workgroups run per CU.  A workgroup is one slice
//     of 64 rows (4 waves x 16 consecutive positions of one head) of a query
//     tile; it walks the tile's list, K tiles double-buffered in LDS (copied
//     from the tile images), S^T and dP^T from shared K fragments, delta from
//     O and dO.  P and scale dS of tile t (bf16) are stored by each lane as
//     one 16-byte non-temporal store each, issued at the top of tile t + 1
//     so the tile-end wait does not wait for them: list entry e of the query
//     tile owns the block pds + e * 2 R * 64 bytes (R = bq H rows), P rows
//     then dS rows, 64 bytes per row, chunk c of row rho at position
//     c ^ ((rho >> 3) & 3).
// ---------------------------------------------------------------------------
template <int NW, bool MASKED>
__global__ void __launch_bounds__(NW * 64, 8 / NW)
    hca_bwd_pds512_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                          const bf16raw *__restrict__ kvt, const bf16raw *__restrict__ kvct,
                          const bf16raw *__restrict__ o, const float *__restrict__ lse,
                          const bf16raw *__restrict__ dout, float scale_log2, float scale,
                          float *__restrict__ delta, char *__restrict__ pds) {
  constexpr int D = 512, KS = D / 32, M = NW * 16;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytes512];  // K, double-buffered

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int nslices = d.bq * d.H / M;
  const int lbq = __builtin_ctz(d.bq);
  const int u = xcd_remap(blockIdx.x, d.B * d.nqt * nslices, 2 * nslices);
  const int li = u / nslices, sl = u - li * nslices;
  const int item = p.qorder[li];
  const int b = item / d.nqt, qt = item - b * d.nqt;
  const int rho = sl * M + wave * 16 + j;
  const int pos = qt * d.bq + (rho & (d.bq - 1)), hh = rho >> lbq;
  const bool valid = pos < d.S;
  const int pc = min(pos, d.S - 1);
  const size_t row = ((size_t)b * d.H + hh) * d.S + pc;

  const int e_begin = p.qptr[item], nent = p.qptr[item + 1] - e_begin;
  const uint32_t ent_lane = lane < nent ? p.qent[e_begin + lane] : 0u;
  auto entry = [&](int t) -> uint32_t {
    return t < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)ent_lane, t)
                  : uniform_load(p.qent, e_begin + t);
  };
  __builtin_amdgcn_s_waitcnt(0);
  const rsrc_t r_img =
      make_rsrc(kvt + (size_t)b * 2 * D * d.S_pad, (uint32_t)d.S_pad * D * 4);
  const rsrc_t r_imgc =
      make_rsrc(kvct + (size_t)b * 2 * D * d.Sc_pad, (uint32_t)d.Sc_pad * D * 4);
  auto stage_k = [&](int t) {
    if (t >= nent) return;
    const uint32_t ent = entry(t);
    stage_img512<NW>((ent & kEntComp) ? r_imgc : r_img, (int)(ent & kEntIdx) * kBK, 0,
                     smem + (t & 1) * kTileBytes512, wave, lane);
  };
  stage_k(0);

  // Rows (padded rows read row S - 1; their intervals are empty, so their P
  // and dS are zero), delta from O and dO.
  const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pc];
  const float lv = lse[row];
  uint4 qv[KS], dv[KS];
  float part = 0.f;
  {
    const bf16raw *qr = q + row * D + 8 * g, *dr = dout + row * D + 8 * g, *orow = o + row * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qv[ks] = *reinterpret_cast<const uint4 *>(qr + 32 * ks);
      dv[ks] = *reinterpret_cast<const uint4 *>(dr + 32 * ks);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      part += dot8(dv[ks], *reinterpret_cast<const uint4 *>(orow + 32 * ks));
  }
  const float dl = group_sum(part);
  if (valid && g == 0) delta[row] = dl;
  const int rlo = valid ? rw.x : INT_MAX;
  const int clo = valid ? rw.y : 0;
  const int chi = valid ? rw.z : 0;
  const float lse2 = valid ? lv * kLog2e : -INFINITY;
  wait_all_loads();
  __syncthreads();

  const int frag_off = 16 * lane;
  const size_t blk_bytes = 2 * (size_t)d.pds_rows * 64;
  char *const prow = pds + (size_t)rho * 64 + ((g ^ ((rho >> 3) & 3)) << 4);
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 pend_p = {0u, 0u, 0u, 0u}, pend_s = {0u, 0u, 0u, 0u};
  auto put = [&](int t) {  // P and dS of tile t, held since it was formed
    char *blk = prow + (size_t)(e_begin + t) * blk_bytes;
    __builtin_nontemporal_store(pend_p, reinterpret_cast<u32x4 *>(blk));
    __builtin_nontemporal_store(pend_s, reinterpret_cast<u32x4 *>(blk + (size_t)d.pds_rows * 64));
  };
  for (int it = 0; it < nent; ++it) {
    if (it > 0) put(it - 1);
    stage_k(it + 1);
    const uint32_t ent = entry(it);
    uint32_t mw = 0u;
    if constexpr (MASKED) {
      if ((ent & kEntComp) && !(ent & kEntFull) && valid)
        mw = p.cmask[((size_t)b * d.S + pos) * d.cmask_ldw + (ent & kEntIdx)];
    }
    // S^T and dP^T of tile it (shared K A-operands), K fragments read three
    // k-steps ahead of their MFMAs.
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, p0 = s0, p1 = s0;
    mfma_phase_begin();
    {
      constexpr int PF = 3;
      const char *kb = smem + (it & 1) * kTileBytes512 + frag_off;
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
        s0 = mfma16x16x32(a0[ks], as_bf16x8(qv[ks]), s0);
        s1 = mfma16x16x32(a1[ks], as_bf16x8(qv[ks]), s1);
        p0 = mfma16x16x32(a0[ks], as_bf16x8(dv[ks]), p0);
        p1 = mfma16x16x32(a1[ks], as_bf16x8(dv[ks]), p1);
      }
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
    mfma_phase_end();
    // P = 2^(S scale log2e - LSE log2e) on visible keys, dS = scale P (dP - delta).
    {
      const bool comp = ent & kEntComp;
      const int k0 = (int)(ent & kEntIdx) * kBK;
      float x[8], y[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[v] = s0[v] * scale_log2 - lse2;
        x[4 + v] = s1[v] * scale_log2 - lse2;
      }
      if (!(ent & kEntFull)) {
        if (MASKED && comp) {
          const uint32_t bits = mw >> (8 * g);
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = ((bits >> t) & 1u) ? x[t] : -INFINITY;
        } else {
          const int lo = (comp ? clo : rlo) - (k0 + 8 * g);
          const int hi = (comp ? chi : pos + 1) - (k0 + 8 * g);
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = (t >= lo && t < hi) ? x[t] : -INFINITY;
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[v] = fast_exp2(x[v]);
        x[4 + v] = fast_exp2(x[4 + v]);
        y[v] = x[v] * (p0[v] - dl) * scale;
        y[4 + v] = x[4 + v] * (p1[v] - dl) * scale;
      }
      pend_p = __builtin_bit_cast(u32x4, pack8(x));
      pend_s = __builtin_bit_cast(u32x4, pack8(y));
    }
    wait_all_loads();  // K of tile it + 1 (and the stores of tile it - 1)
    __syncthreads();   // K buffer it & 1 free
  }
  if (nent > 0) put(nent - 1);
}

// ---------------------------------------------------------------------------
// 1d. Stored-P backward at D = 512, second pass: dQ = sum over the listed
//     tiles of (scale dS) K, streamed from the stored dS.  A workgroup is a
//     slice of M = 16 NW rows of a query tile.  The product is split over D:
//     wave w accumulates dQ^T for columns (512 / NW) w .. of all M rows (128
//     registers), so each K^T fragment it reads from LDS feeds M / 16 MFMAs;
//     the dS B fragments are the stored rows themselves, copied to LDS with
//     the K^T tile (double-buffered) and read in place.  dQ is staged in LDS
//     at the end and stored as whole rows.
// ---------------------------------------------------------------------------
template <int NW>
__global__ void __launch_bounds__(NW * 64, 8 / NW)
    hca_bwd_dqs512_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ kvt,
                          const bf16raw *__restrict__ kvct, const char *__restrict__ pds,
                          bf16raw *__restrict__ dq) {
  constexpr int D = 512, M = NW * 16, RB = M / 16, CB = D / 16 / NW;
  constexpr int DSB = M * 64;                   // the slice's dS rows of one tile
  constexpr int STAGE = kTileBytes512 + DSB;    // K^T | dS
  constexpr int NST = HCA_DQS_STAGES;           // stages in flight
  constexpr int SMEM = NST * STAGE > M * 1024 ? NST * STAGE : M * 1024;
  constexpr int kCopies = 32 / NW + 1;          // copies per wave and stage
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];  // NST stages; dQ rows at the end

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int nslices = d.bq * d.H / M;
  const int lbq = __builtin_ctz(d.bq);
  const int u = xcd_remap(blockIdx.x, d.B * d.nqt * nslices, 2 * nslices);
  const int li = u / nslices, sl = u - li * nslices;
  const int item = p.qorder[li];
  const int b = item / d.nqt, qt = item - b * d.nqt;
  const int e_begin = p.qptr[item], nent = p.qptr[item + 1] - e_begin;
  const uint32_t ent_lane = lane < nent ? p.qent[e_begin + lane] : 0u;
  auto entry = [&](int t) -> uint32_t {
    return t < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)ent_lane, t)
                  : uniform_load(p.qent, e_begin + t);
  };
  __builtin_amdgcn_s_waitcnt(0);
  const rsrc_t r_img =
      make_rsrc(kvt + (size_t)b * 2 * D * d.S_pad, (uint32_t)d.S_pad * D * 4);
  const rsrc_t r_imgc =
      make_rsrc(kvct + (size_t)b * 2 * D * d.Sc_pad, (uint32_t)d.Sc_pad * D * 4);
  const size_t blk_bytes = 2 * (size_t)d.pds_rows * 64;
  // Stage of tile t: its K^T tile, and the slice's rows of its stored dS
  // (M x 64 bytes, contiguous; wave w copies rows 16 w .. 16 w + 15).
  auto stage = [&](int t) {
    if (t >= nent) return;
    const uint32_t ent = entry(t);
    char *st = smem + (t % NST) * STAGE;
    stage_img512<NW>((ent & kEntComp) ? r_imgc : r_img, (int)(ent & kEntIdx) * kBK, 1, st,
                     wave, lane);
    dma16(pds + (size_t)(e_begin + t) * blk_bytes + (size_t)d.pds_rows * 64 +
              (size_t)(sl * M + 16 * wave) * 64,
          16 * lane, lds_addr(st + kTileBytes512 + wave * 1024));
  };

  floatx4 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < CB; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Stages of tiles 0 .. NST - 2 go out first; tile it + NST - 1 is copied at
  // the top of iteration it, into the stage tile it - 1 used.
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) stage(t);
  const int frag_off = 16 * lane;
  // dS B fragment of row block rb: row 16 rb + j, stored chunk g at position
  // g ^ ((row >> 3) & 3) (the slice starts on a multiple of 64 rows).
  auto ds_off = [&](int rb) { return rb * 1024 + j * 64 + ((g ^ ((2 * rb + (j >> 3)) & 3)) << 4); };
  for (int it = 0; it < nent; ++it) {
    // This wave's copies of tile it have landed once at most the later
    // stages' copies are outstanding (copies complete in issue order); the
    // barrier covers the other waves' and frees the stage tile it - 1 used.
    const int later = min(NST - 2, nent - 1 - it);
    if (later >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * kCopies) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kCopies) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    stage(it + NST - 1);
    const char *st = smem + (it % NST) * STAGE;
    const char *tb = st + wave * CB * 1024 + frag_off;
    mfma_phase_begin();
    bf16x8 kt[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) kt[c] = lds_frag(tb + c * 1024);
    bf16x8 df = lds_frag(st + kTileBytes512 + ds_off(0));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bf16x8 cur = df;
      if (rb + 1 < RB) df = lds_frag(st + kTileBytes512 + ds_off(rb + 1));
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[rb][c] = mfma16x16x32(kt[c], cur, acc[rb][c]);
    }
    mfma_phase_end();
  }
  __syncthreads();  // every stage read before the rows are staged over them

  // dQ rows as bf16 into LDS (row r at r * 1024, chunk c at c ^ (r & 15)),
  // then every wave stores 16 whole rows.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + j;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      ushort4 w;
      w.x = f2bf(acc[rb][c][0]);
      w.y = f2bf(acc[rb][c][1]);
      w.z = f2bf(acc[rb][c][2]);
      w.w = f2bf(acc[rb][c][3]);
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
      *reinterpret_cast<uint4 *>(dq + (((size_t)b * d.H + hr) * d.S + pr) * D + 8 * lane) = v;
    }
  }
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
__global__ void __launch_bounds__(256, 4)
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
  __shared__ __attribute__((aligned(16))) float lse_lds[STEP];
  __shared__ __attribute__((aligned(16))) float dl_lds[STEP];
  __shared__ __attribute__((aligned(16))) int2 vis_lds[STEP];  // the row's keys of this kind: [lo, hi]

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

  // Steps of STEP rows: step s covers rows (s % spq) STEP .. + STEP - 1 of the
  // query tile of entry e0 + s / spq (a query tile holds spq whole steps).
  // Four workgroups share a CU (at most 128 registers per lane), so one
  // workgroup's row loads run under the others' math; a step's loads are
  // issued before the barrier that frees the LDS rows.
  // H and bq H / STEP are powers of two (bf16 plans), so row indices split
  // into position and head by shifts.
  const int lh = __builtin_ctz(d.H);
  const int lspq = __builtin_ctz(d.bq * d.H / STEP);
  const int spq = 1 << lspq;
  const int nsteps = (it.e1 - it.e0) << lspq;
  const int r0 = 8 * (j >> 2) + (j & 3);  // A-operand row for the first 16-row block
  constexpr int CPT = RCH / 256;           // 16-B chunks per thread and tensor
  static_assert(RCH % 256 == 0, "whole chunks per thread");
  const bf16raw *qb = q + (size_t)b * d.H * d.S * D;
  const bf16raw *ob = dout + (size_t)b * d.H * d.S * D;
  uint4 nq[CPT], nd[CPT];
  int2 nvis = make_int2(INT_MAX, -1);
  float nlse = -INFINITY, ndl = 0.f;
  auto fetch = [&](int st) {
    const int qt = (int)(p.kvent[it.e0 + (st >> lspq)] & kEntIdx);
    const int base = (st & (spq - 1)) * STEP;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * 256;
      const int r = c / NCH, col = c % NCH;
      const int rho = base + r;
      const int pos = qt * d.bq + (rho >> lh), h = rho & (d.H - 1);
      const bool ok = pos < d.S;
      // Rows past the end read row 0 of the head and are zeroed.
      const size_t off = ((size_t)h * d.S + (ok ? pos : 0)) * D + col * 8;
      const uint4 vq = *reinterpret_cast<const uint4 *>(qb + off);
      const uint4 vd = *reinterpret_cast<const uint4 *>(ob + off);
      const uint32_t m = ok ? 0xffffffffu : 0u;
      nq[u] = make_uint4(vq.x & m, vq.y & m, vq.z & m, vq.w & m);
      nd[u] = make_uint4(vd.x & m, vd.y & m, vd.z & m, vd.w & m);
    }
    if (tid < STEP) {
      const int rho = base + tid;
      const int pos = qt * d.bq + (rho >> lh), h = rho & (d.H - 1);
      nvis = make_int2(INT_MAX, -1);  // padded rows see no key
      nlse = -INFINITY;
      ndl = 0.f;
      if (pos < d.S) {
        const size_t row = ((size_t)b * d.H + h) * d.S + pos;
        const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + pos];
        // Raw keys rlo .. pos, compressed entries clo .. chi - 1.
        nvis = comp ? make_int2(rw.y, rw.z - 1) : make_int2(rw.x, pos);
        nlse = lse[row] * kLog2e;
        ndl = delta[row];
      }
    }
  };
  for (int st = 0; st < nsteps; ++st) {
    {
      const bool full = p.kvent[it.e0 + (st >> lspq)] & kEntFull;
      fetch(st);
      lds_barrier();  // every wave is done with the previous step's rows
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = tid + u * 256;
        const int r = c / NCH, col = c % NCH;
        *reinterpret_cast<uint4 *>(q_lds + r * QROW + (col ^ rsw(r)) * 8) = nq[u];
        *reinterpret_cast<uint4 *>(o_lds + r * QROW + (col ^ rsw(r)) * 8) = nd[u];
      }
      if (tid < STEP) {
        vis_lds[tid] = nvis;
        lse_lds[tid] = nlse;
        dl_lds[tid] = ndl;
      }
      lds_barrier();

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
      // The lane's 8 rows are consecutive: their intervals, LSE and delta are
      // read together, and invisible entries are dropped by selects.
      float pv[8], dsv[8];
      {
        const int rq = wr + 8 * g;
        int4 vr[4];  // rows rq + 2 u and rq + 2 u + 1: lo, hi, lo, hi
#pragma unroll
        for (int u = 0; u < 4; ++u) vr[u] = *reinterpret_cast<const int4 *>(vis_lds + rq + 2 * u);
        const float4 l0 = *reinterpret_cast<const float4 *>(lse_lds + rq);
        const float4 l1 = *reinterpret_cast<const float4 *>(lse_lds + rq + 4);
        const float4 q0 = *reinterpret_cast<const float4 *>(dl_lds + rq);
        const float4 q1 = *reinterpret_cast<const float4 *>(dl_lds + rq + 4);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float dv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int i = 4 * rb + v;
            const int lo = (i & 1) ? vr[i >> 1].z : vr[i >> 1].x;
            const int hi = (i & 1) ? vr[i >> 1].w : vr[i >> 1].y;
            const bool in = (mykey >= lo) & (mykey <= hi);
            const float e = fast_exp2(s[rb][v] * scale_log2 - lv[i]);
            const float pr = (full | in) ? e : 0.f;
            pv[i] = pr;
            dsv[i] = pr * (t[rb][v] - dv[i]) * scale;
          }
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

// Transposed A operand (d-row j of a 16-wide column block, rows 8g..8g+7 of
// a step) from a swizzled row-major [rows][512] tile: two transpose reads.
__device__ __forceinline__ bf16x8 tr_frag(const char *p) { return tr_frag_rows(p, 4096); }

// ---------------------------------------------------------------------------
// 2b. dKV at D = 512, key-stationary, eight waves (two per SIMD).  A work
//     item is a 128-key tile and the query tiles of one chunk of positions
//     that see it.  Query rows stream through LDS in 32-row steps (Q and dO,
//     64 KiB, double-buffered, direct global->LDS copies, rows stored with
//     their 16-byte chunks XOR-swizzled).  Each step has two phases:
//       scores    S = Q K^T and dP = dO K^T for the wave's keys (K fragments
//                 held in VGPRs); P = 2^(S log2e scale - LSE log2e), dS =
//                 scale P (dP - delta), stored as bf16 in exchange tiles in
//                 LDS in MFMA fragment order;
//       gradient  dKV^T[d][key] += Q^T dS + dO^T P over the step's rows, A
//                 operands from ds_read_b64_tr_b16 reads of the row tiles,
//                 B operands from the exchange tiles.
//     Wave w holds the K fragments of 16 keys (64
//     registers) and accumulates dKV^T for 64 columns, d in [64 w, 64 w + 64),
//     over all 128 keys (128 accumulation registers), so each wave needs at
//     most 256 registers and a SIMD runs two waves.  (A four-wave version,
//     32 score keys and 256 accumulators per wave, one wave per SIMD, ran
//     8.9 ms at S = 65536 against 8.6 for this one.)  Used with 128-key
//     tiles (plans whose stored P / dS would pass the planner's budget, or
//     kv_keys = 128); 64-key plans use 2c.  Items over
//     all keys of their tile and items over one 64-key half run in the same
//     launch (a wave-uniform branch per item), so both kinds
//     stream the rows of one chunk together through the L2.
//       full item  wave w scores keys 16 w .. 16 w + 15 of the tile for the
//                  step's 32 rows; the gradient covers key blocks 0..7.
//       half item  wave w scores keys 16 (w & 3) .. of the active half for
//                  row block w >> 2 (16 rows); the gradient covers the half's
//                  four key blocks.
// ---------------------------------------------------------------------------
// MASKED: compressed visibility from the plan's mask bits (separate
// instantiation): each step row's 128 bits of the item's tile travel with the
// row table.
template <bool MASKED>
__global__ void __launch_bounds__(512, 1)
    hca_bwd_dkv512x8_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                            const bf16raw *__restrict__ kv, const bf16raw *__restrict__ kvc,
                            const float *__restrict__ lse, const float *__restrict__ delta,
                            const bf16raw *__restrict__ dout, float scale_log2, float scale,
                            float *__restrict__ part) {
  constexpr int D = 512, KS = D / 32;
  constexpr int STEP = 32, STEP_BYTES = STEP * 1024, XBYTES = 128 * STEP * 2;
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * STEP_BYTES];  // [buf][Q | dO]
  __shared__ __attribute__((aligned(16))) char xs[2 * XBYTES];             // [P | dS]
  __shared__ float4 ri_s[2][STEP];  // per step row: lse log2e, delta, key interval
  // Masked plans: per step slot, the 128 visibility bits of the item's tile
  // for rows lane & 31 (lanes 32..63 copy the same rows again).
  __shared__ __attribute__((aligned(16))) uint4 rm_s[MASKED ? 2 : 1][MASKED ? 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int item = p.kvorder[blockIdx.x];
  if (item < 0) return;  // padding slot of the launch order
  const KvItem it = p.kvitem[item];
  const int b = it.b;
  const bool comp = it.kind != 0;
  const int nk = comp ? d.Sc : d.S;
  const int k0 = it.kt * 128;
  const bf16raw *src = comp ? kvc + (size_t)b * d.Sc * D : kv + (size_t)b * d.S * D;
  const int nq = it.e1 - it.e0;
  const int lbq = __builtin_ctz(d.bq);
  const int SPQ = d.bq * d.H / STEP, lspq = __builtin_ctz(SPQ);
  const int nsteps = nq * SPQ;
  const uint32_t ent_lane = lane < nq ? p.kvent[it.e0 + lane] : 0u;
  auto entry = [&](int e) -> uint32_t {
    return e < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)ent_lane, e)
                  : uniform_load(p.kvent, it.e0 + e);
  };
  const size_t bat = (size_t)b * d.H * d.S * D;
  // Wave w stages rows 4 w .. 4 w + 3 of each step; row r's chunk c sits at
  // slot c ^ sw(r), sw(r) = (r & 3) | ((r >> 3) << 2).
  const uint32_t lane_sw = (uint32_t)(lane ^ ((wave >> 1) << 2));
  auto copy_row = [&](int s, uint32_t qb_lds, int k) {  // row k >> 1 of this wave, Q or dO
    const int e = s >> lspq, u = s & (SPQ - 1);
    const int qt = (int)(entry(e) & kEntIdx);
    const int i = k >> 1, r = 4 * wave + i, rho = u * STEP + r;
    const int pos = min(qt * d.bq + (rho & (d.bq - 1)), d.S - 1), h = rho >> lbq;
    const size_t rowoff = bat + ((size_t)h * d.S + pos) * D;  // wave-uniform
    const uint32_t voff = (lane_sw ^ (uint32_t)i) << 4;
    if (k & 1)
      dma16(dout + rowoff, voff, qb_lds + STEP_BYTES + r * 1024);
    else
      dma16(q + rowoff, voff, qb_lds + r * 1024);
  };
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
    // Masked: the row's 128 bits of the item's tile (words k0 / 32 .. + 3) go
    // straight to LDS (no registers); waited for with the row copies.  A
    // padded row reads its clamped row's bits; the softmax ignores them.
    if (MASKED && comp && wave == 0)
      dma16(p.cmask, (uint32_t)((((size_t)b * d.S + pc) * d.cmask_ldw + k0 / 32) * 4),
            lds_addr(&rm_s[MASKED ? (s & 1) : 0][0]));
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
  // Score A operands: lane j reads step row 8 (j >> 2) + (j & 3) (+ 4 for row
  // block 1), chunk 4 ks + g, so lane (g, j) ends up with rows 8 g + 4 rb + v
  // (v = 0..3) of key j of its 16-key block.
  const int qk_base = (8 * (j >> 2) + (j & 3)) * 1024 + 16 * (g ^ (j & 3));
  // Transposed A operands of the gradient, column block 4 wave + dl: d-row j,
  // rows 8 g .. 8 g + 7 (two transpose reads, rows 8 g + (j >> 2) and + 4).
  const int tr_sw = (8 * (wave & 1) + ((j & 3) >> 1)) ^ ((j >> 2) + 4 * g);
  const int tr_base = (8 * g + (j >> 2)) * 1024 + 256 * (wave >> 1) + ((j & 1) << 3);
  const int xr0 = 16 * lane;

  const bool half = it.halves != 3;
  const int hh = it.halves == 2 ? 1 : 0;  // active half of a half item
  // This wave's 16 score keys.
  const int skey = half ? k0 + 64 * hh + 16 * (wave & 3) : k0 + 16 * wave;
  bf16x8 kf[KS];
  {
    const int key = skey + j;
    const bf16raw *krow = src + (size_t)min(key, nk - 1) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4 *>(krow + 32 * ks + 8 * g);
      kf[ks] = as_bf16x8(key < nk ? v : make_uint4(0, 0, 0, 0));
    }
  }
  floatx4 acc[8][4];  // [key block][column block of this wave]
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int dl = 0; dl < 4; ++dl) acc[kb][dl] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (nsteps > 0) {
    const uint32_t qb0 = lds_addr(smem);
#pragma unroll
    for (int k = 0; k < 8; ++k) copy_row(0, qb0, k);
    rowinfo(0);
    put_rowinfo(0);
  }
  wait_all_loads();
  __syncthreads();

  // One step of `HALF` kind: scores, P / dS to the exchange tiles, gradient.
  auto steps = [&](auto half_tag) {
    constexpr int HALF = decltype(half_tag)::value;
    constexpr int NRB = HALF ? 1 : 2;  // row blocks scored by this wave
    constexpr int NKB = HALF ? 4 : 8;  // key blocks of the gradient
    const int rb0 = HALF ? (wave >> 2) : 0;
    const int xblk = HALF ? (wave & 3) : wave;  // exchange block this wave writes
    for (int s = 0; s < nsteps; ++s) {
      const int sn = min(s + 1, nsteps - 1);
      const uint32_t qb_n = lds_addr(smem + ((s + 1) & 1) * 2 * STEP_BYTES);
      const int slot = s & 1;
      const bool full = entry(s >> lspq) & kEntFull;
      // Per-step opaque copies of the lane offsets: left visible, the
      // compiler hoists every derived address out of the step loop and has
      // to spill them.
      int qkb = qk_base, trb = tr_base, xr = xr0;
      asm volatile("" : "+v"(qkb), "+v"(trb), "+v"(xr));
      const char *qb = smem + slot * 2 * STEP_BYTES;
      const char *ob = qb + STEP_BYTES;
      __builtin_amdgcn_sched_barrier(0);

      // Scores, one row block after the other: fragments of k-step ks + 1 are
      // read while the MFMAs of ks run (group barriers keep the compiler from
      // hoisting every read).  The next step's rows are copied during the
      // first row block, one instruction per two k-steps.
      floatx4 sv[NRB], pv[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        sv[rb] = pv[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int rbo = 4096 * (rb0 + rb);
        bf16x8 fq[KS], fo[KS];
        auto fetch = [&](int ks) {
          const int off = qkb + 64 * ((ks & 3) ^ (j >> 2)) + 256 * (ks >> 2) + rbo;
          fq[ks] = lds_frag(qb + off);
          fo[ks] = lds_frag(ob + off);
        };
        fetch(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (rb == 0 && (ks & 1) == 0) copy_row(sn, qb_n, ks >> 1);
          if (ks + 1 < KS) fetch(ks + 1);
          sv[rb] = mfma16x16x32(fq[ks], kf[ks], sv[rb]);
          pv[rb] = mfma16x16x32(fo[ks], kf[ks], pv[rb]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // P and dS of rows 8 g + 4 rb + v (v = 0..3) for key skey + j: bytes
      // 8 rb .. 8 rb + 7 of this lane's 16 in the exchange block.
      {
        const int key = skey + j;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          bf16x4 pp, dd;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 8 * g + 4 * (rb0 + rb) + v;
            const float4 rr = ri_s[slot][row];
            bool vis;
            if (MASKED && comp) {
              // the word of this lane's key (a padded row's interval start is
              // INT_MAX: never visible)
              const int kk = key - k0;
              const uint32_t word =
                  reinterpret_cast<const uint32_t *>(&rm_s[MASKED ? slot : 0][row])[kk >> 5];
              vis = full | ((((word >> (kk & 31)) & 1u) != 0) &
                            (__float_as_int(rr.z) != INT_MAX));
            } else {
              vis = full | ((int)(key >= __float_as_int(rr.z)) & (int)(key < __float_as_int(rr.w)));
            }
            const float ex = fast_exp2(sv[rb][v] * scale_log2 - rr.x);
            const float e = vis ? ex : 0.f;
            pp[v] = (__bf16)e;
            dd[v] = (__bf16)(e * (pv[rb][v] - rr.y) * scale);
          }
          const int xo = xr + 8 * (rb0 + rb) + 1024 * xblk;
          *reinterpret_cast<bf16x4 *>(xs + xo) = pp;
          *reinterpret_cast<bf16x4 *>(xs + XBYTES + xo) = dd;
        }
      }
      lds_barrier();  // exchange tiles complete; the next step's copies stay in flight
      // Next step's row table, loaded under the gradient and stored after it.
      if (s + 1 < nsteps) rowinfo(s + 1);

      // Gradient, two passes of two column blocks: the pass's transposed row
      // fragments are held while the exchange fragments stream through.
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        bf16x8 tq[2], to[2], xd[NKB], xp[NKB];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int to_ = trb + ((tr_sw ^ (2 * (2 * ps + c))) << 4);
          tq[c] = tr_frag(qb + to_);
          to[c] = tr_frag(ob + to_);
        }
        xd[0] = lds_frag(xs + XBYTES + xr);
        xp[0] = lds_frag(xs + xr);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if (kb + 1 < NKB) {
            xd[kb + 1] = lds_frag(xs + XBYTES + xr + 1024 * (kb + 1));
            xp[kb + 1] = lds_frag(xs + xr + 1024 * (kb + 1));
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            acc[kb][2 * ps + c] = mfma16x16x32(tq[c], xd[kb], acc[kb][2 * ps + c]);
            acc[kb][2 * ps + c] = mfma16x16x32(to[c], xp[kb], acc[kb][2 * ps + c]);
          }
        }
        // 8 transpose reads and the first exchange pair, then per key block
        // the next pair and four MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 8 + 2, 0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if (kb + 1 < NKB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < nsteps) put_rowinfo((s + 1) & 1);
      wait_all_loads();
      __syncthreads();
    }
  };
  if (half)
    steps(std::integral_constant<int, 1>{});
  else
    steps(std::integral_constant<int, 0>{});

  // Partial [128 keys][512] of this item: this wave's 64 columns of every key.
  // A half item's accumulators 0..3 hold its active half; it writes zeros for
  // the idle half unless another half item of the tile shares the block.
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const bool act = !half || (kb >> 2) == hh;
    if (half && it.shared && !act) continue;
    const int ka = half ? (kb & 3) : kb;
    float *out = part + it.part_off + (size_t)(16 * kb + j) * D + 64 * wave + 4 * g;
#pragma unroll
    for (int dl = 0; dl < 4; ++dl) {
      float4 w;
      w.x = act ? acc[ka][dl][0] : 0.f;
      w.y = act ? acc[ka][dl][1] : 0.f;
      w.z = act ? acc[ka][dl][2] : 0.f;
      w.w = act ? acc[ka][dl][3] : 0.f;
      *reinterpret_cast<float4 *>(out + 16 * dl) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// 2c. dKV at D = 512 from stored P and dS (64-key tiles).  The dQ pass has
//     already formed P and scale * dS (bf16) of every listed (query tile,
//     32-key tile) pair; this pass only accumulates dKV^T[d][key] += Q^T dS +
//     dO^T P.  One workgroup of four waves per work item (a 64-key tile and
//     the query tiles of a run of 64-position chunks that see it), two
//     workgroups per CU.  Per 32-row step, Q and dO rows (64 KiB, chunks
//     XOR-swizzled) and the P / dS rows of the tile's two 32-key halves
//     (8 KiB, as stored) are copied straight to LDS, single-buffered, in two
//     halves: Q with dS, dO with P.  Each half's copy runs under the math of
//     the other half (and the other workgroup on the CU covers the rest of
//     the wait).  Wave w accumulates columns d in [128 w, 128 w + 128) of all
//     64 keys (128 fp32 sums per lane); the A operands are transpose reads of
//     the row tiles, the B operands transpose reads of the P / dS tiles.  A half that the query tile does not list is
//     read as zeros (an empty buffer range).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256, 2)
    hca_bwd_dkv512s_kernel(Dims d, DevPlan p, const bf16raw *__restrict__ q,
                           const bf16raw *__restrict__ dout, const char *__restrict__ pds,
                           float *__restrict__ part) {
  constexpr int D = 512, STEP = 32, STEP_BYTES = STEP * 1024;
  constexpr int PT = STEP * 64;  // bytes of one stored half-tile step (32 rows x 32 keys)
  // Copy instructions per wave and half-step: kRowCopies rows of Q or dO and
  // one KiB of dS or P.  The hand-counted waits below rely on these being the
  // only vector-memory instructions between them.
  constexpr int kRowCopies = 8, kHalfCopies = kRowCopies + 1;
  static_assert(4 * kRowCopies == STEP, "four waves copy the step's rows, one per copy");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STEP_BYTES];  // [Q | dO]
  __shared__ __attribute__((aligned(1024))) char ps[4 * PT];           // [P lo|P hi|dS lo|dS hi]

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int item = p.kvorder[blockIdx.x];
  if (item < 0) return;  // padding slot of the launch order
  const KvItem it = p.kvitem[item];
  const int b = it.b;
  const int nq = it.e1 - it.e0;
  const int lbq = __builtin_ctz(d.bq);
  const int SPQ = d.bq * d.H / STEP, lspq = __builtin_ctz(SPQ);
  const int nsteps = nq * SPQ;
  const size_t blk_bytes = 2 * (size_t)d.pds_rows * 64;  // one list entry's P and dS
  const size_t bat = (size_t)b * d.H * d.S * D;
  const uint32_t qb_lds = lds_addr(smem);
  // Wave w stages rows 8 w .. 8 w + 7 of Q and dO; row r's chunk c sits at slot
  // c ^ sw(r), sw(r) = (r & 3) | ((r >> 3) << 2).  Wave w also copies stored
  // block w (P lo, P hi, dS lo, dS hi): 2 KiB, two 1 KiB copies.
  const uint32_t lane_sw = (uint32_t)(lane ^ (wave << 2));
  // The wave's 8 rows of a step are 8 consecutive positions of one head (bq
  // is a power of two >= 8), so away from the sequence end they are 8 KiB
  // in a row: one base address, row i at i KiB.
  uint32_t voff_row[kRowCopies];
#pragma unroll
  for (int i = 0; i < kRowCopies; ++i)
    voff_row[i] = ((lane_sw ^ (uint32_t)(i & 3)) << 4) + 1024u * i;
  // Half-step copies: tensor 0 = the Q rows and both dS halves, tensor 1 =
  // the dO rows and both P halves.
  auto stage = [&](int s, int tensor) {
    const int e = s >> lspq, u = s & (SPQ - 1);
    const int qt = (int)(uniform_load(p.kvent, it.e0 + e) & kEntIdx);
    const int rho0 = u * STEP + 8 * wave;
    const int pos0 = qt * d.bq + (rho0 & (d.bq - 1)), h0 = rho0 >> lbq;
    const bf16raw *src_rows = tensor ? dout : q;
    const uint32_t rows_lds = qb_lds + tensor * STEP_BYTES;
    if (pos0 + kRowCopies - 1 < d.S) {
      const size_t rowoff = bat + ((size_t)h0 * d.S + pos0) * D;  // wave-uniform
#pragma unroll
      for (int i = 0; i < kRowCopies; ++i)
        dma16(src_rows + rowoff, voff_row[i], rows_lds + (8 * wave + i) * 1024);
    } else {
      // Last positions: rows past the end read the last row (never used).
#pragma unroll
      for (int i = 0; i < kRowCopies; ++i) {
        const int r = 8 * wave + i;
        const int pos = min(pos0 + i, d.S - 1);
        const size_t rowoff = bat + ((size_t)h0 * d.S + pos) * D;  // wave-uniform
        const uint32_t voff = (lane_sw ^ (uint32_t)(i & 3)) << 4;
        dma16(src_rows + rowoff, voff, rows_lds + r * 1024);
      }
    }
    // Wave w: KiB (w & 1) of half (w >> 1) of the step's dS (tensor 0) or P.
    const int half = wave >> 1;
    const int ent = (int)uniform_load((const uint32_t *)p.kvpe, 2 * (it.e0 + e) + half);
    const char *src = pds + (ent >= 0 ? (size_t)ent * blk_bytes : 0) +
                      (size_t)(1 - tensor) * d.pds_rows * 64 + (size_t)u * PT;
    const rsrc_t r = make_rsrc(src, ent >= 0 ? PT : 0);
    const int blk = 2 * (1 - tensor) + half;
    buf_load16(r, lds_addr(ps + blk * PT + (wave & 1) * 1024), (wave & 1) * 1024 + 16 * lane);
  };
  // Transposed A operands of column block 8 wave + dl: chunk 16 wave + 2 dl +
  // c0 of rows 8 g + (j >> 2) (and + 4) of the swizzled row tiles.
  const int tr_sw = ((j & 3) >> 1) ^ ((j >> 2) + 4 * g);
  const int tr_base = (8 * g + (j >> 2)) * 1024 + 256 * wave + ((j & 1) << 3);
  // B operands of key block kb (keys 16 kb .. 16 kb + 15): rows 8 g + (j >> 2)
  // (and + 4) of the stored half kb >> 1, keys 16 (kb & 1) + 4 (j & 3) .. + 3,
  // i.e. chunk 2 (kb & 1) + ((j & 3) >> 1) at position chunk ^ g.
  auto xfrag = [&](int tensor, int kb) {
    const int chunk = 2 * (kb & 1) + ((j & 3) >> 1);
    const int off = (2 * tensor + (kb >> 1)) * PT + (8 * g + (j >> 2)) * 64 +
                    ((chunk ^ g) << 4) + ((j & 1) << 3);
    return tr_frag_rows(ps + off, 256);
  };

  floatx4 acc[4][8];  // [key block][column block of this wave]
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int dl = 0; dl < 8; ++dl) acc[kb][dl] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One half-step: acc += (row tile of `tensor`)^T x (its stored partner),
  // Q with dS (tensor 0), dO with P (tensor 1).
  auto half_step = [&](int tensor) {
    mfma_phase_begin();
    int trb = tr_base;
    asm volatile("" : "+v"(trb));
    const char *rb = smem + tensor * STEP_BYTES;
    bf16x8 x[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) x[kb] = xfrag(1 - tensor, kb);
#pragma unroll
    for (int ps_ = 0; ps_ < 2; ++ps_) {
      bf16x8 tr[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) tr[c] = tr_frag(rb + trb + ((tr_sw ^ (2 * (4 * ps_ + c))) << 4));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[kb][4 * ps_ + c] = mfma16x16x32(tr[c], x[kb], acc[kb][4 * ps_ + c]);
    }
    mfma_phase_end();
  };
  // Each half-step's copy runs under the other half-step's math: the dO / P
  // copy of step s under the Q / dS half of step s, the Q / dS copy of step
  // s + 1 under the dO / P half of step s.  Per element the sums keep the
  // order dS Q (s), P dO (s), dS Q (s + 1), ...
  if (nsteps > 0) {
    stage(0, 0);
    stage(0, 1);
  }
  for (int s = 0; s < nsteps; ++s) {
    if (s == 0)
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kHalfCopies) : "memory");
    else
      wait_all_loads();
    __syncthreads();  // Q / dS of step s visible; the dO / P buffers are free
    if (s > 0) stage(s, 1);
    half_step(0);
    wait_all_loads();
    __syncthreads();  // dO / P of step s visible; the Q / dS buffers are free
    if (s + 1 < nsteps) stage(s + 1, 0);
    half_step(1);
  }

  // Partial [64 keys][512]: this wave's 128 columns of every key.
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float *out = part + it.part_off + (size_t)(16 * kb + j) * D + 128 * wave + 4 * g;
#pragma unroll
    for (int dl = 0; dl < 8; ++dl) {
      float4 w;
      w.x = acc[kb][dl][0];
      w.y = acc[kb][dl][1];
      w.z = acc[kb][dl][2];
      w.w = acc[kb][dl][3];
      *reinterpret_cast<float4 *>(out + 16 * dl) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. Fixed-order sum of the partials of every key tile -> dKV / dKV_comp.
// ---------------------------------------------------------------------------
// One launch, the raw key tiles' workgroups first; a workgroup takes one
// (key tile, chunk of the tile's [kv_bk][D] block).  Thread (g, c)
// sums the float4 column c of the tile's partial blocks i = g, g + G, g + 2 G,
// ... in increasing order (eight loads in flight), and the G group sums are
// added in group order.  The grouping is fixed, so the result is bitwise
// reproducible.  Raw tiles have a few blocks each (G = 1, 1024-element
// chunks); a compressed tile has tens to hundreds, streamed by G = 8 groups
// over 128-element chunks.
template <int G>
__device__ __forceinline__ void dkv_reduce_block(const Dims &d, const DevPlan &p,
                                                 const float *__restrict__ part, int dtype,
                                                 void *__restrict__ dkv, void *__restrict__ dkvc,
                                                 int comp, int blk, float4 (*red)[256 / G]) {
  constexpr int C = 256 / G, CHUNK = 4 * C;  // float4 columns per group, elements per workgroup
  const int nkt = d.nkv_raw + d.nkv_comp;
  const int ntl = comp ? d.nkv_comp : d.nkv_raw;  // tiles of this launch per batch row
  const int per_tile = d.kv_bk * d.D / CHUNK;
  const int tile = blk / per_tile, chunk = blk - tile * per_tile;
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

// Both kinds in one launch: blocks [0, raw_blk) reduce raw key tiles (G = 1),
// the rest compressed ones (G = 8).
__global__ void __launch_bounds__(256)
    hca_dkv_reduce_kernel(Dims d, DevPlan p, const float *__restrict__ part, int dtype,
                          void *__restrict__ dkv, void *__restrict__ dkvc, int raw_blk) {
  __shared__ float4 red[8][32];
  if ((int)blockIdx.x < raw_blk)
    dkv_reduce_block<1>(d, p, part, dtype, dkv, dkvc, 0, blockIdx.x,
                        reinterpret_cast<float4 (*)[256]>(&red[0][0]));
  else
    dkv_reduce_block<8>(d, p, part, dtype, dkv, dkvc, 1, blockIdx.x - raw_blk, red);
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
                       void *pds, void *stream) {
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
      const int grid = units < cus ? units : cus;
      if (d.pds_rows) {
        // Stored P / dS (written by launch_bwd_pds_bf16): the streaming dQ pass.
        if (!pds) return (int)hipErrorInvalidValue;
        constexpr int QW = HCA_DQS_NW;
        const int qu = d.B * d.nqt * (d.bq * d.H / (16 * QW));
        hipLaunchKernelGGL(hca_bwd_dqs512_kernel<QW>, dim3(qu), dim3(QW * 64), 0, s, d, p,
                           (const bf16raw *)kvt, (const bf16raw *)kvct, (const char *)pds,
                           (bf16raw *)dq);
        break;
      }
      if (d.cmask_ldw)
        go(hca_bwd_dq512_kernel<4, true>, 4, grid);
      else
        go(hca_bwd_dq512_kernel<4, false>, 4, grid);
      break;
    }
    case 128: go(hca_bwd_dq_kernel<128, 8, 1>, 8, d.B * d.nqt * (d.bq * d.H / 128)); break;
    case 64: go(hca_bwd_dq_kernel<64, 8, 1>, 8, d.B * d.nqt * (d.bq * d.H / 128)); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_bwd_pds_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kvt,
                        const void *kvct, const void *o, const float *lse, const void *dout,
                        float scale, float *delta, void *pds, void *stream) {
  if (d.D != 512 || !d.pds_rows || !pds) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  const float sl2 = scale * kLog2e;
  constexpr int PW = HCA_PDS_NW;
  const int pu = d.B * d.nqt * (d.bq * d.H / (16 * PW));
  auto gp = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(pu), dim3(PW * 64), 0, s, d, p, (const bf16raw *)q,
                       (const bf16raw *)kvt, (const bf16raw *)kvct, (const bf16raw *)o, lse,
                       (const bf16raw *)dout, sl2, scale, delta, (char *)pds);
  };
  if (d.cmask_ldw)
    gp(hca_bwd_pds512_kernel<PW, true>);
  else
    gp(hca_bwd_pds512_kernel<PW, false>);
  return (int)hipGetLastError();
}

int launch_bwd_dkv_bf16(const Dims &d, const DevPlan &p, const void *q, const void *kv,
                        const void *kvc, const float *lse, const float *delta,
                        const void *dout, float scale, const void *pds, float *part,
                        void *stream) {
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
      if (d.pds_rows) {
        // P and dS were stored by the dQ pass.
        if (!pds) return (int)hipErrorInvalidValue;
        if (d.kv_bk != 64) return (int)hipErrorInvalidValue;
        hipLaunchKernelGGL(hca_bwd_dkv512s_kernel, dim3(d.n_items), dim3(256), 0, s, d, p,
                           (const bf16raw *)q, (const bf16raw *)dout, (const char *)pds, part);
        break;
      }
      if (d.kv_bk != 128) return (int)hipErrorInvalidValue;
      // Every item (over all keys of its tile or over one half) in one launch.
      if (d.cmask_ldw)
        hipLaunchKernelGGL(hca_bwd_dkv512x8_kernel<true>, dim3(d.n_items), dim3(512), 0, s, d,
                           p, (const bf16raw *)q, (const bf16raw *)kv, (const bf16raw *)kvc, lse,
                           delta, (const bf16raw *)dout, sl2, scale, part);
      else
        hipLaunchKernelGGL(hca_bwd_dkv512x8_kernel<false>, dim3(d.n_items), dim3(512), 0, s, d,
                           p, (const bf16raw *)q, (const bf16raw *)kv, (const bf16raw *)kvc, lse,
                           delta, (const bf16raw *)dout, sl2, scale, part);
      break;
    case 128:
    case 64:
      // The kernel stages whole 64-row steps of a query tile and splits rows
      // by shifts.
      if ((d.bq * d.H) % 64 || (d.H & (d.H - 1)) || ((d.bq * d.H / 64) & (d.bq * d.H / 64 - 1)))
        return (int)hipErrorInvalidValue;
      if (d.D == 128) go(hca_bwd_dkv_kernel<128>);
      else go(hca_bwd_dkv_kernel<64>);
      break;
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
  if (raw_blk + comp_blk > 0)
    hipLaunchKernelGGL(hca_dkv_reduce_kernel, dim3(raw_blk + comp_blk), dim3(256), 0, s, d, p,
                       part, dtype, dkv, dkvc, raw_blk);
  return (int)hipGetLastError();
}

}  // namespace hca
