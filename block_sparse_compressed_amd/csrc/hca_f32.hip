// hca_f32.hip -- float32 HCA attention on gfx950 (vector ALU, one workgroup per row or key).
//
// The float32 path serves small problems that need float32 accuracy; every
// product and sum is float32.  A workgroup owns one query row (forward, dQ)
// or one key (dKV); its wavefronts share out the row's keys (or the key's
// rows) and the 64 lanes of each split the head dimension.  Each row walks
// exactly its visible intervals -- raw keys raw_lo..i and compressed entries
// comp_lo..comp_hi-1 from the host plan -- so nothing invisible is touched.
// Same mathematics as the bf16 path: one softmax over the union of the sliding
// window and the completed compressed entries ("Add HCA Static Compilation
// for Splash Attention [Deepseek v4]", Description), with the shared K = V
// tensor ("[DeepSeek-V4] Implement Compressed Attention Layers", review
// suggestions).
#include "hca_device.h"
#include "hca_internal.h"

namespace hca {

namespace {

// Sum over the 64 lanes, the result in every lane, without LDS round trips:
// DPP within each 16-lane row (swap neighbours, swap pairs, mirror the half
// row, mirror the row), then the gfx950 lane swaps across rows.  (A shuffle
// ladder goes through the LDS crossbar once per step; with two sums per
// visited key it was most of the float32 kernels' time.)
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_plus<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_plus<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_plus<0x141>(v);  // row_half_mirror
  v = dpp_plus<0x140>(v);  // row_mirror
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  u = __float_as_uint(v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

// Loads of this many visits (keys of a row, heads of a position) are issued
// together before any of them is used.
constexpr int kBatch = 4;

// Forward and dQ: one workgroup of kRowWaves wavefronts per query row; wave w
// takes every kRowWaves-th visible key (raw window first, then compressed
// entries), so the chains of dependent loads and wave-wide sums run side by
// side.  The waves' partial results are merged in a fixed order.
constexpr int kRowWaves = 4;

template <int NDU>
__global__ void __launch_bounds__(kRowWaves * 64)
    hca_fwd_f32_kernel(Dims d, DevPlan p, const float *__restrict__ q, const float *__restrict__ kv,
                       const float *__restrict__ kvc, float scale_log2, float *__restrict__ o,
                       float *__restrict__ lse) {
  __shared__ float red_acc[kRowWaves][NDU * 64];
  __shared__ float red_ml[kRowWaves][2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;  // whole workgroup: same row
  if (row >= (int64_t)d.B * d.H * d.S) return;
  const int D = NDU * 64;
  const int i = (int)(row % d.S);
  const int b = (int)(row / d.S / d.H);
  const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + i];
  float qv[NDU], acc[NDU];
#pragma unroll
  for (int u = 0; u < NDU; ++u) {
    qv[u] = q[row * D + lane + 64 * u];
    acc[u] = 0.f;
  }
  // Online softmax of this wave's keys (log2 units).
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const float (&kr)[NDU]) {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < NDU; ++u) s += qv[u] * kr[u];
    const float x = wave_sum(s) * scale_log2;
    const float mn = fmaxf(m, x);
    const float a = fast_exp2(m - mn), pr = fast_exp2(x - mn);
    l = l * a + pr;
#pragma unroll
    for (int u = 0; u < NDU; ++u) acc[u] = acc[u] * a + pr * kr[u];
    m = mn;
  };
  const int nraw = max(i + 1 - rw.x, 0);
  const int nkeys = nraw + max(rw.z - rw.y, 0);
  // The wave's keys in order, kBatch rows loaded at a time.
  for (int n0 = wave; n0 < nkeys; n0 += kBatch * kRowWaves) {
    float kr[kBatch][NDU];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int n = n0 + t * kRowWaves;
      if (n < nkeys) {
        const float *krow = n < nraw ? kv + ((size_t)b * d.S + rw.x + n) * D
                                     : kvc + ((size_t)b * d.Sc + rw.y + (n - nraw)) * D;
#pragma unroll
        for (int u = 0; u < NDU; ++u) kr[t][u] = krow[lane + 64 * u];
      }
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
      if (n0 + t * kRowWaves < nkeys) visit(kr[t]);
  }
  // Merge: M = max m_w, L = sum l_w 2^(m_w - M), acc = sum acc_w 2^(m_w - M).
#pragma unroll
  for (int u = 0; u < NDU; ++u) red_acc[wave][lane + 64 * u] = acc[u];
  if (lane == 0) {
    red_ml[wave][0] = m;
    red_ml[wave][1] = l;
  }
  __syncthreads();
  if (wave == 0) {
    float M = -INFINITY;
    for (int w = 0; w < kRowWaves; ++w) M = fmaxf(M, red_ml[w][0]);
    float L = 0.f, out[NDU];
#pragma unroll
    for (int u = 0; u < NDU; ++u) out[u] = 0.f;
    for (int w = 0; w < kRowWaves; ++w) {
      const float mw = red_ml[w][0];
      const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      L += red_ml[w][1] * f;
#pragma unroll
      for (int u = 0; u < NDU; ++u) out[u] += red_acc[w][lane + 64 * u] * f;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int u = 0; u < NDU; ++u) o[row * D + lane + 64 * u] = out[u] * inv;
    if (lane == 0) lse[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  }
}

template <int NDU>
__global__ void __launch_bounds__(kRowWaves * 64)
    hca_bwd_dq_f32_kernel(Dims d, DevPlan p, const float *__restrict__ q,
                          const float *__restrict__ kv, const float *__restrict__ kvc,
                          const float *__restrict__ o, const float *__restrict__ lse,
                          const float *__restrict__ dout, float scale_log2, float scale,
                          float *__restrict__ dq, float *__restrict__ delta) {
  __shared__ float red_acc[kRowWaves - 1][NDU * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;  // whole workgroup: same row
  if (row >= (int64_t)d.B * d.H * d.S) return;
  const int D = NDU * 64;
  const int i = (int)(row % d.S);
  const int b = (int)(row / d.S / d.H);
  const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + i];
  float qv[NDU], dv[NDU], acc[NDU], dl = 0.f;
#pragma unroll
  for (int u = 0; u < NDU; ++u) {
    qv[u] = q[row * D + lane + 64 * u];
    dv[u] = dout[row * D + lane + 64 * u];
    dl += dv[u] * o[row * D + lane + 64 * u];
    acc[u] = 0.f;
  }
  dl = wave_sum(dl);  // every wave computes delta; wave 0 stores it
  if (wave == 0 && lane == 0) delta[row] = dl;
  const float lse2 = lse[row] * kLog2e;
  auto visit = [&](const float (&kr)[NDU]) {
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int u = 0; u < NDU; ++u) {
      s += qv[u] * kr[u];
      t += dv[u] * kr[u];
    }
    s = wave_sum(s);
    t = wave_sum(t);
    const float pr = fast_exp2(s * scale_log2 - lse2);
    const float ds = pr * (t - dl) * scale;
#pragma unroll
    for (int u = 0; u < NDU; ++u) acc[u] += ds * kr[u];
  };
  const int nraw = max(i + 1 - rw.x, 0);
  const int nkeys = nraw + max(rw.z - rw.y, 0);
  // The wave's keys n = wave, wave + kRowWaves, ... in order, kBatch at a time:
  // their rows are loaded together, so one load latency covers the batch.
  for (int n0 = wave; n0 < nkeys; n0 += kBatch * kRowWaves) {
    float kr[kBatch][NDU];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int n = n0 + t * kRowWaves;
      if (n < nkeys) {
        const float *krow = n < nraw ? kv + ((size_t)b * d.S + rw.x + n) * D
                                     : kvc + ((size_t)b * d.Sc + rw.y + (n - nraw)) * D;
#pragma unroll
        for (int u = 0; u < NDU; ++u) kr[t][u] = krow[lane + 64 * u];
      }
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
      if (n0 + t * kRowWaves < nkeys) visit(kr[t]);
  }
  if (wave > 0) {
#pragma unroll
    for (int u = 0; u < NDU; ++u) red_acc[wave - 1][lane + 64 * u] = acc[u];
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 0; w < kRowWaves - 1; ++w)
#pragma unroll
      for (int u = 0; u < NDU; ++u) acc[u] += red_acc[w][lane + 64 * u];
#pragma unroll
    for (int u = 0; u < NDU; ++u) dq[row * D + lane + 64 * u] = acc[u];
  }
}

// dKV, sixteen lanes per visit: one workgroup of kGroupWaves wavefronts per
// key; each 16-lane row of a wavefront takes one (position, head) visit at a
// time, a lane holding D / 16 columns of the visit's q and dO rows (16-byte
// pieces c, c + 16, ... of the row, so a row's loads are whole and
// contiguous).  <q, k> and <dO, k> need only a 16-lane sum (four DPP steps,
// no lane swaps across rows), and dS q + P dO is added to the lane's own
// columns.  At the end the four rows of each wavefront are added with the
// lane swaps and the wavefronts' sums in a fixed order (wave 0, 1, ...), so the
// result is the same on every run.  A compressed entry is seen by every later
// position of its document; against one visit per wavefront (64 lanes over D,
// two full wave sums per visit) a wavefront works on four visits at once with
// a quarter of the cross-lane steps each.
constexpr int kGroupWaves = 8;

__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_plus<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_plus<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_plus<0x141>(v);  // row_half_mirror
  return dpp_plus<0x140>(v);  // row_mirror
}

__device__ __forceinline__ float rows4_sum(float v) {  // the 4 rows of a wave
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  u = __float_as_uint(v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int NDU>
__global__ void __launch_bounds__(kGroupWaves * 64)
    hca_bwd_dkv_f32_rows_kernel(Dims d, DevPlan p, const float *__restrict__ q,
                                const float *__restrict__ kv, const float *__restrict__ kvc,
                                const float *__restrict__ lse, const float *__restrict__ delta,
                                const float *__restrict__ dout, float scale_log2, float scale,
                                float *__restrict__ dkv, float *__restrict__ dkvc) {
  constexpr int D = NDU * 64, C4 = D / 4;     // 16-byte pieces per row
  constexpr int NG = kGroupWaves * 4;          // 16-lane rows per workgroup
  constexpr int VB = NDU <= 1 ? 8 : NDU <= 2 ? 4 : NDU <= 4 ? 2 : 1;  // visits per batch
  __shared__ float4 red[kGroupWaves][C4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, grp = wave * 4 + (lane >> 4);
  const int per_b = d.S + d.Sc;
  const int64_t kk = blockIdx.x;  // whole workgroup: same key
  if (kk >= (int64_t)d.B * per_b) return;
  const int b = (int)(kk / per_b), idx = (int)(kk % per_b);
  const bool comp = idx >= d.S;
  const int k = comp ? idx - d.S : idx;
  const float4 *krow = reinterpret_cast<const float4 *>(
      comp ? kvc + ((size_t)b * d.Sc + k) * D : kv + ((size_t)b * d.S + k) * D);
  float4 kr[NDU], acc[NDU];
#pragma unroll
  for (int m = 0; m < NDU; ++m) {
    kr[m] = krow[c + 16 * m];
    acc[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Positions that can see key k (each then checked against its own interval).
  int i0, i1;
  if (comp) {
    i0 = (k + 1) * d.r - 1;
    i1 = d.S - 1;
  } else {
    i0 = k;
    i1 = d.W > 0 ? min(d.S - 1, k + d.W - 1) : k - 1;
  }
  const int nvis = i1 >= i0 ? (i1 - i0 + 1) * d.H : 0;
  // Row group g takes visits g, g + NG, g + 2 NG, ... (position-major), VB at
  // a time with their loads issued together.
  for (int v0 = grp; v0 < nvis; v0 += VB * NG) {
    float4 qv[VB][NDU], dv[VB][NDU];
    float ls[VB], dt[VB];
    bool on[VB];
#pragma unroll
    for (int t = 0; t < VB; ++t) {
      const int v = v0 + t * NG;
      on[t] = v < nvis;
      const int vc = on[t] ? v : grp;  // (an in-range visit; its result is dropped)
      const int i = i0 + vc / d.H, h = vc % d.H;
      const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + i];
      on[t] = on[t] && (comp ? (rw.y <= k && k < rw.z) : (rw.x <= k));
      const size_t row = ((size_t)b * d.H + h) * d.S + i;
      const float4 *qr = reinterpret_cast<const float4 *>(q + row * D);
      const float4 *dr = reinterpret_cast<const float4 *>(dout + row * D);
#pragma unroll
      for (int m = 0; m < NDU; ++m) {
        qv[t][m] = qr[c + 16 * m];
        dv[t][m] = dr[c + 16 * m];
      }
      ls[t] = lse[row];
      dt[t] = delta[row];
    }
#pragma unroll
    for (int t = 0; t < VB; ++t) {
      float sv = 0.f, tv = 0.f;
#pragma unroll
      for (int m = 0; m < NDU; ++m) {
        sv += qv[t][m].x * kr[m].x + qv[t][m].y * kr[m].y + qv[t][m].z * kr[m].z +
              qv[t][m].w * kr[m].w;
        tv += dv[t][m].x * kr[m].x + dv[t][m].y * kr[m].y + dv[t][m].z * kr[m].z +
              dv[t][m].w * kr[m].w;
      }
      sv = row16_sum(sv);
      tv = row16_sum(tv);
      const float pr = on[t] ? fast_exp2(sv * scale_log2 - ls[t] * kLog2e) : 0.f;
      const float ds = pr * (tv - dt[t]) * scale;
#pragma unroll
      for (int m = 0; m < NDU; ++m) {
        acc[m].x += ds * qv[t][m].x + pr * dv[t][m].x;
        acc[m].y += ds * qv[t][m].y + pr * dv[t][m].y;
        acc[m].z += ds * qv[t][m].z + pr * dv[t][m].z;
        acc[m].w += ds * qv[t][m].w + pr * dv[t][m].w;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NDU; ++m) {
    acc[m].x = rows4_sum(acc[m].x);
    acc[m].y = rows4_sum(acc[m].y);
    acc[m].z = rows4_sum(acc[m].z);
    acc[m].w = rows4_sum(acc[m].w);
    if (lane < 16) red[wave][c + 16 * m] = acc[m];
  }
  __syncthreads();
  if (tid < C4) {
    float4 t = red[0][tid];
    for (int w = 1; w < kGroupWaves; ++w) {
      const float4 x = red[w][tid];
      t.x += x.x;
      t.y += x.y;
      t.z += x.z;
      t.w += x.w;
    }
    float4 *out = reinterpret_cast<float4 *>(comp ? dkvc + ((size_t)b * d.Sc + k) * D
                                                  : dkv + ((size_t)b * d.S + k) * D);
    out[tid] = t;
  }
}

#define HCA_F32_SWITCH(D, CALL) \
  switch ((D) / 64) {           \
    case 1: CALL(1); break;     \
    case 2: CALL(2); break;     \
    case 3: CALL(3); break;     \
    case 4: CALL(4); break;     \
    case 5: CALL(5); break;     \
    case 6: CALL(6); break;     \
    case 7: CALL(7); break;     \
    case 8: CALL(8); break;     \
    default: return (int)hipErrorInvalidValue; \
  }

int launch_fwd_f32(const Dims &d, const DevPlan &p, const float *q, const float *kv,
                   const float *kvc, float scale, float *o, float *lse, void *stream) {
  const int64_t rows = (int64_t)d.B * d.H * d.S;
  const dim3 grid((unsigned)rows);
  hipStream_t s = (hipStream_t)stream;
  const float sl2 = scale * kLog2e;
#define CALL(N)                                                                              \
  hipLaunchKernelGGL(hca_fwd_f32_kernel<N>, grid, dim3(kRowWaves * 64), 0, s, d, p, q, kv, kvc, \
                     sl2, o, lse)
  HCA_F32_SWITCH(d.D, CALL)
#undef CALL
  return (int)hipGetLastError();
}

int launch_bwd_f32(const Dims &d, const DevPlan &p, const float *q, const float *kv,
                   const float *kvc, const float *o, const float *lse, const float *dout,
                   float scale, float *dq, float *dkv, float *dkvc, float *delta, void *stream) {
  const int64_t rows = (int64_t)d.B * d.H * d.S;
  const int64_t keys = (int64_t)d.B * (d.S + d.Sc);
  hipStream_t s = (hipStream_t)stream;
  const float sl2 = scale * kLog2e;
#define CALL(N)                                                                              \
  hipLaunchKernelGGL(hca_bwd_dq_f32_kernel<N>, dim3((unsigned)rows), dim3(kRowWaves * 64), 0, \
                     s, d, p, q, kv, kvc, o, lse, dout, sl2, scale, dq, delta)
  HCA_F32_SWITCH(d.D, CALL)
#undef CALL
  int err = (int)hipGetLastError();
  if (err) return err;
#define CALL(N)                                                                          \
  hipLaunchKernelGGL(hca_bwd_dkv_f32_rows_kernel<N>, dim3((unsigned)keys),               \
                     dim3(kGroupWaves * 64), 0, s, d, p, q, kv, kvc, lse, delta, dout, sl2, \
                     scale, dkv, dkvc)
  HCA_F32_SWITCH(d.D, CALL)
#undef CALL
  return (int)hipGetLastError();
}

}  // namespace hca
