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

// dKV: one workgroup of kDkvWaves wavefronts per key.  A compressed entry is
// seen by every later position of its document, so a single wavefront walking
// its rows one by one (each a chain of loads and wave-wide sums) took most of
// the backward; the waves take interleaved positions and their partial sums are
// added in a fixed order (wave 0, then 1, 2, ...), so the result is the same on
// every run.
constexpr int kDkvWaves = 16;

template <int NDU>
__global__ void __launch_bounds__(kDkvWaves * 64)
    hca_bwd_dkv_f32_kernel(Dims d, DevPlan p, const float *__restrict__ q,
                           const float *__restrict__ kv, const float *__restrict__ kvc,
                           const float *__restrict__ lse, const float *__restrict__ delta,
                           const float *__restrict__ dout, float scale_log2, float scale,
                           float *__restrict__ dkv, float *__restrict__ dkvc) {
  __shared__ float red[kDkvWaves - 1][NDU * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per_b = d.S + d.Sc;
  const int64_t kk = blockIdx.x;  // whole workgroup: same key
  if (kk >= (int64_t)d.B * per_b) return;
  const int D = NDU * 64;
  const int b = (int)(kk / per_b), idx = (int)(kk % per_b);
  const bool comp = idx >= d.S;
  const int k = comp ? idx - d.S : idx;
  const float *krow = comp ? kvc + ((size_t)b * d.Sc + k) * D : kv + ((size_t)b * d.S + k) * D;
  float kr[NDU], acc[NDU];
#pragma unroll
  for (int u = 0; u < NDU; ++u) {
    kr[u] = krow[lane + 64 * u];
    acc[u] = 0.f;
  }
  // Positions that can see key k: raw k .. k+W-1, compressed (k+1) r - 1 .. S-1;
  // each is then checked against its own visible interval.
  int i0, i1;
  if (comp) {
    i0 = (k + 1) * d.r - 1;
    i1 = d.S - 1;
  } else {
    i0 = k;
    i1 = d.W > 0 ? min(d.S - 1, k + d.W - 1) : k - 1;
  }
  // The wave's (position, head) visits in order -- positions i0 + wave,
  // i0 + wave + kDkvWaves, ..., all heads of each -- VB at a time: the rows'
  // visible intervals, Q and dO rows, LSE and delta of a batch are loaded
  // together, so one load latency covers the batch (fewer for wide heads: a
  // 16-wave workgroup has 128 registers per lane).  A position that does not
  // see key k adds nothing.
  constexpr int VB = NDU <= 1 ? 8 : NDU <= 2 ? 4 : NDU <= 4 ? 2 : 1;
  const int npos = i1 >= i0 + wave ? (i1 - i0 - wave) / kDkvWaves + 1 : 0;
  const int nvis = npos * d.H;
  for (int v0 = 0; v0 < nvis; v0 += VB) {
    float qv[VB][NDU], dv[VB][NDU], ls[VB], dt[VB];
    bool on[VB];
#pragma unroll
    for (int t = 0; t < VB; ++t) {
      const int v = v0 + t;
      on[t] = false;
      if (v < nvis) {
        const int i = i0 + wave + (v / d.H) * kDkvWaves, h = v % d.H;
        const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + i];
        on[t] = comp ? (rw.y <= k && k < rw.z) : (rw.x <= k);
        const size_t row = ((size_t)b * d.H + h) * d.S + i;
#pragma unroll
        for (int u = 0; u < NDU; ++u) {
          qv[t][u] = q[row * D + lane + 64 * u];
          dv[t][u] = dout[row * D + lane + 64 * u];
        }
        ls[t] = lse[row];
        dt[t] = delta[row];
      }
    }
#pragma unroll
    for (int t = 0; t < VB; ++t) {
      if (!on[t]) continue;
      float s = 0.f, tt = 0.f;
#pragma unroll
      for (int u = 0; u < NDU; ++u) {
        s += qv[t][u] * kr[u];
        tt += dv[t][u] * kr[u];
      }
      s = wave_sum(s);
      tt = wave_sum(tt);
      const float pr = fast_exp2(s * scale_log2 - ls[t] * kLog2e);
      const float ds = pr * (tt - dt[t]) * scale;
#pragma unroll
      for (int u = 0; u < NDU; ++u) acc[u] += ds * qv[t][u] + pr * dv[t][u];
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int u = 0; u < NDU; ++u) red[wave - 1][lane + 64 * u] = acc[u];
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 0; w < kDkvWaves - 1; ++w)
#pragma unroll
      for (int u = 0; u < NDU; ++u) acc[u] += red[w][lane + 64 * u];
    float *out = comp ? dkvc + ((size_t)b * d.Sc + k) * D : dkv + ((size_t)b * d.S + k) * D;
#pragma unroll
    for (int u = 0; u < NDU; ++u) out[lane + 64 * u] = acc[u];
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
#define CALL(N)                                                                                \
  hipLaunchKernelGGL(hca_bwd_dkv_f32_kernel<N>, dim3((unsigned)keys), dim3(kDkvWaves * 64), 0, \
                     s, d, p, q, kv, kvc, lse, delta, dout, sl2, scale, dkv, dkvc)
  HCA_F32_SWITCH(d.D, CALL)
#undef CALL
  return (int)hipGetLastError();
}

}  // namespace hca
