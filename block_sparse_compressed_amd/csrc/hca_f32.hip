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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace

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
  auto visit = [&](const float *krow) {
    float kr[NDU], s = 0.f;
#pragma unroll
    for (int u = 0; u < NDU; ++u) {
      kr[u] = krow[lane + 64 * u];
      s += qv[u] * kr[u];
    }
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
  for (int n = wave; n < nkeys; n += kRowWaves)
    visit(n < nraw ? kv + ((size_t)b * d.S + rw.x + n) * D
                   : kvc + ((size_t)b * d.Sc + rw.y + (n - nraw)) * D);
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
  auto visit = [&](const float *krow) {
    float kr[NDU], s = 0.f, t = 0.f;
#pragma unroll
    for (int u = 0; u < NDU; ++u) {
      kr[u] = krow[lane + 64 * u];
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
  for (int n = wave; n < nkeys; n += kRowWaves)
    visit(n < nraw ? kv + ((size_t)b * d.S + rw.x + n) * D
                   : kvc + ((size_t)b * d.Sc + rw.y + (n - nraw)) * D);
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
  for (int i = i0 + wave; i <= i1; i += kDkvWaves) {
    const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + i];
    const bool vis = comp ? (rw.y <= k && k < rw.z) : (rw.x <= k);
    if (!vis) continue;
    for (int h = 0; h < d.H; ++h) {
      const size_t row = ((size_t)b * d.H + h) * d.S + i;
      float qv[NDU], dv[NDU], s = 0.f, t = 0.f;
#pragma unroll
      for (int u = 0; u < NDU; ++u) {
        qv[u] = q[row * D + lane + 64 * u];
        dv[u] = dout[row * D + lane + 64 * u];
        s += qv[u] * kr[u];
        t += dv[u] * kr[u];
      }
      s = wave_sum(s);
      t = wave_sum(t);
      const float pr = fast_exp2(s * scale_log2 - lse[row] * kLog2e);
      const float ds = pr * (t - delta[row]) * scale;
#pragma unroll
      for (int u = 0; u < NDU; ++u) acc[u] += ds * qv[u] + pr * dv[u];
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
