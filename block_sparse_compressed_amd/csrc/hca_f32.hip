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

// Cross-lane sums without LDS round trips.  Within each 16-lane row: DPP
// steps (swap neighbours, swap pairs, mirror the half row, mirror the row),
// the row's sum in each of its lanes.  (A shuffle ladder goes through the LDS
// crossbar once per step; with two sums per visited key it had been most of
// the float32 kernels' time.)
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, true));
}

__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_plus<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_plus<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_plus<0x141>(v);  // row_half_mirror
  return dpp_plus<0x140>(v);  // row_mirror
}

// Sum / max over the four 16-lane rows of a wavefront (lanes l, l ^ 16,
// l ^ 32, l ^ 48) with the gfx950 lane swaps, the result in every lane.
__device__ __forceinline__ float rows4_sum(float v) {
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  u = __float_as_uint(v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float rows4_max(float v) {
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  u = __float_as_uint(v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace

// Forward and dQ: one workgroup of kRowWaves wavefronts per query row, and
// sixteen lanes per visited key: each 16-lane row of a wavefront (group g =
// 4 wave + lane / 16) takes keys g, g + 16, g + 32, ... of the row (raw window
// first, then compressed entries), a lane holding D / 16 columns of the q, dO
// and key rows as whole 16-byte pieces (c, c + 16, ... for lane c of the row),
// so a key's dot products need only a 16-lane sum.  kBatch keys' rows are
// loaded together.  The 16 groups' partial results are merged at the end in a
// fixed order (the four rows of a wavefront with the lane swaps, then the
// wavefronts), so every run gives the same result.
constexpr int kRowWaves = 4;
constexpr int kBatch = 4;

template <int NDU>
__global__ void __launch_bounds__(kRowWaves * 64)
    hca_fwd_f32_kernel(Dims d, DevPlan p, const float *__restrict__ q, const float *__restrict__ kv,
                       const float *__restrict__ kvc, float scale_log2, float *__restrict__ o,
                       float *__restrict__ lse) {
  constexpr int D = NDU * 64, C4 = D / 4, NG = kRowWaves * 4;
  __shared__ float4 red_acc[kRowWaves][C4];
  __shared__ float red_ml[kRowWaves][2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, grp = wave * 4 + (lane >> 4);
  const int64_t row = blockIdx.x;  // whole workgroup: same row
  if (row >= (int64_t)d.B * d.H * d.S) return;
  const int i = (int)(row % d.S);
  const int b = (int)(row / d.S / d.H);
  const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + i];
  const float4 *qr = reinterpret_cast<const float4 *>(q + row * D);
  float4 qv[NDU], acc[NDU];
#pragma unroll
  for (int m = 0; m < NDU; ++m) {
    qv[m] = qr[c + 16 * m];
    acc[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Online softmax of this group's keys (log2 units).
  float mx = -INFINITY, l = 0.f;
  const int nraw = max(i + 1 - rw.x, 0);
  const int nkeys = nraw + max(rw.z - rw.y, 0);
  for (int n0 = grp; n0 < nkeys; n0 += kBatch * NG) {
    float4 kr[kBatch][NDU];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int n = min(n0 + t * NG, nkeys - 1);  // (past the end: a key that is dropped)
      const float4 *krow = reinterpret_cast<const float4 *>(
          n < nraw ? kv + ((size_t)b * d.S + rw.x + n) * D
                   : kvc + ((size_t)b * d.Sc + rw.y + (n - nraw)) * D);
#pragma unroll
      for (int m = 0; m < NDU; ++m) kr[t][m] = krow[c + 16 * m];
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      if (n0 + t * NG >= nkeys) break;  // uniform within the group
      float sv = 0.f;
#pragma unroll
      for (int m = 0; m < NDU; ++m)
        sv += qv[m].x * kr[t][m].x + qv[m].y * kr[t][m].y + qv[m].z * kr[t][m].z +
              qv[m].w * kr[t][m].w;
      const float x = row16_sum(sv) * scale_log2;
      const float mn = fmaxf(mx, x);
      const float a = fast_exp2(mx - mn), pr = fast_exp2(x - mn);
      l = l * a + pr;
#pragma unroll
      for (int m = 0; m < NDU; ++m) {
        acc[m].x = acc[m].x * a + pr * kr[t][m].x;
        acc[m].y = acc[m].y * a + pr * kr[t][m].y;
        acc[m].z = acc[m].z * a + pr * kr[t][m].z;
        acc[m].w = acc[m].w * a + pr * kr[t][m].w;
      }
      mx = mn;
    }
  }
  // Merge the wavefront's four groups: M = max m_g, L = sum l_g 2^(m_g - M),
  // acc = sum acc_g 2^(m_g - M); then the wavefronts the same way.
  const float mw = rows4_max(mx);
  const float f = mx == -INFINITY ? 0.f : fast_exp2(mx - mw);
  const float lw = rows4_sum(l * f);
#pragma unroll
  for (int m = 0; m < NDU; ++m) {
    acc[m].x = rows4_sum(acc[m].x * f);
    acc[m].y = rows4_sum(acc[m].y * f);
    acc[m].z = rows4_sum(acc[m].z * f);
    acc[m].w = rows4_sum(acc[m].w * f);
    if (lane < 16) red_acc[wave][c + 16 * m] = acc[m];
  }
  if (lane == 0) {
    red_ml[wave][0] = mw;
    red_ml[wave][1] = lw;
  }
  __syncthreads();
  if (threadIdx.x < C4) {
    const int e = threadIdx.x;
    float M = -INFINITY;
    for (int w = 0; w < kRowWaves; ++w) M = fmaxf(M, red_ml[w][0]);
    float L = 0.f;
    float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int w = 0; w < kRowWaves; ++w) {
      const float m_w = red_ml[w][0];
      const float fw = m_w == -INFINITY ? 0.f : fast_exp2(m_w - M);
      L += red_ml[w][1] * fw;
      const float4 x = red_acc[w][e];
      out.x += x.x * fw;
      out.y += x.y * fw;
      out.z += x.z * fw;
      out.w += x.w * fw;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    reinterpret_cast<float4 *>(o + row * D)[e] =
        make_float4(out.x * inv, out.y * inv, out.z * inv, out.w * inv);
    if (e == 0) lse[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  }
}

template <int NDU>
__global__ void __launch_bounds__(kRowWaves * 64)
    hca_bwd_dq_f32_kernel(Dims d, DevPlan p, const float *__restrict__ q,
                          const float *__restrict__ kv, const float *__restrict__ kvc,
                          const float *__restrict__ o, const float *__restrict__ lse,
                          const float *__restrict__ dout, float scale_log2, float scale,
                          float *__restrict__ dq, float *__restrict__ delta) {
  constexpr int D = NDU * 64, C4 = D / 4, NG = kRowWaves * 4;
  __shared__ float4 red_acc[kRowWaves][C4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, grp = wave * 4 + (lane >> 4);
  const int64_t row = blockIdx.x;  // whole workgroup: same row
  if (row >= (int64_t)d.B * d.H * d.S) return;
  const int i = (int)(row % d.S);
  const int b = (int)(row / d.S / d.H);
  const int4 rw = reinterpret_cast<const int4 *>(p.rows)[(size_t)b * d.S + i];
  const float4 *qr = reinterpret_cast<const float4 *>(q + row * D);
  const float4 *dr = reinterpret_cast<const float4 *>(dout + row * D);
  const float4 *orow = reinterpret_cast<const float4 *>(o + row * D);
  float4 qv[NDU], dv[NDU], acc[NDU];
  float dl = 0.f;
#pragma unroll
  for (int m = 0; m < NDU; ++m) {
    qv[m] = qr[c + 16 * m];
    dv[m] = dr[c + 16 * m];
    const float4 ov = orow[c + 16 * m];
    dl += dv[m].x * ov.x + dv[m].y * ov.y + dv[m].z * ov.z + dv[m].w * ov.w;
    acc[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  dl = row16_sum(dl);  // every group holds the whole row: delta in every lane
  if (threadIdx.x == 0) delta[row] = dl;
  const float lse2 = lse[row] * kLog2e;
  const int nraw = max(i + 1 - rw.x, 0);
  const int nkeys = nraw + max(rw.z - rw.y, 0);
  for (int n0 = grp; n0 < nkeys; n0 += kBatch * NG) {
    float4 kr[kBatch][NDU];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int n = min(n0 + t * NG, nkeys - 1);  // (past the end: a key that is dropped)
      const float4 *krow = reinterpret_cast<const float4 *>(
          n < nraw ? kv + ((size_t)b * d.S + rw.x + n) * D
                   : kvc + ((size_t)b * d.Sc + rw.y + (n - nraw)) * D);
#pragma unroll
      for (int m = 0; m < NDU; ++m) kr[t][m] = krow[c + 16 * m];
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      if (n0 + t * NG >= nkeys) break;  // uniform within the group
      float sv = 0.f, tv = 0.f;
#pragma unroll
      for (int m = 0; m < NDU; ++m) {
        sv += qv[m].x * kr[t][m].x + qv[m].y * kr[t][m].y + qv[m].z * kr[t][m].z +
              qv[m].w * kr[t][m].w;
        tv += dv[m].x * kr[t][m].x + dv[m].y * kr[t][m].y + dv[m].z * kr[t][m].z +
              dv[m].w * kr[t][m].w;
      }
      sv = row16_sum(sv);
      tv = row16_sum(tv);
      const float pr = fast_exp2(sv * scale_log2 - lse2);
      const float ds = pr * (tv - dl) * scale;
#pragma unroll
      for (int m = 0; m < NDU; ++m) {
        acc[m].x += ds * kr[t][m].x;
        acc[m].y += ds * kr[t][m].y;
        acc[m].z += ds * kr[t][m].z;
        acc[m].w += ds * kr[t][m].w;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NDU; ++m) {
    acc[m].x = rows4_sum(acc[m].x);
    acc[m].y = rows4_sum(acc[m].y);
    acc[m].z = rows4_sum(acc[m].z);
    acc[m].w = rows4_sum(acc[m].w);
    if (lane < 16) red_acc[wave][c + 16 * m] = acc[m];
  }
  __syncthreads();
  if (threadIdx.x < C4) {
    const int e = threadIdx.x;
    float4 t = red_acc[0][e];
    for (int w = 1; w < kRowWaves; ++w) {
      const float4 x = red_acc[w][e];
      t.x += x.x;
      t.y += x.y;
      t.z += x.z;
      t.w += x.w;
    }
    reinterpret_cast<float4 *>(dq + row * D)[e] = t;
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

template <int NDU>
__global__ void __launch_bounds__(kGroupWaves * 64)
    hca_bwd_dkv_f32_rows_kernel(Dims d, DevPlan p, const float *__restrict__ q,
                                const float *__restrict__ kv, const float *__restrict__ kvc,
                                const float *__restrict__ lse, const float *__restrict__ delta,
                                const float *__restrict__ dout, float scale_log2, float scale,
                                float *__restrict__ dkv, float *__restrict__ dkvc,
                                float *__restrict__ part) {
  constexpr int D = NDU * 64, C4 = D / 4;     // 16-byte pieces per row
  constexpr int NG = kGroupWaves * 4;          // 16-lane rows per workgroup
  constexpr int VB = NDU <= 1 ? 8 : NDU <= 2 ? 4 : NDU <= 4 ? 2 : 1;  // visits per batch
  __shared__ float4 red[kGroupWaves][C4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, grp = wave * 4 + (lane >> 4);
  // Whole workgroup: one key, or one of the f32_split parts of a compressed
  // entry's visits.  The compressed entries (each seen by every later
  // position of its document: the longest walks) take the first workgroup
  // ids, so they start first and the raw keys fill in beside them.
  const int nsplit = d.f32_split;
  const int64_t x = blockIdx.x, ncomp = (int64_t)d.B * d.Sc * nsplit;
  if (x >= ncomp + (int64_t)d.B * d.S) return;
  const bool comp = x < ncomp;
  const int64_t centry = comp ? x / nsplit : 0;  // b * Sc + k
  const int split = comp ? (int)(x % nsplit) : 0;
  const int b = comp ? (int)(centry / d.Sc) : (int)((x - ncomp) / d.S);
  const int k = comp ? (int)(centry % d.Sc) : (int)((x - ncomp) % d.S);
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
  const int nvis_all = i1 >= i0 ? (i1 - i0 + 1) * d.H : 0;
  // This workgroup's visits [vlo, nvis): all of them, or split `split` of
  // nsplit equal ranges.
  const int per = (nvis_all + nsplit - 1) / nsplit;
  const int vlo = comp ? min(nvis_all, split * per) : 0;
  const int nvis = comp ? min(nvis_all, vlo + per) : nvis_all;
  // Row group g takes visits vlo + g, vlo + g + NG, ... (position-major), VB
  // at a time with their loads issued together.
  for (int v0 = vlo + grp; v0 < nvis; v0 += VB * NG) {
    float4 qv[VB][NDU], dv[VB][NDU];
    float ls[VB], dt[VB];
    bool on[VB];
#pragma unroll
    for (int t = 0; t < VB; ++t) {
      const int v = v0 + t * NG;
      on[t] = v < nvis;
      const int vc = on[t] ? v : vlo + grp;  // (an in-range visit; its result is dropped)
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
    // A split's sum goes to the partial area; hca_dkv_f32_split_sum_kernel
    // adds the splits of each entry in split order.
    float4 *out = reinterpret_cast<float4 *>(
        comp ? (nsplit > 1 ? part + ((size_t)centry * nsplit + split) * D
                           : dkvc + ((size_t)b * d.Sc + k) * D)
             : dkv + ((size_t)b * d.S + k) * D);
    out[tid] = t;
  }
}

// Compressed entries' dKV from their split partial sums: one workgroup per
// entry, thread e adds 16-byte piece e of the f32_split partials in split
// order.
__global__ void __launch_bounds__(128)
    hca_dkv_f32_split_sum_kernel(Dims d, const float *__restrict__ part, float *__restrict__ dkvc) {
  const int C4 = d.D / 4, e = threadIdx.x;
  if (e >= C4) return;
  const size_t entry = blockIdx.x;  // b * Sc + k
  const float4 *pe = reinterpret_cast<const float4 *>(part + entry * d.f32_split * d.D);
  float4 t = pe[e];
  for (int s = 1; s < d.f32_split; ++s) {
    const float4 x = pe[s * C4 + e];
    t.x += x.x;
    t.y += x.y;
    t.z += x.z;
    t.w += x.w;
  }
  reinterpret_cast<float4 *>(dkvc + entry * d.D)[e] = t;
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
                   float scale, float *dq, float *dkv, float *dkvc, float *delta,
                   float *f32_part, void *stream) {
  const int64_t rows = (int64_t)d.B * d.H * d.S;
  const int64_t keys = (int64_t)d.B * (d.S + (int64_t)d.Sc * d.f32_split);
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
                     scale, dkv, dkvc, f32_part)
  HCA_F32_SWITCH(d.D, CALL)
#undef CALL
  err = (int)hipGetLastError();
  if (err || d.f32_split <= 1 || d.Sc == 0) return err;
  hipLaunchKernelGGL(hca_dkv_f32_split_sum_kernel, dim3((unsigned)(d.B * d.Sc)),
                     dim3(d.D / 4 < 64 ? 64 : d.D / 4), 0, s, d, (const float *)f32_part, dkvc);
  return (int)hipGetLastError();
}

}  // namespace hca
