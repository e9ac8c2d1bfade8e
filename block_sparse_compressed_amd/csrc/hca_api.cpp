// hca_api.cpp -- C ABI entry points: argument validation (before any HIP call),
// plan upload, and the kernel sequences of the forward and backward passes.
// Validation guards follow the pages' practice of refusing unsupported
// configurations explicitly rather than computing something else ("Add HCA
// Static Compilation for Splash Attention [Deepseek v4]", Description:
// explicit errors for modes the compressed path does not support).
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hca_internal.h"

namespace hca {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

Dims make_dims(const hca_plan *plan) {
  const hca_plan_info &in = plan->info;
  Dims d{};
  // B x kv_heads MQA problems of H / kv_heads heads each (see hca_block_mask_build_gqa)
  d.B = plan->rows_b; d.S = in.S; d.H = in.H / in.kv_heads; d.D = in.D; d.r = in.r;
  d.W = in.W; d.Sc = in.S_c;
  d.bq = in.bq; d.bk_raw = in.bk_raw; d.bk_comp = in.bk_comp;
  d.nqt = in.nqt; d.nkt_raw = in.nkt_raw; d.nkt_comp = in.nkt_comp;
  d.S_pad = in.nkt_raw * in.bk_raw;
  d.Sc_pad = in.nkt_comp * in.bk_comp;
  d.n_items = (int32_t)plan->kvorder.size();  // launch slots (items + padding)
  d.kv_bk = plan->kv_bk;
  d.nkv_raw = plan->nkv_raw;
  d.nkv_comp = plan->nkv_comp;
  d.cmask_ldw = plan->cmask_ldw;
  d.pds_rows = plan->pds_rows;
  d.f32_split = plan->f32_split;
  return d;
}

DevPlan make_devplan(const hca_plan *plan) {
  const uint8_t *base = static_cast<const uint8_t *>(plan->dev);
  const DevLayout &L = plan->lay;
  DevPlan p{};
  p.rows = reinterpret_cast<const int32_t *>(base + L.rows);
  p.qptr = reinterpret_cast<const int32_t *>(base + L.qptr);
  p.qent = reinterpret_cast<const uint32_t *>(base + L.qent);
  p.qorder = reinterpret_cast<const int32_t *>(base + L.qorder);
  p.kvitem = reinterpret_cast<const KvItem *>(base + L.kvitem);
  p.kvorder = reinterpret_cast<const int32_t *>(base + L.kvorder);
  p.kvent = reinterpret_cast<const uint32_t *>(base + L.kvent);
  p.kvtile = reinterpret_cast<const int32_t *>(base + L.kvtile);
  p.cmask = plan->cmask_ldw ? reinterpret_cast<const uint32_t *>(base + L.cmask) : nullptr;
  p.kvpe = plan->pds_rows ? reinterpret_cast<const int32_t *>(base + L.kvpe) : nullptr;
  return p;
}

hca_status fail(hca_status s, const std::string &msg) {
  set_error(msg);
  return s;
}

hca_status hip_fail(const char *what, int err) {
  return fail(HCA_ERR_HIP, std::string(what) + ": " + hipGetErrorString((hipError_t)err));
}

// Checks shared by the forward and backward entry points.
hca_status check_common(const char *fn, const hca_plan *plan, float scale, void *ws,
                        uint64_t ws_bytes, uint64_t ws_needed) {
  if (!plan) return fail(HCA_ERR_INVALID_ARG, std::string(fn) + ": plan is NULL");
  if (!plan->info.kernel_ok)
    return fail(HCA_ERR_UNSUPPORTED, std::string(fn) + ": " + plan->unsupported);
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(HCA_ERR_INVALID_ARG, std::string(fn) + ": scale must be finite and > 0");
  if (ws_bytes < ws_needed)
    return fail(HCA_ERR_WORKSPACE, std::string(fn) + ": workspace needs " +
                                       std::to_string(ws_needed) + " bytes, got " +
                                       std::to_string(ws_bytes));
  if (ws_needed && (!ws || !aligned16(ws)))
    return fail(HCA_ERR_INVALID_ARG, std::string(fn) + ": workspace is NULL or misaligned");
  return HCA_OK;
}

// ---- kernel timing instrumentation ----------------------------------------
enum KernelId { K_TRANSPOSE, K_FWD, K_BWD_DQ, K_BWD_DKV, K_DKV_REDUCE, K_FWD_F32, K_BWD_F32,
                K_BWD_PDS, K_COUNT };
const char *const kKernelNames[K_COUNT] = {"transpose", "fwd",     "bwd_dq",  "bwd_dkv",
                                           "dkv_reduce", "fwd_f32", "bwd_f32", "bwd_pds"};
struct TimingRec {
  int kid, dev;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_recs;
// Events read back and ready for reuse, per device (an event is recorded only
// on streams of the device it was created on).
std::vector<std::vector<hipEvent_t>> g_free_events;

// An event for a timed region on device `dev`: a reused one when
// available (creating events costs host time inside the region being
// measured), else a new one.
hipEvent_t take_event(int dev) {
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    if ((size_t)dev < g_free_events.size() && !g_free_events[dev].empty()) {
      hipEvent_t e = g_free_events[dev].back();
      g_free_events[dev].pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

void give_event(int dev, hipEvent_t e) {  // caller holds g_tmu
  if (g_free_events.size() <= (size_t)dev) g_free_events.resize(dev + 1);
  g_free_events[dev].push_back(e);
}

// Runs `launch` (which enqueues one library kernel on `stream`), bracketed by
// events when timing is enabled and `allowed` (the allocation-free entry
// point never creates events).
template <class F>
int timed(int kid, void *stream, F launch, bool allowed = true) {
  int dev = 0;
  if (!g_timing || !allowed || hipGetDevice(&dev) != hipSuccess || dev < 0) return launch();
  hipEvent_t a = take_event(dev), b = take_event(dev);
  if (!a || !b) {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (a) give_event(dev, a);
    if (b) give_event(dev, b);
    return launch();
  }
  hipEventRecord(a, (hipStream_t)stream);
  int err = launch();
  hipEventRecord(b, (hipStream_t)stream);
  std::lock_guard<std::mutex> lk(g_tmu);
  g_recs.push_back({kid, dev, a, b});
  return err;
}

// The library's second stream on the current device: default priority,
// non-blocking (ordered against the caller's stream by events only), created
// on first use and kept until the process ends; nullptr if it cannot be made.
hipStream_t side_stream() {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!streams[dev] && hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking) != hipSuccess)
    streams[dev] = nullptr;
  return streams[dev];
}

// Fork of the second stream from a caller's stream and its join back: work
// enqueued on `stream` after fork() starts after what the caller's stream
// held at the fork, and the caller's stream waits, from join() on, for all of
// it.  The destructor joins a fork left open by an early return.
struct SideStream {
  hipStream_t stream = nullptr;
  hipStream_t caller = nullptr;
  // Without a second stream (it could not be created) the work stays on the
  // caller's stream: `stream` remains nullptr and the call runs serially.
  int fork(void *caller_stream) {
    hipStream_t s = side_stream();
    if (!s) return 0;
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev, (hipStream_t)caller_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, ev, 0);
    if (ev) (void)hipEventDestroy(ev);  // released once the recorded work completes
    if (e != hipSuccess) return (int)e;
    stream = s;
    caller = (hipStream_t)caller_stream;
    return 0;
  }
  int join() {
    if (!stream) return 0;
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(caller, ev, 0);
    if (ev) (void)hipEventDestroy(ev);
    if (e != hipSuccess) {
      // The caller's stream cannot be ordered after the second stream's work:
      // wait for that work on the host instead.
      (void)hipStreamSynchronize(stream);
    }
    stream = nullptr;
    return (int)e;
  }
  ~SideStream() { join(); }
};

hca_status check_ptr(const char *fn, const char *name, const void *p) {
  if (!p) return fail(HCA_ERR_INVALID_ARG, std::string(fn) + ": " + name + " is NULL");
  if (!aligned16(p))
    return fail(HCA_ERR_INVALID_ARG, std::string(fn) + ": " + name + " is not 16-byte aligned");
  return HCA_OK;
}

}  // namespace

void set_error(const std::string &msg) { g_last_error = msg; }

}  // namespace hca

using namespace hca;

extern "C" const char *hca_status_string(hca_status s) {
  switch (s) {
    case HCA_OK: return "HCA_OK";
    case HCA_ERR_INVALID_ARG: return "HCA_ERR_INVALID_ARG";
    case HCA_ERR_UNSUPPORTED: return "HCA_ERR_UNSUPPORTED";
    case HCA_ERR_WORKSPACE: return "HCA_ERR_WORKSPACE";
    case HCA_ERR_HIP: return "HCA_ERR_HIP";
    case HCA_ERR_NOMEM: return "HCA_ERR_NOMEM";
    case HCA_ERR_STATE: return "HCA_ERR_STATE";
  }
  return "HCA_ERR_UNKNOWN";
}

extern "C" const char *hca_last_error(void) { return g_last_error.c_str(); }

extern "C" hca_status hca_plan_upload(hca_plan *plan, void *dev_buf, uint64_t bytes,
                                      void *hip_stream) {
  if (!plan) return fail(HCA_ERR_INVALID_ARG, "hca_plan_upload: plan is NULL");
  if (hca_status s = check_ptr("hca_plan_upload", "dev_buf", dev_buf)) return s;
  if (bytes < plan->info.device_bytes)
    return fail(HCA_ERR_WORKSPACE, "hca_plan_upload: buffer needs " +
                                       std::to_string(plan->info.device_bytes) + " bytes, got " +
                                       std::to_string(bytes));
  hipError_t e = hipMemcpyAsync(dev_buf, plan->image.data(), plan->image.size(),
                                hipMemcpyHostToDevice, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail("hca_plan_upload", e);
  plan->dev = dev_buf;
  return HCA_OK;
}

namespace {

// Checks of the forward's pointer arguments (after check_common).
hca_status check_fwd_ptrs(const char *fn, const hca_plan *plan, const void *q, const void *kv,
                          const void *kv_comp, const void *o, const float *lse) {
  if (hca_status s = check_ptr(fn, "q", q)) return s;
  if (hca_status s = check_ptr(fn, "kv", kv)) return s;
  if (plan->info.S_c > 0)
    if (hca_status s = check_ptr(fn, "kv_comp", kv_comp)) return s;
  if (hca_status s = check_ptr(fn, "o", o)) return s;
  if (hca_status s = check_ptr(fn, "lse", lse)) return s;
  return HCA_OK;
}

// The forward's kernel sequence on a checked plan and workspace.
hca_status run_fwd(const char *fn, const hca_plan *plan, const void *q, const void *kv,
                   const void *kv_comp, float scale, void *o, float *lse, void *ws,
                   void *hip_stream, bool timing = true) {
  const Dims d = make_dims(plan);
  const DevPlan p = make_devplan(plan);
  int err;
  if (plan->info.dtype == HCA_F32) {
    err = timed(K_FWD_F32, hip_stream, [&] {
      return launch_fwd_f32(d, p, (const float *)q, (const float *)kv, (const float *)kv_comp,
                            scale, (float *)o, lse, hip_stream);
    }, timing);
    if (err) return hip_fail((std::string(fn) + " (float32 kernel)").c_str(), err);
    return HCA_OK;
  }
  uint8_t *w = static_cast<uint8_t *>(ws);
  void *kvt = w + plan->ws.kvt, *kvct = w + plan->ws.kvct;
  // The D = 512 kernels stage K tiles from tile images made here; the D = 64
  // / 128 kernels stage the row-major tensor itself.
  if (d.D == 512) {
    err = timed(K_TRANSPOSE, hip_stream, [&] {
      return launch_transpose_kv(kv, kvt, d.S, d.S_pad, d.Sc > 0 ? kv_comp : nullptr, kvct, d.Sc,
                                 d.Sc_pad, d.B, d.D, hip_stream);
    }, timing);
    if (err) return hip_fail((std::string(fn) + " (transpose)").c_str(), err);
  }
  err = timed(K_FWD, hip_stream, [&] {
    return launch_fwd_bf16(d, p, q, kv, kv_comp ? kv_comp : kv, kvt, kvct, scale, o, lse,
                           hip_stream);
  }, timing);
  if (err) return hip_fail((std::string(fn) + " (forward kernel)").c_str(), err);
  return HCA_OK;
}

}  // namespace

extern "C" hca_status hca_attn_fwd(const hca_plan *plan, const void *q, const void *kv,
                                   const void *kv_comp, float scale, void *o, float *lse,
                                   void *ws, uint64_t ws_bytes, void *hip_stream) {
  const char *fn = "hca_attn_fwd";
  if (hca_status s = check_common(fn, plan, scale, ws, ws_bytes, plan ? plan->ws.fwd_total : 0))
    return s;
  if (hca_status s = check_fwd_ptrs(fn, plan, q, kv, kv_comp, o, lse)) return s;
  if (!plan->dev) return fail(HCA_ERR_STATE, std::string(fn) + ": plan was not uploaded");
  return run_fwd(fn, plan, q, kv, kv_comp, scale, o, lse, ws, hip_stream);
}

extern "C" hca_status hca_attn_fwd_noalloc(const hca_plan *plan, const void *q, const void *kv,
                                           const void *kv_comp, float scale, void *o,
                                           float *lse, void *hip_stream) {
  const char *fn = "hca_attn_fwd_noalloc";
  if (!plan) return fail(HCA_ERR_INVALID_ARG, std::string(fn) + ": plan is NULL");
  if (!plan->info.kernel_ok)
    return fail(HCA_ERR_UNSUPPORTED, std::string(fn) + ": " + plan->unsupported);
  if (plan->ws.fwd_total > kNoAllocScratchBytes)
    return fail(HCA_ERR_WORKSPACE,
                std::string(fn) + ": the forward needs " + std::to_string(plan->ws.fwd_total) +
                    " bytes of workspace; the library's scratch holds " +
                    std::to_string(kNoAllocScratchBytes) + " (use hca_attn_fwd)");
  // The scratch stands in for the workspace: its size is the limit checked
  // above, its address is known only after the checks that precede any HIP call.
  static char placeholder alignas(16);
  if (hca_status s = check_common(fn, plan, scale, &placeholder, kNoAllocScratchBytes,
                                  plan->ws.fwd_total))
    return s;
  if (hca_status s = check_fwd_ptrs(fn, plan, q, kv, kv_comp, o, lse)) return s;
  if (!plan->dev) return fail(HCA_ERR_STATE, std::string(fn) + ": plan was not uploaded");
  void *ws = nullptr;
  if (plan->ws.fwd_total > 0) {
    int err = 0;
    ws = noalloc_scratch(&err);
    if (!ws) return hip_fail("hca_attn_fwd_noalloc (scratch address)", err);
  }
  return run_fwd(fn, plan, q, kv, kv_comp, scale, o, lse, ws, hip_stream, false);
}

extern "C" hca_status hca_attn_bwd(const hca_plan *plan, const void *q, const void *kv,
                                   const void *kv_comp, const void *o, const float *lse,
                                   const void *dout, float scale, void *dq, void *dkv,
                                   void *dkv_comp, void *ws, uint64_t ws_bytes,
                                   void *hip_stream) {
  const char *fn = "hca_attn_bwd";
  if (hca_status s = check_common(fn, plan, scale, ws, ws_bytes, plan ? plan->ws.bwd_total : 0))
    return s;
  if (hca_status s = check_ptr(fn, "q", q)) return s;
  if (hca_status s = check_ptr(fn, "kv", kv)) return s;
  if (hca_status s = check_ptr(fn, "o", o)) return s;
  if (hca_status s = check_ptr(fn, "lse", lse)) return s;
  if (hca_status s = check_ptr(fn, "dout", dout)) return s;
  if (hca_status s = check_ptr(fn, "dq", dq)) return s;
  if (hca_status s = check_ptr(fn, "dkv", dkv)) return s;
  if (plan->info.S_c > 0) {
    if (hca_status s = check_ptr(fn, "kv_comp", kv_comp)) return s;
    if (hca_status s = check_ptr(fn, "dkv_comp", dkv_comp)) return s;
  }
  if (!plan->dev) return fail(HCA_ERR_STATE, std::string(fn) + ": plan was not uploaded");

  const Dims d = make_dims(plan);
  const DevPlan p = make_devplan(plan);
  uint8_t *w = static_cast<uint8_t *>(ws);
  float *delta = reinterpret_cast<float *>(w + plan->ws.delta);
  int err;
  if (plan->info.dtype == HCA_F32) {
    err = timed(K_BWD_F32, hip_stream, [&] {
      return launch_bwd_f32(d, p, (const float *)q, (const float *)kv, (const float *)kv_comp,
                            (const float *)o, lse, (const float *)dout, scale, (float *)dq,
                            (float *)dkv, (float *)dkv_comp, delta,
                            reinterpret_cast<float *>(w + plan->ws.f32_part), hip_stream);
    });
    if (err) return hip_fail("hca_attn_bwd (float32 kernels)", err);
    return HCA_OK;
  }
  void *kvt = w + plan->ws.kvt, *kvct = w + plan->ws.kvct;
  float *part = reinterpret_cast<float *>(w + plan->ws.part);
  void *pds = plan->pds_rows ? w + plan->ws.pds : nullptr;
  const void *kvc = kv_comp ? kv_comp : kv;
  if (d.D == 512) {  // tile images (see the forward)
    err = timed(K_TRANSPOSE, hip_stream, [&] {
      return launch_transpose_kv(kv, kvt, d.S, d.S_pad, d.Sc > 0 ? kv_comp : nullptr, kvct, d.Sc,
                                 d.Sc_pad, d.B, d.D, hip_stream);
    });
    if (err) return hip_fail("hca_attn_bwd (transpose)", err);
  }
  if (pds) {
    err = timed(K_BWD_PDS, hip_stream, [&] {
      return launch_bwd_pds_bf16(d, p, q, kvt, kvct, o, lse, dout, scale, delta, pds,
                                 hip_stream);
    });
    if (err) return hip_fail("hca_attn_bwd (P / dS kernel)", err);
  }
  // With stored P / dS the dQ pass only reads the stored tiles and K^T, and
  // writes dQ alone, so it runs on the library's second stream of the device,
  // concurrently with the key-stationary pass, and fills the tail of that
  // launch.  The second stream forks from the caller's stream after the P / dS
  // pass and joins it again before the call returns (also on error paths).
  SideStream side;
  if (pds && (err = side.fork(hip_stream)) != 0) return hip_fail("hca_attn_bwd (second stream)", err);
  void *dq_stream = side.stream ? (void *)side.stream : hip_stream;
  err = timed(K_BWD_DQ, dq_stream, [&] {
    return launch_bwd_dq_bf16(d, p, q, kv, kvc, kvt, kvct, o, lse, dout, scale, dq, delta, pds,
                              dq_stream);
  });
  if (err) return hip_fail("hca_attn_bwd (dQ kernel)", err);
  err = timed(K_BWD_DKV, hip_stream, [&] {
    return launch_bwd_dkv_bf16(d, p, q, kv, kvc, lse, delta, dout, scale, pds, part,
                               hip_stream);
  });
  if (err) return hip_fail("hca_attn_bwd (dKV kernel)", err);
  err = timed(K_DKV_REDUCE, hip_stream, [&] {
    return launch_dkv_reduce(d, p, part, HCA_BF16, dkv, dkv_comp, hip_stream);
  });
  if (err) return hip_fail("hca_attn_bwd (dKV reduction)", err);
  if ((err = side.join()) != 0) return hip_fail("hca_attn_bwd (second stream)", err);
  return HCA_OK;
}

extern "C" hca_status hca_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  return HCA_OK;
}

extern "C" hca_status hca_timing_read(hca_kernel_time *out, int32_t capacity, int32_t *count) {
  if (!count || (capacity > 0 && !out))
    return fail(HCA_ERR_INVALID_ARG, "hca_timing_read: NULL output");
  std::vector<TimingRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs.swap(g_recs);
  }
  double ms[K_COUNT] = {0};
  int64_t n[K_COUNT] = {0};
  hca_status st = HCA_OK;
  std::vector<bool> ok(recs.size(), true);
  for (size_t i = 0; i < recs.size(); ++i) {
    const TimingRec &r = recs[i];
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      st = fail(HCA_ERR_HIP, "hca_timing_read: event query failed");
      ok[i] = false;
    }
    ms[r.kid] += t;
    n[r.kid] += 1;
  }
  {
    // Completed pairs go back to the pool; a pair whose query failed is
    // destroyed instead of being reused.
    std::lock_guard<std::mutex> lk(g_tmu);
    for (size_t i = 0; i < recs.size(); ++i) {
      if (ok[i]) {
        give_event(recs[i].dev, recs[i].a);
        give_event(recs[i].dev, recs[i].b);
      } else {
        (void)hipEventDestroy(recs[i].a);
        (void)hipEventDestroy(recs[i].b);
      }
    }
  }
  int32_t c = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (!n[k]) continue;
    if (c < capacity) {
      std::memset(out[c].name, 0, sizeof out[c].name);
      std::strncpy(out[c].name, kKernelNames[k], sizeof out[c].name - 1);
      out[c].launches = n[k];
      out[c].total_ms = ms[k];
    }
    ++c;
  }
  *count = c;
  return st;
}
