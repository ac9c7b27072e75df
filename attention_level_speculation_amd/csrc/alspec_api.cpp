// C ABI of the speculative flash-decode step: argument validation, the split
// plan, and the order of kernels and events on the caller's streams.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "alspec.h"
#include "alspec_kernels.h"
#include "alspec_plan.h"
#include "alspec_scratch.h"

static_assert(ALSPEC_NOALLOC_SCRATCH_BYTES == alspec::kScratchBytes,
              "the header states the static scratch's size");

// Fused calls remember, per workspace, the event that follows the last
// verify reading it, so that a later call on that workspace in another
// stream waits for it.
constexpr int kWsTable = 16;

struct WsEntry {
  const void *ws;
  hipEvent_t ev;
  hipStream_t stream;  // stream `ev` was recorded on
  uint64_t tick;
  bool used;
};

// Whether `s` is capturing into a graph.
static bool capturing(hipStream_t s) {
  hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &status) == hipSuccess &&
         status == hipStreamCaptureStatusActive;
}

// Id of the capture `s` belongs to (0: not capturing).
static unsigned long long capture_id(hipStream_t s) {
  hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
  unsigned long long id = 0;
  if (hipStreamGetCaptureInfo(s, &status, &id) != hipSuccess ||
      status != hipStreamCaptureStatusActive)
    return 0;
  return id;
}

struct alspec_handle {
  int device;
  hipStream_t sv;        // verify stream of pipelined calls
  hipEvent_t ev_join;    // exact stream -> approximation stream
  hipEvent_t ev_approx;  // approximation done
  hipEvent_t ev_mid;     // middle splits done (pipelined calls)
  hipEvent_t ev_verify;  // verify stream tail (alspec_order_after_verify)
  WsEntry ws_table[kWsTable];
  uint64_t tick;
  void *scratch;  // this device's static scratch (allocation-free call)
};

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Description of the last HIP failure on this thread (alspec_last_error).
thread_local char g_last_error[200];

// True when e is an error; the failing call is then noted for
// alspec_last_error.
bool failed(hipError_t e, const char *what) {
  if (e == hipSuccess) return false;
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what,
           hipGetErrorName(e), (int)e);
  return true;
}

alspec_status hip_status(hipError_t e, const char *what) {
  return failed(e, what) ? ALSPEC_ERR_HIP : ALSPEC_OK;
}

// Common checks of the q/k/v pointers and the workspace.
alspec_status check_inputs(const float *q, const void *k, const void *v) {
  if (!q || !k || !v) return ALSPEC_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return ALSPEC_ERR_INVALID_ARG;
  return ALSPEC_OK;
}

// Output arrays are written with 16-byte vector stores.
alspec_status check_outputs(const float *a, const float *b, const float *c) {
  if ((a && !aligned(a, 16)) || (b && !aligned(b, 16)) ||
      (c && !aligned(c, 16)))
    return ALSPEC_ERR_INVALID_ARG;
  return ALSPEC_OK;
}

alspec_status check_ws(const void *ws, size_t ws_bytes,
                       const alspec::Workspace &wl) {
  if (!ws) return ALSPEC_ERR_WORKSPACE;
  if (!aligned(ws, alspec::kWsAlign)) return ALSPEC_ERR_WORKSPACE;
  if (ws_bytes < wl.total) return ALSPEC_ERR_WORKSPACE;
  return ALSPEC_OK;
}

// Entry of the workspace table for `ws`: its own entry if the table has
// one, else (*fresh = true) a free entry or the least recently used one,
// whose old event the caller still has to honour.
WsEntry *ws_entry(alspec_handle *h, const void *ws, bool *fresh) {
  *fresh = false;
  for (int i = 0; i < kWsTable; ++i)
    if (h->ws_table[i].used && h->ws_table[i].ws == ws) return &h->ws_table[i];
  *fresh = true;
  for (int i = 0; i < kWsTable; ++i)
    if (!h->ws_table[i].used) return &h->ws_table[i];
  WsEntry *e = &h->ws_table[0];
  for (int i = 1; i < kWsTable; ++i)
    if (h->ws_table[i].tick < e->tick) e = &h->ws_table[i];
  return e;
}

// Caller's timing events; inside a stream capture they become event nodes
// that take their timestamps when the graph runs.
alspec_status record(void *ev, hipStream_t s) {
  if (!ev) return ALSPEC_OK;
  if (capturing(s))
    return hip_status(
        hipEventRecordWithFlags((hipEvent_t)ev, s, hipEventRecordExternal),
        "hipEventRecordWithFlags");
  return hip_status(hipEventRecord((hipEvent_t)ev, s), "hipEventRecord");
}

}  // namespace

extern "C" {

const char *alspec_status_string(alspec_status s) {
  switch (s) {
    case ALSPEC_OK: return "ALSPEC_OK";
    case ALSPEC_ERR_INVALID_ARG: return "ALSPEC_ERR_INVALID_ARG";
    case ALSPEC_ERR_UNSUPPORTED: return "ALSPEC_ERR_UNSUPPORTED";
    case ALSPEC_ERR_WORKSPACE: return "ALSPEC_ERR_WORKSPACE";
    case ALSPEC_ERR_HIP: return "ALSPEC_ERR_HIP";
  }
  return "ALSPEC_UNKNOWN_STATUS";
}

int32_t alspec_version(void) { return 100; }

const char *alspec_last_error(void) { return g_last_error; }

alspec_status alspec_workspace_size(const alspec_params *p, size_t *bytes) {
  if (!p || !bytes) return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  *bytes = wl.total;
  return ALSPEC_OK;
}

alspec_status alspec_plan_splits(const alspec_params *p, int32_t b,
                                 int32_t *kind, int32_t *begin, int32_t *end,
                                 int32_t cap, int32_t *count,
                                 int32_t *split_tokens,
                                 int32_t *window_split_tokens) {
  if (!p || !count || cap < 0 || (cap > 0 && (!kind || !begin || !end)))
    return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  if (b < 0 || b >= pa.B) return ALSPEC_ERR_INVALID_ARG;
  int n = 0;
  auto put = [&](int kd, int t0, int t1) {
    if (n < cap) {
      kind[n] = kd;
      begin[n] = t0;
      end[n] = t1;
    }
    ++n;
  };
  if (pa.nsink[b]) put(0, 0, pa.s_end[b]);
  for (int w = 0; w < pa.nwin[b]; ++w) {
    const int t0 = pa.w_begin[b] + w * pa.Tw;
    put(1, t0, t0 + pa.Tw < pa.L[b] ? t0 + pa.Tw : pa.L[b]);
  }
  for (int m = 0; m < pa.nmid[b]; ++m) {
    const int t0 = pa.s_end[b] + m * pa.T;
    put(2, t0, t0 + pa.T < pa.w_begin[b] ? t0 + pa.T : pa.w_begin[b]);
  }
  *count = n;
  if (split_tokens) *split_tokens = pa.T;
  if (window_split_tokens) *window_split_tokens = pa.Tw;
  return ALSPEC_OK;
}

alspec_status alspec_create(int device, alspec_handle **out) {
  if (!out) return ALSPEC_ERR_INVALID_ARG;
  *out = nullptr;
  int n = 0;
  if (failed(hipGetDeviceCount(&n), "hipGetDeviceCount"))
    return ALSPEC_ERR_HIP;
  if (device < 0 || device >= n) return ALSPEC_ERR_INVALID_ARG;
  int prev = 0;
  if (failed(hipGetDevice(&prev), "hipGetDevice")) return ALSPEC_ERR_HIP;
  if (failed(hipSetDevice(device), "hipSetDevice")) return ALSPEC_ERR_HIP;
  alspec_handle *h = (alspec_handle *)calloc(1, sizeof(alspec_handle));
  alspec_status st = ALSPEC_OK;
  if (!h) {
    st = ALSPEC_ERR_INVALID_ARG;
  } else {
    h->device = device;
    // The handle's events only order work between streams of this device,
    // so they skip the system-scope cache writeback and invalidation a
    // default event performs when it completes (which stalls, and slows,
    // the streaming kernels around it).
    auto event = [](hipEvent_t *e) {
      return !failed(hipEventCreateWithFlags(
                         e, hipEventDisableTiming | hipEventDisableSystemFence),
                     "hipEventCreateWithFlags");
    };
    bool ok = event(&h->ev_join) && event(&h->ev_approx) &&
              event(&h->ev_mid) && event(&h->ev_verify) &&
              !failed(hipStreamCreateWithFlags(&h->sv, hipStreamNonBlocking),
                      "hipStreamCreateWithFlags");
    for (int i = 0; ok && i < kWsTable; ++i) ok = event(&h->ws_table[i].ev);
    // the allocation-free call's scratch on this device (set up once per
    // device and process, with the device current)
    ok = ok && !failed(alspec::scratch_setup(device, h->sv, &h->scratch),
                       "scratch_setup");
    if (!ok) {
      alspec_destroy(h);
      h = nullptr;
      st = ALSPEC_ERR_HIP;
    }
  }
  (void)hipSetDevice(prev);
  *out = h;
  return st;
}

alspec_status alspec_destroy(alspec_handle *h) {
  if (!h) return ALSPEC_ERR_INVALID_ARG;
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->ev_approx) (void)hipEventDestroy(h->ev_approx);
  if (h->ev_mid) (void)hipEventDestroy(h->ev_mid);
  if (h->ev_verify) (void)hipEventDestroy(h->ev_verify);
  if (h->sv) (void)hipStreamDestroy(h->sv);
  for (int i = 0; i < kWsTable; ++i)
    if (h->ws_table[i].ev) (void)hipEventDestroy(h->ws_table[i].ev);
  free(h);
  return ALSPEC_OK;
}

alspec_status alspec_sink_approx(alspec_handle *h, const alspec_params *p,
                                 const float *q, const void *k, const void *v,
                                 float *o_approx, float *lse_approx, void *ws,
                                 size_t ws_bytes, void *stream) {
  if (!h || !p || !o_approx) return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  if ((st = check_inputs(q, k, v)) != ALSPEC_OK) return st;
  if ((st = check_ws(ws, ws_bytes, wl)) != ALSPEC_OK) return st;
  const alspec::WsPtrs w = alspec::ws_ptrs(ws, wl);
  alspec::Outs o{};
  o.o_approx = o_approx;
  o.lse_approx = lse_approx;
  return hip_status(
      alspec::launch_approx_fused(pa, p->kv_dtype, q, k, v,
                                  p->sm_scale * kLog2e, w, o,
                                  (hipStream_t)stream),
      "launch_approx_fused");
}

alspec_status alspec_flash_decode_exact(alspec_handle *h,
                                        const alspec_params *p,
                                        const float *q, const void *k,
                                        const void *v,
                                        int32_t include_sink_window, void *ws,
                                        size_t ws_bytes, void *stream) {
  if (!h || !p) return ALSPEC_ERR_INVALID_ARG;
  if (include_sink_window != 0 && include_sink_window != 1)
    return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  if ((st = check_inputs(q, k, v)) != ALSPEC_OK) return st;
  if ((st = check_ws(ws, ws_bytes, wl)) != ALSPEC_OK) return st;
  const alspec::WsPtrs w = alspec::ws_ptrs(ws, wl);
  const float sm_log2 = p->sm_scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  return hip_status(
      alspec::launch_partials(pa, p->kv_dtype,
                              include_sink_window ? alspec::kPartialsAll
                                                  : alspec::kPartialsMiddle,
                              q, k, v, sm_log2, w, s),
      "launch_partials");
}

alspec_status alspec_lse_combine(alspec_handle *h, const alspec_params *p,
                                 void *ws, size_t ws_bytes, float *o_exact,
                                 float *lse_exact, void *stream) {
  if (!h || !p || !o_exact) return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  if ((st = check_ws(ws, ws_bytes, wl)) != ALSPEC_OK) return st;
  const alspec::WsPtrs w = alspec::ws_ptrs(ws, wl);
  return hip_status(alspec::launch_lse_combine(pa, w, o_exact, lse_exact,
                                               (hipStream_t)stream),
                    "launch_lse_combine");
}

alspec_status alspec_verify(alspec_handle *h, const alspec_params *p,
                            const float *o_approx, const float *o_exact,
                            float *ratio, uint8_t *commit, float *o_committed,
                            void *stream) {
  if (!h || !p || !o_approx || !o_exact || !ratio || !commit)
    return ALSPEC_ERR_INVALID_ARG;
  alspec_status st = check_outputs(o_approx, o_exact, o_committed);
  if (st != ALSPEC_OK) return st;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  return hip_status(alspec::launch_verify(pa, o_approx, o_exact, ratio, commit,
                                          o_committed, p->lambda,
                                          (hipStream_t)stream),
                    "launch_verify");
}

alspec_status alspec_spec_decode(alspec_handle *h, const alspec_params *p,
                                 const float *q, const void *k, const void *v,
                                 float *o_approx, float *lse_approx,
                                 float *o_exact, float *lse_exact,
                                 float *ratio, uint8_t *commit,
                                 float *o_committed, void *ws,
                                 size_t ws_bytes, void *stream_approx,
                                 void *stream_exact, const alspec_events *ev) {
  if (!h || !p || !o_approx || !o_exact || !ratio || !commit)
    return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  if ((st = check_inputs(q, k, v)) != ALSPEC_OK) return st;
  if ((st = check_outputs(o_approx, o_exact, o_committed)) != ALSPEC_OK)
    return st;
  if ((st = check_ws(ws, ws_bytes, wl)) != ALSPEC_OK) return st;
  const alspec::WsPtrs w = alspec::ws_ptrs(ws, wl);
  const float sm_log2 = p->sm_scale * kLog2e;
  hipStream_t sa = (hipStream_t)stream_approx;
  hipStream_t se = (hipStream_t)stream_exact;
  const bool two = sa != se;
  alspec_events none;
  memset(&none, 0, sizeof none);
  const alspec_events &E = ev ? *ev : none;
  alspec::Outs o{o_approx, lse_approx, o_exact, lse_exact, ratio,
                 commit,   o_committed, p->lambda};
  // The sequential schedule runs the approximation in one launch; where it
  // runs beside the streaming middle pass it takes two fence-free launches.
  auto approx = [&](hipStream_t s) -> alspec_status {
    alspec_status r = record(E.approx_begin, s);
    if (r != ALSPEC_OK) return r;
    if (p->overlap == 0) {
      if (failed(alspec::launch_approx_fused(pa, p->kv_dtype, q, k, v,
                                             sm_log2, w, o, s),
                 "launch_approx_fused"))
        return ALSPEC_ERR_HIP;
    } else if (failed(alspec::launch_partials(pa, p->kv_dtype,
                                              alspec::kPartialsApprox, q, k,
                                              v, sm_log2, w, s),
                      "launch_partials") ||
               failed(alspec::launch_approx_combine(pa, w, o, s),
                      "launch_approx_combine")) {
      return ALSPEC_ERR_HIP;
    }
    return record(E.approx_end, s);
  };
  auto middle = [&](hipStream_t s) -> alspec_status {
    alspec_status r = record(E.exact_begin, s);
    if (r != ALSPEC_OK) return r;
    if (failed(alspec::launch_partials(pa, p->kv_dtype,
                                       alspec::kPartialsMiddle, q, k, v,
                                       sm_log2, w, s),
               "launch_partials"))
      return ALSPEC_ERR_HIP;
    return record(E.exact_end, s);
  };
  auto verify = [&](hipStream_t s) -> alspec_status {
    if (failed(alspec::launch_merge_verify(pa, w, o, s),
               "launch_merge_verify"))
      return ALSPEC_ERR_HIP;
    return record(E.verify_end, s);
  };

  // Ordering after the last uncaptured fused call that used this
  // workspace: its entry's event follows that call's verify, the last of
  // its kernels to read the workspace.  Under stream capture the library
  // adds no such ordering (the caller orders captured calls that share a
  // workspace): there such a wait could make a stream wait on a branch of
  // the capture that was forked from that same stream.
  const unsigned long long cap_e = capture_id(se);
  if (two && capture_id(sa) != cap_e)
    return ALSPEC_ERR_INVALID_ARG;  // half of the call would be captured
  const bool cap = cap_e != 0;
  bool fresh = false;
  WsEntry *ent = cap ? nullptr : ws_entry(h, ws, &fresh);
  auto wait_ws = [&](hipStream_t s) -> alspec_status {
    if (!ent || !ent->used || ent->stream == s) return ALSPEC_OK;
    return hip_status(hipStreamWaitEvent(s, ent->ev, 0), "hipStreamWaitEvent");
  };
  auto done_ws = [&](hipStream_t s) -> alspec_status {
    if (!ent) return ALSPEC_OK;
    if (failed(hipEventRecord(ent->ev, s), "hipEventRecord"))
      return ALSPEC_ERR_HIP;
    ent->ws = ws;
    ent->stream = s;
    ent->used = true;
    ent->tick = ++h->tick;
    return ALSPEC_OK;
  };
  // An evicted entry's workspace stays safe: the streams of this call are
  // ordered after its last verify before the entry is reused.
  if (fresh && (st = wait_ws(sa)) != ALSPEC_OK) return st;
  if (fresh && two && (st = wait_ws(se)) != ALSPEC_OK) return st;
  if (fresh) ent->used = false;

  if (p->overlap == 0) {
    // Approximation first, then the exact pass, in one stream: no
    // cross-stream wait between the kernels.  The approximation stream is
    // handed o_approx through an event, so work queued there after this
    // call runs while the exact pass does.
    if ((st = wait_ws(se)) != ALSPEC_OK) return st;
    if ((st = approx(se)) != ALSPEC_OK) return st;
    if (two) {
      if (failed(hipEventRecord(h->ev_approx, se), "hipEventRecord"))
        return ALSPEC_ERR_HIP;
      if (failed(hipStreamWaitEvent(sa, h->ev_approx, 0),
                 "hipStreamWaitEvent"))
        return ALSPEC_ERR_HIP;
    }
    if ((st = middle(se)) != ALSPEC_OK) return st;
    if ((st = verify(se)) != ALSPEC_OK) return st;
    return done_ws(se);
  }

  if (p->overlap == 2) {
    // Pipelined: stream_exact carries only middle splits, so successive
    // calls' exact passes run back to back; the approximation goes on
    // stream_approx, and the merge, verify and commit on the handle's own
    // verify stream once both are done.
    if ((st = wait_ws(sa)) != ALSPEC_OK) return st;
    if (two && (st = wait_ws(se)) != ALSPEC_OK) return st;
    if ((st = approx(sa)) != ALSPEC_OK) return st;
    if (failed(hipEventRecord(h->ev_approx, sa), "hipEventRecord"))
      return ALSPEC_ERR_HIP;
    if ((st = middle(se)) != ALSPEC_OK) return st;
    if (failed(hipEventRecord(h->ev_mid, se), "hipEventRecord"))
      return ALSPEC_ERR_HIP;
    if (failed(hipStreamWaitEvent(h->sv, h->ev_approx, 0),
               "hipStreamWaitEvent") ||
        failed(hipStreamWaitEvent(h->sv, h->ev_mid, 0), "hipStreamWaitEvent"))
      return ALSPEC_ERR_HIP;
    if ((st = verify(h->sv)) != ALSPEC_OK) return st;
    return done_ws(h->sv);
  }

  // Overlap: the approximation (on stream_approx) and the middle splits (on
  // stream_exact) start together; the exact merge and verify follow on
  // stream_exact once both are done.  Outside a capture the approximation,
  // which rewrites this workspace, first waits for the last verify that
  // read it, or with no record of one for everything already queued on
  // stream_exact.
  if (two && ent && ent->used) {
    if ((st = wait_ws(sa)) != ALSPEC_OK) return st;
    if ((st = wait_ws(se)) != ALSPEC_OK) return st;
  } else if (two && ent) {
    if (failed(hipEventRecord(h->ev_join, se), "hipEventRecord") ||
        failed(hipStreamWaitEvent(sa, h->ev_join, 0), "hipStreamWaitEvent"))
      return ALSPEC_ERR_HIP;
  } else if ((st = wait_ws(se)) != ALSPEC_OK) {
    return st;
  }
  if ((st = approx(sa)) != ALSPEC_OK) return st;
  if (two && failed(hipEventRecord(h->ev_approx, sa), "hipEventRecord"))
    return ALSPEC_ERR_HIP;
  if ((st = middle(se)) != ALSPEC_OK) return st;
  if (two &&
      failed(hipStreamWaitEvent(se, h->ev_approx, 0), "hipStreamWaitEvent"))
    return ALSPEC_ERR_HIP;
  if ((st = verify(se)) != ALSPEC_OK) return st;
  return done_ws(se);
}

alspec_status alspec_spec_decode_noalloc(
    alspec_handle *h, const alspec_params *p, const float *q, const void *k,
    const void *v, float *o_approx, float *lse_approx, float *o_exact,
    float *lse_exact, float *ratio, uint8_t *commit, float *o_committed,
    void *stream_approx, void *stream_exact, const alspec_events *ev) {
  if (!h) return ALSPEC_ERR_INVALID_ARG;
  if (!h->scratch) {
    snprintf(g_last_error, sizeof g_last_error,
             "no static scratch on device %d (devices 0..%d have one)",
             h->device, alspec::kScratchMaxDevices - 1);
    return ALSPEC_ERR_UNSUPPORTED;
  }
  size_t need = 0;
  alspec_status st = alspec_workspace_size(p, &need);
  if (st != ALSPEC_OK) return st;
  if (need > alspec::kScratchBytes) {
    snprintf(g_last_error, sizeof g_last_error,
             "workspace of %zu bytes exceeds the static scratch of %zu bytes",
             need, alspec::kScratchBytes);
    return ALSPEC_ERR_WORKSPACE;
  }
  // The scratch is passed as the fused call's workspace: the same kernels,
  // the same bits, and the same workspace ordering of uncaptured calls.
  return alspec_spec_decode(h, p, q, k, v, o_approx, lse_approx, o_exact,
                            lse_exact, ratio, commit, o_committed, h->scratch,
                            alspec::kScratchBytes, stream_approx,
                            stream_exact, ev);
}

alspec_status alspec_spec_decode_layers(alspec_handle *h,
                                        const alspec_params *p,
                                        int32_t n_layers,
                                        const alspec_layer *layers,
                                        void *stream) {
  if (!h || !p || !layers || n_layers < 1) return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  for (int j = 0; j < n_layers; ++j) {
    const alspec_layer &L = layers[j];
    if (!L.o_approx || !L.o_exact || !L.ratio || !L.commit)
      return ALSPEC_ERR_INVALID_ARG;
    if ((st = check_inputs(L.q, L.k, L.v)) != ALSPEC_OK) return st;
    if ((st = check_outputs(L.o_approx, L.o_exact, L.o_committed)) !=
        ALSPEC_OK)
      return st;
    if ((st = check_ws(L.ws, L.ws_bytes, wl)) != ALSPEC_OK) return st;
    // A workspace is in use from the launch before its layer's to the one
    // after it.  In the one-launch form a layer's splits wait for the verify
    // of the layer before on the same workspace, which the queue places
    // ahead of them only if that layer is at least three back.
    for (int d = 1; d <= 2 && j + d < n_layers; ++d)
      if (layers[j + d].ws == L.ws) return ALSPEC_ERR_WORKSPACE;
  }
  const float sm_log2 = p->sm_scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  if (p->overlap != 1) {
    // One launch per kChainMaxLayers layers, each self-contained, after the
    // table of its layers has been written into its first layer's
    // workspace by a small kernel on the same stream.
    for (int a = 0; a < n_layers; a += alspec::kChainMaxLayers) {
      const int n = n_layers - a < alspec::kChainMaxLayers
                        ? n_layers - a
                        : alspec::kChainMaxLayers;
      alspec::ChainEntry tab[alspec::kChainMaxLayers];
      for (int j = 0; j < n; ++j) {
        const alspec_layer &L = layers[a + j];
        int prev = -1;
        for (int i = j - 1; i >= 0 && prev < 0; --i)
          if (layers[a + i].ws == L.ws) prev = i;
        tab[j] = alspec::ChainEntry{L.q,          L.k,       L.v,
                                    (char *)L.ws, L.o_approx, L.lse_approx,
                                    L.o_exact,    L.lse_exact, L.ratio,
                                    L.commit,     L.o_committed, prev, 0};
      }
      char *ws0 = (char *)layers[a].ws;
      alspec::OneChainArgs ca;
      ca.n = n;
      ca.lambda = p->lambda;
      ca.ctl = ws0 + wl.off_chain_ctl;
      ca.table = (const alspec::ChainEntry *)(ws0 + wl.off_chain_table);
      ca.off_counters = (unsigned)wl.off_counters;
      ca.off_part_ml = (unsigned)wl.off_part_ml;
      ca.off_part_acc = (unsigned)wl.off_part_acc;
      ca.off_stA_ml = (unsigned)wl.off_stA_ml;
      ca.off_stA_acc = (unsigned)wl.off_stA_acc;
      ca.off_headnd = (unsigned)wl.off_headnd;
      if (failed(alspec::launch_chain_table(
                     tab, n, (alspec::ChainEntry *)(ws0 + wl.off_chain_table),
                     s),
                 "launch_chain_table") ||
          failed(alspec::launch_one_chain(pa, p->kv_dtype, ca, sm_log2, s),
                 "launch_one_chain"))
        return ALSPEC_ERR_HIP;
    }
    return ALSPEC_OK;
  }
  auto chain_layer = [&](int j) {
    const alspec_layer &L = layers[j];
    alspec::ChainLayer c;
    c.q = L.q;
    c.k = L.k;
    c.v = L.v;
    c.w = alspec::ws_ptrs(L.ws, wl);
    c.o = alspec::Outs{L.o_approx, L.lse_approx, L.o_exact, L.lse_exact,
                       L.ratio,    L.commit,     L.o_committed, p->lambda};
    return c;
  };
  alspec::ChainLayer first = chain_layer(0);
  if (failed(alspec::launch_approx_fused(pa, p->kv_dtype, first.q, first.k,
                                         first.v, sm_log2, first.w, first.o,
                                         s),
             "launch_approx_fused"))
    return ALSPEC_ERR_HIP;
  for (int j = 0; j < n_layers; ++j) {
    const alspec::ChainLayer mid = chain_layer(j);
    alspec::ChainLayer app{}, ver{};
    if (j + 1 < n_layers) app = chain_layer(j + 1);
    if (j >= 1) ver = chain_layer(j - 1);
    if (failed(alspec::launch_chain(pa, p->kv_dtype, &mid,
                                    j + 1 < n_layers ? &app : nullptr,
                                    j >= 1 ? &ver : nullptr, j >= 1,
                                    sm_log2, s),
               "launch_chain"))
      return ALSPEC_ERR_HIP;
  }
  const alspec::ChainLayer last = chain_layer(n_layers - 1);
  return hip_status(alspec::launch_merge_verify(pa, last.w, last.o, s),
                    "launch_merge_verify");
}

alspec_status alspec_order_after_verify(alspec_handle *h, void *stream) {
  if (!h) return ALSPEC_ERR_INVALID_ARG;
  // The verify stream is part of a capture only after a pipelined call was
  // captured; it must then belong to the caller's capture, and it holds
  // nothing to order a capturing stream after otherwise.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone, vs = cs;
  unsigned long long cid = 0, vid = 0;
  if (failed(hipStreamGetCaptureInfo((hipStream_t)stream, &cs, &cid),
             "hipStreamGetCaptureInfo") ||
      failed(hipStreamGetCaptureInfo(h->sv, &vs, &vid),
             "hipStreamGetCaptureInfo"))
    return ALSPEC_ERR_HIP;
  const bool c_on = cs == hipStreamCaptureStatusActive;
  const bool v_on = vs == hipStreamCaptureStatusActive;
  if (v_on && (!c_on || cid != vid)) return ALSPEC_ERR_UNSUPPORTED;
  if (c_on && !v_on) return ALSPEC_OK;
  if (failed(hipEventRecord(h->ev_verify, h->sv), "hipEventRecord"))
    return ALSPEC_ERR_HIP;
  return hip_status(hipStreamWaitEvent((hipStream_t)stream, h->ev_verify, 0),
                    "hipStreamWaitEvent");
}

}  // extern "C"

// ------------------------------------------------------ post-attention ---

namespace {

alspec_status check_post(const alspec_post_params *p) {
  if (!p) return ALSPEC_ERR_INVALID_ARG;
  if (p->batch < 1 || p->attn_dim < 8 || p->hidden < 8 || p->ffn < 8 ||
      p->qkv_dim < 1)
    return ALSPEC_ERR_INVALID_ARG;
  if (p->attn_dim % 8 || p->hidden % 8 || p->ffn % 8)
    return ALSPEC_ERR_INVALID_ARG;
  if (!(p->eps > 0.f) || !std::isfinite(p->eps)) return ALSPEC_ERR_INVALID_ARG;
  if (p->batch > ALSPEC_POST_MAX_BATCH) return ALSPEC_ERR_UNSUPPORTED;
  return ALSPEC_OK;
}

size_t post_ws_bytes(const alspec_post_params *p) {
  return alspec::align_up((size_t)p->batch * p->ffn * 4, alspec::kWsAlign);
}

}  // namespace

alspec_status alspec_post_workspace_size(const alspec_post_params *p,
                                         size_t *bytes) {
  if (!bytes) return ALSPEC_ERR_INVALID_ARG;
  const alspec_status st = check_post(p);
  if (st != ALSPEC_OK) return st;
  *bytes = post_ws_bytes(p);
  return ALSPEC_OK;
}

alspec_status alspec_post_attention(alspec_handle *h,
                                    const alspec_post_params *p,
                                    const alspec_post_weights *w,
                                    const float *o, const float *h_in,
                                    float *h_out, float *qkv,
                                    const uint8_t *skip, void *ws,
                                    size_t ws_bytes, void *stream) {
  if (!h || !w) return ALSPEC_ERR_INVALID_ARG;
  alspec_status st = check_post(p);
  if (st != ALSPEC_OK) return st;
  const void *ptrs[] = {w->w_o,    w->norm_mlp,  w->w_gate, w->w_up,
                        w->w_down, w->norm_attn, w->w_qkv,  o,
                        h_in,      h_out,        qkv};
  for (const void *q : ptrs)
    if (!q || !aligned(q, 16)) return ALSPEC_ERR_INVALID_ARG;
  if (skip && h_out == h_in) return ALSPEC_ERR_INVALID_ARG;
  if ((const void *)h_out == (const void *)o ||
      (const void *)h_out == (const void *)qkv)
    return ALSPEC_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, alspec::kWsAlign)) return ALSPEC_ERR_WORKSPACE;
  if (ws_bytes < post_ws_bytes(p)) return ALSPEC_ERR_WORKSPACE;
  alspec::PostShape sh{p->batch, p->attn_dim, p->hidden, p->ffn, p->qkv_dim,
                       p->eps};
  alspec::PostPtrs pp{};
  pp.w_o = (const uint16_t *)w->w_o;
  pp.norm_mlp = (const uint16_t *)w->norm_mlp;
  pp.w_gate = (const uint16_t *)w->w_gate;
  pp.w_up = (const uint16_t *)w->w_up;
  pp.w_down = (const uint16_t *)w->w_down;
  pp.norm_attn = (const uint16_t *)w->norm_attn;
  pp.w_qkv = (const uint16_t *)w->w_qkv;
  pp.o = o;
  pp.h_in = h_in;
  pp.h_out = h_out;
  pp.qkv = qkv;
  pp.m = (float *)ws;
  pp.skip = skip;
  return hip_status(
      alspec::launch_post_attention(sh, pp, (hipStream_t)stream),
      "launch_post_attention");
}
