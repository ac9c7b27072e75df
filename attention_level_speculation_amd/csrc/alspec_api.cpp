// C ABI of the speculative flash-decode step: argument validation, the split
// plan, and the order of kernels and events on the caller's streams.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "alspec.h"
#include "alspec_kernels.h"
#include "alspec_plan.h"

struct alspec_handle {
  int device;
  hipEvent_t ev_join;    // exact stream -> approximation stream
  hipEvent_t ev_approx;  // approximation stream -> exact stream
};

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

alspec_status hip_status(hipError_t e) {
  return e == hipSuccess ? ALSPEC_OK : ALSPEC_ERR_HIP;
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
  if ((a && !aligned(a, 16)) || (b && !aligned(b, 16)) || (c && !aligned(c, 16)))
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

alspec_status record(void *ev, hipStream_t s) {
  if (!ev) return ALSPEC_OK;
  return hip_status(hipEventRecord((hipEvent_t)ev, s));
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
  if (hipGetDeviceCount(&n) != hipSuccess) return ALSPEC_ERR_HIP;
  if (device < 0 || device >= n) return ALSPEC_ERR_INVALID_ARG;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return ALSPEC_ERR_HIP;
  if (hipSetDevice(device) != hipSuccess) return ALSPEC_ERR_HIP;
  alspec_handle *h = (alspec_handle *)calloc(1, sizeof(alspec_handle));
  alspec_status st = ALSPEC_OK;
  if (!h) {
    st = ALSPEC_ERR_INVALID_ARG;
  } else {
    h->device = device;
    if (hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) !=
            hipSuccess ||
        hipEventCreateWithFlags(&h->ev_approx, hipEventDisableTiming) !=
            hipSuccess) {
      if (h->ev_join) (void)hipEventDestroy(h->ev_join);
      free(h);
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
  return hip_status(alspec::launch_partials(
      pa, p->kv_dtype, alspec::kPartialsApprox, true, q, k, v,
      p->sm_scale * kLog2e, w, o, (hipStream_t)stream));
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
  const alspec::Outs none{};
  if (include_sink_window) {
    hipError_t e =
        alspec::launch_partials(pa, p->kv_dtype, alspec::kPartialsStates,
                                true, q, k, v, sm_log2, w, none, s);
    if (e != hipSuccess) return ALSPEC_ERR_HIP;
  }
  return hip_status(alspec::launch_partials(pa, p->kv_dtype,
                                            alspec::kPartialsStates, false, q,
                                            k, v, sm_log2, w, none, s));
}

alspec_status alspec_lse_combine(alspec_handle *h, const alspec_params *p,
                                 const void *ws, size_t ws_bytes,
                                 float *o_exact, float *lse_exact,
                                 void *stream) {
  if (!h || !p || !o_exact) return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  if ((st = check_ws(ws, ws_bytes, wl)) != ALSPEC_OK) return st;
  const alspec::WsPtrs w = alspec::ws_ptrs((void *)ws, wl);
  return hip_status(alspec::launch_lse_combine(pa, w, o_exact, lse_exact,
                                               (hipStream_t)stream));
}

alspec_status alspec_verify(alspec_handle *h, const alspec_params *p,
                            const float *o_approx, const float *o_exact,
                            float *ratio, uint8_t *commit, float *o_committed,
                            void *stream) {
  if (!h || !p || !o_approx || !o_exact || !ratio || !commit)
    return ALSPEC_ERR_INVALID_ARG;
  alspec::PlanArgs pa;
  alspec::Workspace wl;
  alspec_status st = alspec::make_plan(p, &pa, &wl);
  if (st != ALSPEC_OK) return st;
  return hip_status(alspec::launch_verify(pa, o_approx, o_exact, ratio, commit,
                                          o_committed, p->lambda,
                                          (hipStream_t)stream));
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

  if (!p->overlap) {
    // Approximation first, then the exact pass, in one stream: no
    // cross-stream wait between the kernels.  The approximation stream is
    // handed o_approx through an event, so work queued there after this
    // call runs while the exact pass does.
    if ((st = record(E.approx_begin, se)) != ALSPEC_OK) return st;
    if (alspec::launch_partials(pa, p->kv_dtype, alspec::kPartialsApprox,
                                true, q, k, v, sm_log2, w, o,
                                se) != hipSuccess)
      return ALSPEC_ERR_HIP;
    if ((st = record(E.approx_end, se)) != ALSPEC_OK) return st;
    if (two) {
      if (hipEventRecord(h->ev_approx, se) != hipSuccess) return ALSPEC_ERR_HIP;
      if (hipStreamWaitEvent(sa, h->ev_approx, 0) != hipSuccess)
        return ALSPEC_ERR_HIP;
    }
    if ((st = record(E.exact_begin, se)) != ALSPEC_OK) return st;
    if (alspec::launch_partials(pa, p->kv_dtype, alspec::kPartialsStates,
                                false, q, k, v, sm_log2, w, o,
                                se) != hipSuccess)
      return ALSPEC_ERR_HIP;
    if ((st = record(E.exact_end, se)) != ALSPEC_OK) return st;
    if (alspec::launch_merge_verify(pa, w, o, se) != hipSuccess)
      return ALSPEC_ERR_HIP;
    return record(E.verify_end, se);
  }

  // Overlap: the approximation (on stream_approx) and the middle splits (on
  // stream_exact) start together; the exact merge waits for both.  The
  // approximation reuses this workspace, so it is first ordered after
  // everything the exact stream already holds (earlier calls' merges).
  if (two) {
    if (hipEventRecord(h->ev_join, se) != hipSuccess) return ALSPEC_ERR_HIP;
    if (hipStreamWaitEvent(sa, h->ev_join, 0) != hipSuccess)
      return ALSPEC_ERR_HIP;
  }
  if ((st = record(E.approx_begin, sa)) != ALSPEC_OK) return st;
  if (alspec::launch_partials(pa, p->kv_dtype, alspec::kPartialsApprox, true,
                              q, k, v, sm_log2, w, o, sa) != hipSuccess)
    return ALSPEC_ERR_HIP;
  if ((st = record(E.approx_end, sa)) != ALSPEC_OK) return st;
  if (two && hipEventRecord(h->ev_approx, sa) != hipSuccess)
    return ALSPEC_ERR_HIP;
  if ((st = record(E.exact_begin, se)) != ALSPEC_OK) return st;
  if (alspec::launch_partials(pa, p->kv_dtype, alspec::kPartialsStates, false,
                              q, k, v, sm_log2, w, o, se) != hipSuccess)
    return ALSPEC_ERR_HIP;
  if ((st = record(E.exact_end, se)) != ALSPEC_OK) return st;
  if (two && hipStreamWaitEvent(se, h->ev_approx, 0) != hipSuccess)
    return ALSPEC_ERR_HIP;
  if (alspec::launch_merge_verify(pa, w, o, se) != hipSuccess)
    return ALSPEC_ERR_HIP;
  return record(E.verify_end, se);
}

}  // extern "C"
