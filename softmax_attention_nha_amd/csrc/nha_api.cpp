// nha_api.cpp -- the C ABI declared in include/nha.h.
//
// Host-side validation, workspace sizing and dispatch.  Every check runs before
// the first HIP call, so argument errors are reported on hosts without a GPU.
#include <math.h>
#include <string.h>

#include "nha_internal.h"

using namespace nha;

namespace {


bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Fill `s` from the descriptor; `need_T` = false for decode (T ignored).
nha_status make_shape(const nha_desc* d, bool need_T, Shape* s) {
  if (!d) return NHA_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->Hkv < 1 || d->w < 0 || d->m < 0 || d->d < 1) return NHA_ERR_INVALID_ARG;
  if (d->m == 0 && d->w < 1) return NHA_ERR_INVALID_ARG;  // no slots and no window: no keys
  if (need_T && d->T < 1) return NHA_ERR_INVALID_ARG;
  if (d->H % d->Hkv) return NHA_ERR_INVALID_ARG;
  if (!(d->rope_base >= 0.f) || !isfinite(d->rope_base)) return NHA_ERR_INVALID_ARG;
  if (!(d->scale >= 0.f) || !isfinite(d->scale)) return NHA_ERR_INVALID_ARG;
  if (d->dtype != NHA_DTYPE_F32 && d->dtype != NHA_DTYPE_BF16) return NHA_ERR_INVALID_ARG;
  if (d->no_token_shift != 0 && d->no_token_shift != 1) return NHA_ERR_INVALID_ARG;
  if (d->d != 32 && d->d != 64 && d->d != 128) return NHA_ERR_UNSUPPORTED;
  if (d->m > 64) return NHA_ERR_UNSUPPORTED;
  if (d->C != 16 && d->C != 32 && d->C != 64) return NHA_ERR_UNSUPPORTED;
  s->B = d->B;
  s->T = need_T ? d->T : 1;
  s->H = d->H;
  s->Hkv = d->Hkv;
  s->d = d->d;
  s->m = d->m;
  s->w = d->w;
  s->sh = d->no_token_shift ? 0 : d->w;
  s->C = d->C;
  s->G = d->H / d->Hkv;
  s->mp = d->m <= 32 ? 32 : 64;
  s->NC = (s->T + s->C - 1) / s->C;
  s->NQ = (s->T + 63) / 64;
  s->rope = d->rope_base > 0.f;
  s->win = d->w > 0;
  s->scale = d->scale > 0.f ? d->scale : 1.f / sqrtf((float)d->d);
  s->dtype = d->dtype;
  s->esz = d->dtype == NHA_DTYPE_BF16 ? 2 : 4;
  // grid limits (y dimension) and int32 row counts inside the kernels
  if ((long long)s->B * s->H > 65535) return NHA_ERR_UNSUPPORTED;
  if ((long long)s->B * s->T * s->H > (1LL << 31) / 8) return NHA_ERR_UNSUPPORTED;
  if ((long long)s->T + s->w > (1LL << 31) - 1) return NHA_ERR_UNSUPPORTED;
  if (need_T && slot_fwd_lds_bytes(*s) > kMaxLds) return NHA_ERR_UNSUPPORTED;
  return NHA_OK;
}

RopeTheta make_theta(const nha_desc* d) {
  RopeTheta th;
  memset(&th, 0, sizeof(th));
  if (d->rope_base > 0.f)
    for (int i = 0; i < d->d / 2; ++i) th.theta[i] = pow((double)d->rope_base, -2.0 * i / d->d);
  th.pos0 = 0;
  return th;
}

// Shapes of a continued segment: s (the segment), se (P = min(pos0, w) ring
// rows prepended) and the RoPE position of extended row 0.
nha_status cont_shapes(const nha_desc* desc, long long pos0, Shape* s, Shape* se, RopeTheta* th) {
  nha_status rc = make_shape(desc, true, s);
  if (rc != NHA_OK) return rc;
  if (pos0 < 0 || pos0 > (1LL << 40)) return NHA_ERR_INVALID_ARG;
  if (desc->no_token_shift) return NHA_ERR_UNSUPPORTED;
  const long long P = pos0 < desc->w ? pos0 : desc->w;
  if ((long long)desc->T + P > (1LL << 31) - 1) return NHA_ERR_UNSUPPORTED;
  nha_desc de = *desc;
  de.T = desc->T + (int)P;
  rc = make_shape(&de, true, se);
  if (rc != NHA_OK) return rc;
  *th = make_theta(desc);
  th->pos0 = pos0 - P;
  return NHA_OK;
}

}  // namespace

namespace nha {
int device_cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// The calling thread's side stream and events, per device (created on first
// use, released by nha_release_side_streams).
static thread_local Fork side_cache[64];

Fork side_fork(bool enabled) {
  Fork none;
  if (!enabled) return none;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return none;
  Fork& c = side_cache[dev];
  if (!c.side) {
    hipStream_t s = nullptr;
    hipEvent_t a = nullptr, b = nullptr, e = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return none;
    if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      if (b) (void)hipEventDestroy(b);
      (void)hipStreamDestroy(s);
      return none;
    }
    c.side = s;
    c.ev_fork = a;
    c.ev_join = b;
    c.ev_mid = e;
  }
  return c;
}
}  // namespace nha


extern "C" {

const char* nha_status_string(nha_status s) {
  switch (s) {
    case NHA_OK: return "NHA_OK";
    case NHA_ERR_INVALID_ARG: return "NHA_ERR_INVALID_ARG: invalid argument";
    case NHA_ERR_UNSUPPORTED: return "NHA_ERR_UNSUPPORTED: valid but unsupported shape";
    case NHA_ERR_WORKSPACE: return "NHA_ERR_WORKSPACE: workspace too small";
    case NHA_ERR_HIP: return "NHA_ERR_HIP: HIP launch failed";
  }
  return "unknown nha_status";
}

nha_status nha_release_side_streams(void) {
  nha_status rc = NHA_OK;
  int cur = -1;
  bool have_cur = false;
  for (int dev = 0; dev < 64; ++dev) {
    Fork& c = side_cache[dev];
    if (!c.side) continue;
    if (!have_cur) have_cur = hipGetDevice(&cur) == hipSuccess;
    // the handles belong to `dev`: destroy them with it current
    if (hipSetDevice(dev) != hipSuccess) rc = NHA_ERR_HIP;
    if (hipEventDestroy(c.ev_fork) != hipSuccess) rc = NHA_ERR_HIP;
    if (hipEventDestroy(c.ev_join) != hipSuccess) rc = NHA_ERR_HIP;
    if (hipEventDestroy(c.ev_mid) != hipSuccess) rc = NHA_ERR_HIP;
    if (hipStreamDestroy(c.side) != hipSuccess) rc = NHA_ERR_HIP;
    c = Fork();
  }
  if (have_cur && hipSetDevice(cur) != hipSuccess) rc = NHA_ERR_HIP;
  return rc;
}

nha_status nha_check_desc(const nha_desc* desc) {
  Shape s;
  return make_shape(desc, true, &s);
}

size_t nha_fwd_workspace_size(const nha_desc* desc) {
  Shape s;
  if (make_shape(desc, true, &s) != NHA_OK) return 0;
  return fwd_ws_layout(s).total;
}

size_t nha_bwd_workspace_size(const nha_desc* desc) {
  Shape s;
  if (make_shape(desc, true, &s) != NHA_OK) return 0;
  if (slot_bwd_lds_bytes(s) > kMaxLds) return 0;
  return bwd_ws_bytes(s);
}

size_t nha_decode_state_size(const nha_desc* desc) {
  Shape s;
  if (make_shape(desc, false, &s) != NHA_OK) return 0;
  return state_layout(s).total;
}

nha_status nha_fwd(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                   void* o, float* lse, void* state_out, void* ws, size_t ws_bytes, void* stream) {
  return nha_fwd_timed(desc, q, k, v, alpha, o, lse, state_out, ws, ws_bytes, stream, nullptr);
}

nha_status nha_fwd_timed(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                         void* o, float* lse, void* state_out, void* ws, size_t ws_bytes, void* stream,
                         void* const* events) {
  Shape s;
  nha_status rc = make_shape(desc, true, &s);
  if (rc != NHA_OK) return rc;
  if (!q || !k || !v || (!alpha && s.m > 0) || !o || !ws) return NHA_ERR_INVALID_ARG;  // m = 0: no gates
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(alpha) || !aligned16(o) || !aligned16(ws) ||
      (lse && !aligned16(lse)) || (state_out && !aligned16(state_out)))
    return NHA_ERR_INVALID_ARG;
  if (ws_bytes < fwd_ws_layout(s).total) return NHA_ERR_WORKSPACE;
  FwdPtrs p{q, k, v, alpha, o, lse, state_out, (char*)ws, events};
  hipError_t e = launch_fwd(s, make_theta(desc), p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

nha_status nha_fwd_noalloc(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                           void* o, float* lse, void* state_out, void* stream) {
  Shape s;
  nha_status rc = make_shape(desc, true, &s);
  if (rc != NHA_OK) return rc;
  if (!q || !k || !v || (!alpha && s.m > 0) || !o) return NHA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(alpha) || !aligned16(o) ||
      (lse && !aligned16(lse)) || (state_out && !aligned16(state_out)))
    return NHA_ERR_INVALID_ARG;
  if (fwd_ws_layout(s).total > kNoallocScratchBytes) return NHA_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (noalloc_scratch(&scratch) != hipSuccess || !scratch) return NHA_ERR_HIP;
  FwdPtrs p{q, k, v, alpha, o, lse, state_out, (char*)scratch, nullptr};
  p.one_stream = true;
  hipError_t e = launch_fwd(s, make_theta(desc), p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

size_t nha_weighted_workspace_size(const nha_desc* desc) {
  Shape s;
  if (make_shape(desc, true, &s) != NHA_OK || s.m < 1 || s.w < 1) return 0;
  if (slot_bwd_lds_bytes(s) > kMaxLds) return 0;
  return weighted_ws_bytes(s);
}

nha_status nha_fwd_weighted(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                            const float* lam, void* o, float* lse2, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  nha_status rc = make_shape(desc, true, &s);
  if (rc != NHA_OK) return rc;
  if (s.m < 1 || s.w < 1) return NHA_ERR_INVALID_ARG;  // both softmaxes need keys
  if (!q || !k || !v || !alpha || !lam || !o || !ws) return NHA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, alpha, lam, o, ws};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return NHA_ERR_INVALID_ARG;
  if (lse2 && !aligned16(lse2)) return NHA_ERR_INVALID_ARG;
  if (slot_bwd_lds_bytes(s) > kMaxLds) return NHA_ERR_UNSUPPORTED;
  if (ws_bytes < weighted_ws_bytes(s)) return NHA_ERR_WORKSPACE;
  WeightedPtrs p{q, k, v, alpha, lam, o, lse2, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, (char*)ws};
  hipError_t e = launch_fwd_weighted(s, make_theta(desc), p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

nha_status nha_bwd_weighted(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                            const float* lam, const void* dO, void* dq, void* dk, void* dv, float* dalpha,
                            float* dlam, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  nha_status rc = make_shape(desc, true, &s);
  if (rc != NHA_OK) return rc;
  if (s.m < 1 || s.w < 1) return NHA_ERR_INVALID_ARG;
  if (!q || !k || !v || !alpha || !lam || !dO || !dq || !dk || !dv || !dalpha || !ws) return NHA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, alpha, lam, dO, dq, dk, dv, dalpha, ws};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return NHA_ERR_INVALID_ARG;
  if (dlam && !aligned16(dlam)) return NHA_ERR_INVALID_ARG;
  if (slot_bwd_lds_bytes(s) > kMaxLds) return NHA_ERR_UNSUPPORTED;
  if (ws_bytes < weighted_ws_bytes(s)) return NHA_ERR_WORKSPACE;
  WeightedPtrs p{q, k, v, alpha, lam, nullptr, nullptr, dO, dq, dk, dv, dalpha, dlam, (char*)ws};
  hipError_t e = launch_bwd_weighted(s, make_theta(desc), p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

size_t nha_continue_workspace_size(const nha_desc* desc) {
  Shape s, se;
  RopeTheta th;
  if (cont_shapes(desc, desc ? desc->w : 0, &s, &se, &th) != NHA_OK) return 0;  // P = w: the largest
  if (slot_bwd_lds_bytes(se) > kMaxLds) return 0;
  const size_t f = cont_ws_bytes(se, false), b = cont_ws_bytes(se, true);
  return f > b ? f : b;
}

nha_status nha_fwd_continue(const nha_desc* desc, long long pos0, const void* state_in, const void* q, const void* k,
                            const void* v, const void* alpha, void* o, float* lse, void* state_out, void* ws,
                            size_t ws_bytes, void* stream) {
  Shape s, se;
  RopeTheta th;
  nha_status rc = cont_shapes(desc, pos0, &s, &se, &th);
  if (rc != NHA_OK) return rc;
  if (!state_in || !q || !k || !v || (!alpha && s.m > 0) || !o || !ws) return NHA_ERR_INVALID_ARG;
  const void* ptrs[] = {state_in, q, k, v, alpha, o, ws};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return NHA_ERR_INVALID_ARG;
  if ((lse && !aligned16(lse)) || (state_out && !aligned16(state_out))) return NHA_ERR_INVALID_ARG;
  if (ws_bytes < cont_ws_bytes(se, false)) return NHA_ERR_WORKSPACE;
  ContPtrs p{q, k, v, alpha, state_in, o, lse, state_out, nullptr, nullptr, nullptr, nullptr, nullptr,
             nullptr, nullptr, nullptr, nullptr, (char*)ws};
  hipError_t e = launch_fwd_continue(s, se, th, p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

nha_status nha_bwd_continue(const nha_desc* desc, long long pos0, const void* state_in, const void* q, const void* k,
                            const void* v, const void* alpha, const void* o, const float* lse, const void* dO,
                            void* dq, void* dk, void* dv, float* dalpha, float* ds0k, float* ds0v, void* drk,
                            void* drv, void* ws, size_t ws_bytes, void* stream) {
  Shape s, se;
  RopeTheta th;
  nha_status rc = cont_shapes(desc, pos0, &s, &se, &th);
  if (rc != NHA_OK) return rc;
  if (slot_bwd_lds_bytes(se) > kMaxLds) return NHA_ERR_UNSUPPORTED;
  if (!state_in || !q || !k || !v || ((!alpha || !dalpha) && s.m > 0) || !o || !lse || !dO || !dq || !dk || !dv ||
      !ds0k || !ds0v || !ws)
    return NHA_ERR_INVALID_ARG;
  const void* ptrs[] = {state_in, q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, ds0k, ds0v, ws};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return NHA_ERR_INVALID_ARG;
  if ((drk && !aligned16(drk)) || (drv && !aligned16(drv))) return NHA_ERR_INVALID_ARG;
  if (ws_bytes < cont_ws_bytes(se, true)) return NHA_ERR_WORKSPACE;
  ContPtrs p{q, k, v, alpha, state_in, (void*)o, (float*)lse, nullptr, dO, dq, dk, dv, dalpha, ds0k, ds0v,
             drk, drv, (char*)ws};
  hipError_t e = launch_bwd_continue(s, se, th, p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

nha_status nha_fwd_s0(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                      const float* s0k, const float* s0v, void* o, float* lse, void* state_out, void* ws,
                      size_t ws_bytes, void* stream) {
  Shape s;
  nha_status rc = make_shape(desc, true, &s);
  if (rc != NHA_OK) return rc;
  if (!q || !k || !v || !alpha || !o || !ws || !s0k || !s0v) return NHA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(alpha) || !aligned16(o) || !aligned16(ws) ||
      !aligned16(s0k) || !aligned16(s0v) || (lse && !aligned16(lse)) || (state_out && !aligned16(state_out)))
    return NHA_ERR_INVALID_ARG;
  if (ws_bytes < fwd_ws_layout(s).total) return NHA_ERR_WORKSPACE;
  FwdPtrs p{q, k, v, alpha, o, lse, state_out, (char*)ws, nullptr};
  p.s0k = s0k;
  p.s0v = s0v;
  hipError_t e = launch_fwd(s, make_theta(desc), p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

nha_status nha_bwd(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                   const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv, float* dalpha,
                   void* ws, size_t ws_bytes, void* stream) {
  return nha_bwd_timed(desc, q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, ws, ws_bytes, stream, nullptr);
}

static nha_status bwd_common(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                             const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                             float* dalpha, void* ws, size_t ws_bytes, void* stream, void* const* events,
                             bool after_fwd, const float* s0k = nullptr, const float* s0v = nullptr,
                             float* ds0k = nullptr, float* ds0v = nullptr) {
  Shape s;
  nha_status rc = make_shape(desc, true, &s);
  if (rc != NHA_OK) return rc;
  if (slot_bwd_lds_bytes(s) > kMaxLds) return NHA_ERR_UNSUPPORTED;
  if (!q || !k || !v || ((!alpha || !dalpha) && s.m > 0) || !o || !lse || !dO || !dq || !dk || !dv || !ws)
    return NHA_ERR_INVALID_ARG;  // m = 0: no gates, no dalpha
  const void* ptrs[] = {q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, ws};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return NHA_ERR_INVALID_ARG;
  if (ws_bytes < bwd_ws_bytes(s)) return NHA_ERR_WORKSPACE;
  BwdPtrs p{q, k, v, alpha, o, dO, lse, dq, dk, dv, dalpha, (char*)ws, events, after_fwd};
  p.s0k = s0k;
  p.s0v = s0v;
  p.ds0k = ds0k;
  p.ds0v = ds0v;
  hipError_t e = launch_bwd(s, make_theta(desc), p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

nha_status nha_bwd_timed(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                         const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                         float* dalpha, void* ws, size_t ws_bytes, void* stream, void* const* events) {
  return bwd_common(desc, q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, ws, ws_bytes, stream, events, false);
}

nha_status nha_bwd_after_fwd(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                             const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                             float* dalpha, void* ws, size_t ws_bytes, void* stream) {
  return bwd_common(desc, q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, ws, ws_bytes, stream, nullptr, true);
}

nha_status nha_bwd_after_fwd_timed(const nha_desc* desc, const void* q, const void* k, const void* v,
                                   const void* alpha, const void* o, const float* lse, const void* dO, void* dq,
                                   void* dk, void* dv, float* dalpha, void* ws, size_t ws_bytes, void* stream,
                                   void* const* events) {
  return bwd_common(desc, q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, ws, ws_bytes, stream, events, true);
}

nha_status nha_bwd_s0(const nha_desc* desc, const void* q, const void* k, const void* v, const void* alpha,
                      const float* s0k, const float* s0v, const void* o, const float* lse, const void* dO, void* dq,
                      void* dk, void* dv, float* dalpha, float* ds0k, float* ds0v, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!s0k || !s0v || !ds0k || !ds0v) return NHA_ERR_INVALID_ARG;
  if (!aligned16(s0k) || !aligned16(s0v) || !aligned16(ds0k) || !aligned16(ds0v)) return NHA_ERR_INVALID_ARG;
  return bwd_common(desc, q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, ws, ws_bytes, stream, nullptr, false, s0k,
                    s0v, ds0k, ds0v);
}

int nha_stage_names(const nha_desc* desc, int backward, int with_state, const char** names, int max) {
  Shape s;
  if (make_shape(desc, true, &s) != NHA_OK) return -1;
  return backward ? bwd_stages(s, backward == 2, names, max) : fwd_stages(s, with_state != 0, names, max);
}

nha_status nha_decode_step(const nha_desc* desc, const void* q_t, const void* k_t, const void* v_t,
                           const void* alpha_t, void* state, void* o_t, void* stream) {
  Shape s;
  nha_status rc = make_shape(desc, false, &s);
  if (rc != NHA_OK) return rc;
  if (!q_t || !k_t || !v_t || (!alpha_t && s.m > 0) || !state || !o_t) return NHA_ERR_INVALID_ARG;
  const void* ptrs[] = {q_t, k_t, v_t, alpha_t, state, o_t};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return NHA_ERR_INVALID_ARG;
  if ((long long)s.m + s.w > (long long)kDecodeSplitMax * kDecodeKeysPerSplit) return NHA_ERR_UNSUPPORTED;
  DecodePtrs p{q_t, k_t, v_t, alpha_t, state, o_t};
  hipError_t e = launch_decode(s, make_theta(desc), p, (hipStream_t)stream);
  return e == hipSuccess ? NHA_OK : NHA_ERR_HIP;
}

}  // extern "C"
