// nha_continue.hip -- chunked prefill: the forward (and its backward) over a
// segment of T tokens that continues a decode state (gfx950).
//
// The ai.info page's "Future Directions" (item 1) names the slot states as
// the place to carry context across segments; here a segment continues the
// state that nha_fwd / nha_decode_step / a previous segment left after pos0
// tokens: its m slot states, its ring of the last w raw keys and values, and
// the absorptions those ring tokens still owe (token p enters the slots at
// step p + w, with that step's gate).
//
// Reduction to the whole-sequence forward: prepend the P = min(pos0, w) ring
// tokens (positions pos0 - P .. pos0 - 1) to the segment.  On that extended
// sequence, row e (absolute position pos0 - P + e) absorbs row e - w with
// gate alpha_e exactly when e >= w -- the token-shift rule of nha_fwd:
//   * P = w (pos0 >= w): the ring rows e < w absorb nothing (their own
//     absorptions happened before pos0), and every segment row e >= w absorbs
//     the token w before it;
//   * P = pos0 < w: rows are absolute positions, and the rule is the
//     sequence's own;
// the slots start from the state's S (decayed only by absorbing steps, as
// for nha_fwd_s0), and the window of the first segment rows reaches back into
// the ring rows.  The ring rows get zero queries and their outputs are
// dropped; RoPE uses absolute positions (row e at pos0 - P + e).  The
// backward runs the same way with zero incoming gradients on the ring rows,
// and returns, besides the segment's gradients, those of the state it
// started from: dS0 of the slots and the gradients of the ring's keys and
// values (window reads and pending absorptions).
#include "nha_common.h"
#include "nha_internal.h"

namespace nha {

namespace {

// Extended-sequence buffers after the whole-sequence workspace of the
// extended shape.
struct ContWs {
  size_t base;                  // nha_fwd / nha_bwd workspace of the extended shape
  size_t qe, ke, ve, ae, oe, le;  // extended q, k, v, alpha, o ([B][Te][heads][*]); lse [B][H][Te] float
  size_t doe, dqe, dke, dve, dae;  // backward: dO, dq, dk, dv (dtype), dalpha (float)
  size_t total;
};

ContWs cont_ws_layout(const Shape& se, bool bwd) {
  ContWs L;
  size_t off = align256(bwd ? bwd_ws_bytes(se) : fwd_ws_layout(se).total);
  L.base = 0;
  const size_t BT = (size_t)se.B * se.T;
  const size_t qb = BT * se.H * se.d * se.esz, kb = BT * se.Hkv * se.d * se.esz;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.qe = take(qb);
  L.ke = take(kb);
  L.ve = take(kb);
  L.ae = take(BT * se.Hkv * se.m * se.esz);
  L.oe = take(qb);
  L.le = take(BT * se.H * 4);
  L.doe = L.dqe = L.dke = L.dve = L.dae = 0;
  if (bwd) {
    L.doe = take(qb);
    L.dqe = take(qb);
    L.dke = take(kb);
    L.dve = take(kb);
    L.dae = take(BT * se.Hkv * se.m * 4);
  }
  L.total = off;
  return L;
}

// dst [B][Te][heads][width]: rows e >= P copy src [B][Te - P][heads][width]
// row e - P; rows e < P take ring row (rpos0 + e) mod w of ring
// [B][heads][w][width] when ring is given, else `fill`.  One element per
// thread (grid-stride).
template <typename T>
__global__ __launch_bounds__(256) void k_ext_rows(T* __restrict__ dst, const T* __restrict__ src,
                                                  const T* __restrict__ ring, int B, int Te, int P, int heads,
                                                  int width, long long rpos0, int w, float fill) {
  const long n = (long)B * Te * heads * width;
  const int Tn = Te - P;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int c = (int)(i % width);
    const long r = i / width;
    const int hd = (int)(r % heads);
    const long be = r / heads;
    const int e = (int)(be % Te), b = (int)(be / Te);
    T x;
    if (e >= P)
      x = src[(((long)b * Tn + (e - P)) * heads + hd) * width + c];
    else if (ring)
      x = ring[(((long)b * heads + hd) * w + (long)((rpos0 + e) % w)) * width + c];
    else
      x = to_t<T>(fill);
    dst[i] = x;
  }
}

// dst [B][Tn][heads][width] = rows P .. P + Tn - 1 of src [B][Te][heads][width].
template <typename T>
__global__ __launch_bounds__(256) void k_seg_rows(T* __restrict__ dst, const T* __restrict__ src, int B, int Tn,
                                                  int P, int heads, int width) {
  const long n = (long)B * Tn * heads * width, per_b = (long)Tn * heads * width;
  const int Te = Tn + P;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long b = i / per_b, rest = i % per_b;
    dst[i] = src[(b * Te + P) * heads * width + rest];
  }
}

// Per-row statistics [B*H][Te] <-> [B*H][Tn]: to_ext copies the segment's
// values to columns >= P and zeroes columns < P; otherwise columns >= P are
// copied back.
__global__ __launch_bounds__(256) void k_stat_cols(float* __restrict__ ext, float* __restrict__ seg, int BH, int Tn,
                                                   int P, int to_ext) {
  const int Te = Tn + P;
  const long n = (long)BH * (to_ext ? Te : Tn);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    if (to_ext) {
      const long bh = i / Te;
      const int e = (int)(i % Te);
      ext[i] = e >= P ? seg[bh * Tn + (e - P)] : 0.f;
    } else {
      const long bh = i / Tn;
      const int t = (int)(i % Tn);
      seg[i] = ext[bh * Te + P + t];
    }
  }
}

// Ring-layout gradients dring [B][Hkv][w][d]: ring row r holds position p =
// the one of rpos0 .. rpos0 + P - 1 congruent to r mod w (if any), whose
// gradient is row p - rpos0 of the extended dk / dv; other rows are zero.
template <typename T>
__global__ __launch_bounds__(256) void k_ring_grad(T* __restrict__ dring, const T* __restrict__ dext, int B, int Te,
                                                   int P, int Hkv, int d, int w, long long rpos0) {
  const long n = (long)B * Hkv * w * d;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int c = (int)(i % d);
    const long rr = i / d;
    const int r = (int)(rr % w);
    const long u = rr / w;
    const int b = (int)(u / Hkv), g = (int)(u % Hkv);
    const int e = (int)(((r - rpos0) % w + w) % w);  // rpos0 + e == r (mod w), 0 <= e < w
    dring[i] = e < P ? dext[(((long)b * Te + e) * Hkv + g) * d + c] : to_t<T>(0.f);
  }
}

unsigned grid_for(long n) {
  long g = (n + 255) / 256;
  return (unsigned)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

template <typename T>
hipError_t fwd_cont_t(const Shape& s, const Shape& se, const RopeTheta& th, const ContPtrs& p, hipStream_t st) {
  const ContWs L = cont_ws_layout(se, false);
  const StateLayout SL = state_layout(s);
  const char* sin = (const char*)p.state_in;
  const int P = se.T - s.T, B = s.B;
  const long long rpos0 = th.pos0;  // absolute position of extended row 0
  char* ws = p.ws;
  auto ext = [&](size_t off, const void* src, const void* ring, int heads, int width, float fill) {
    const long n = (long)B * se.T * heads * width;
    hipLaunchKernelGGL(k_ext_rows<T>, dim3(grid_for(n)), dim3(256), 0, st, (T*)(ws + off), (const T*)src,
                       (const T*)ring, B, se.T, P, heads, width, rpos0, s.w, fill);
  };
  ext(L.qe, p.q, nullptr, s.H, s.d, 0.f);
  ext(L.ke, p.k, s.w > 0 ? sin + SL.rk : nullptr, s.Hkv, s.d, 0.f);
  ext(L.ve, p.v, s.w > 0 ? sin + SL.rv : nullptr, s.Hkv, s.d, 0.f);
  ext(L.ae, p.alpha, nullptr, s.Hkv, s.m, 1.f);
  FwdPtrs f{ws + L.qe, ws + L.ke, ws + L.ve, ws + L.ae, ws + L.oe, (float*)(ws + L.le), p.state_out, ws, nullptr};
  f.s0k = (const float*)(sin + SL.sk);
  f.s0v = (const float*)(sin + SL.sv);
  hipError_t e = launch_fwd(se, th, f, st);
  if (e != hipSuccess) return e;
  const long no = (long)B * s.T * s.H * s.d;
  hipLaunchKernelGGL(k_seg_rows<T>, dim3(grid_for(no)), dim3(256), 0, st, (T*)p.o, (const T*)(ws + L.oe), B, s.T,
                     P, s.H, s.d);
  if (p.lse)
    hipLaunchKernelGGL(k_stat_cols, dim3(grid_for((long)B * s.H * s.T)), dim3(256), 0, st, (float*)(ws + L.le),
                       p.lse, B * s.H, s.T, P, 0);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_cont_t(const Shape& s, const Shape& se, const RopeTheta& th, const ContPtrs& p, hipStream_t st) {
  const ContWs L = cont_ws_layout(se, true);
  const StateLayout SL = state_layout(s);
  const char* sin = (const char*)p.state_in;
  const int P = se.T - s.T, B = s.B;
  const long long rpos0 = th.pos0;
  char* ws = p.ws;
  auto ext = [&](size_t off, const void* src, const void* ring, int heads, int width, float fill) {
    const long n = (long)B * se.T * heads * width;
    hipLaunchKernelGGL(k_ext_rows<T>, dim3(grid_for(n)), dim3(256), 0, st, (T*)(ws + off), (const T*)src,
                       (const T*)ring, B, se.T, P, heads, width, rpos0, s.w, fill);
  };
  ext(L.qe, p.q, nullptr, s.H, s.d, 0.f);
  ext(L.ke, p.k, s.w > 0 ? sin + SL.rk : nullptr, s.Hkv, s.d, 0.f);
  ext(L.ve, p.v, s.w > 0 ? sin + SL.rv : nullptr, s.Hkv, s.d, 0.f);
  ext(L.ae, p.alpha, nullptr, s.Hkv, s.m, 1.f);
  // ring rows: zero query, output, incoming gradient and lse -- every term
  // they would contribute to the gradients carries their zero dO
  ext(L.oe, p.o, nullptr, s.H, s.d, 0.f);
  ext(L.doe, p.dO, nullptr, s.H, s.d, 0.f);
  hipLaunchKernelGGL(k_stat_cols, dim3(grid_for((long)B * s.H * se.T)), dim3(256), 0, st, (float*)(ws + L.le),
                     (float*)p.lse, B * s.H, s.T, P, 1);
  BwdPtrs b{ws + L.qe, ws + L.ke, ws + L.ve, ws + L.ae, ws + L.oe, ws + L.doe, (const float*)(ws + L.le),
            ws + L.dqe, ws + L.dke, ws + L.dve, (float*)(ws + L.dae), ws, nullptr, false};
  b.s0k = (const float*)(sin + SL.sk);
  b.s0v = (const float*)(sin + SL.sv);
  b.ds0k = p.ds0k;
  b.ds0v = p.ds0v;
  hipError_t e = launch_bwd(se, th, b, st);
  if (e != hipSuccess) return e;
  auto seg = [&](void* dst, size_t off, int heads, int width, bool isf) {
    const long n = (long)B * s.T * heads * width;
    if (isf)
      hipLaunchKernelGGL(k_seg_rows<float>, dim3(grid_for(n)), dim3(256), 0, st, (float*)dst,
                         (const float*)(ws + off), B, s.T, P, heads, width);
    else
      hipLaunchKernelGGL(k_seg_rows<T>, dim3(grid_for(n)), dim3(256), 0, st, (T*)dst, (const T*)(ws + off), B, s.T,
                         P, heads, width);
  };
  seg(p.dq, L.dqe, s.H, s.d, false);
  seg(p.dk, L.dke, s.Hkv, s.d, false);
  seg(p.dv, L.dve, s.Hkv, s.d, false);
  seg(p.dalpha, L.dae, s.Hkv, s.m, true);
  if (s.w > 0) {
    const long n = (long)B * s.Hkv * s.w * s.d;
    if (p.drk)
      hipLaunchKernelGGL(k_ring_grad<T>, dim3(grid_for(n)), dim3(256), 0, st, (T*)p.drk, (const T*)(ws + L.dke), B,
                         se.T, P, s.Hkv, s.d, s.w, rpos0);
    if (p.drv)
      hipLaunchKernelGGL(k_ring_grad<T>, dim3(grid_for(n)), dim3(256), 0, st, (T*)p.drv, (const T*)(ws + L.dve), B,
                         se.T, P, s.Hkv, s.d, s.w, rpos0);
  }
  return hipGetLastError();
}

}  // namespace

size_t cont_ws_bytes(const Shape& se, bool bwd) { return cont_ws_layout(se, bwd).total; }

hipError_t launch_fwd_continue(const Shape& s, const Shape& se, const RopeTheta& th, const ContPtrs& p,
                               hipStream_t st) {
  return s.dtype == NHA_DTYPE_BF16 ? fwd_cont_t<bf16>(s, se, th, p, st) : fwd_cont_t<float>(s, se, th, p, st);
}

hipError_t launch_bwd_continue(const Shape& s, const Shape& se, const RopeTheta& th, const ContPtrs& p,
                               hipStream_t st) {
  return s.dtype == NHA_DTYPE_BF16 ? bwd_cont_t<bf16>(s, se, th, p, st) : bwd_cont_t<float>(s, se, th, p, st);
}

}  // namespace nha
