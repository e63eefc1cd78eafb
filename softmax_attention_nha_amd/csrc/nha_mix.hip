// nha_mix.hip -- the weighted-fusion ablation of the NHA operator (gfx950).
//
// The ai.info page's findings ("Unified softmax beats weighted fusion")
// compare the unified softmax with a weighted sum of separately normalised
// reads -- a fixed coefficient, or a learned sequence-dependent one -- which
// is how the intra-layer hybrids of the Paper-Notes page's 现有痛点 paragraph
// fuse their linear and local branches.  Per (token t, query head h), with the
// slot logits and the window logits each under their own softmax,
//     o_t = lam_t o^L_t + (1 - lam_t) o^W_t .
// The same kernels as the method compute both reads: the slot branch's
// partial o^L / lse^L is exactly the separately normalised slot read, and the
// window kernel started from an empty softmax is the window read.  Gradients:
// with dO^L = lam dO and dO^W = (1 - lam) dO the slot kernels run on (o^L,
// lse^L, dO^L) and the window kernels on (o^W, lse^W, dO^W) -- each branch is
// then an ordinary softmax read -- and dlam_t = <dO_t, o^L_t - o^W_t>.
//
// Kernels:
//   k_mix_out       o = lam o^L + (1 - lam) o^W
//   k_mix_bwd_prep  dO^L, dO^W, D^W_t = <dO^W_t, o^W_t>, dlam
#include "nha_common.h"
#include "nha_internal.h"

namespace nha {

namespace {

// Weighted-fusion workspace: the unified forward's / backward's workspace
// (whichever is larger; the prologue regions sit at the same offsets in
// both), then the two reads, their lse, the scaled incoming gradients and the
// window branch's D_t.
struct MixWs {
  size_t ol, ow, dol, dow;  // [B][T][H][d] dtype
  size_t lsel, lsew, dw;    // [B][H][T] float
  size_t total;
};

MixWs mix_ws_layout(const Shape& s) {
  MixWs L;
  const size_t f = fwd_ws_layout(s).total, b = bwd_ws_bytes(s);
  size_t off = align256(f > b ? f : b);
  const size_t rows = (size_t)s.B * s.T * s.H * s.d * s.esz, stats = (size_t)s.B * s.H * s.T * 4;
  L.ol = off;
  off += align256(rows);
  L.ow = off;
  off += align256(rows);
  L.dol = off;
  off += align256(rows);
  L.dow = off;
  off += align256(rows);
  L.lsel = off;
  off += align256(stats);
  L.lsew = off;
  off += align256(stats);
  L.dw = off;
  off += align256(stats);
  L.total = off;
  return L;
}

// o[r][:] = lam[r] oL[r][:] + (1 - lam[r]) oW[r][:] over nrows rows of d
// (row r = (b T + t) H + h, the index of lam); 8 elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_mix_out(const T* __restrict__ oL, const T* __restrict__ oW,
                                                 const float* __restrict__ lam, T* __restrict__ o, long nrows,
                                                 int d) {
  const long e = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e >= nrows * d) return;
  const float c = lam[e / d];
  float a[8], b[8], y[8];
  ld8f<T>(oL + e, a);
  ld8f<T>(oW + e, b);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = c * a[i] + (1.f - c) * b[i];
  st8<T>(o + e, pack8<T>(y));
}

// Per row r = (b T + t) H + h: dO^L = lam dO, dO^W = (1 - lam) dO (rounded
// to the input dtype, which the branch kernels then read), D^W = <dO^W, o^W>
// from the rounded values ([B][H][T]), dlam = <dO, o^L - o^W> (nullable).
// D/8 threads per row, 8 channels each.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_mix_bwd_prep(const T* __restrict__ dO, const T* __restrict__ oL,
                                                      const T* __restrict__ oW, const float* __restrict__ lam,
                                                      T* __restrict__ dOL, T* __restrict__ dOW,
                                                      float* __restrict__ DW, float* __restrict__ dlam, int Tn,
                                                      int H, long nrows) {
  constexpr int TPR = D / 8;  // 4, 8 or 16: a divisor of the wave
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long r = gid / TPR;
  const int part = (int)(gid % TPR);
  float dw = 0.f, dl = 0.f;
  if (r < nrows) {
    const long e = r * D + part * 8;
    const float c = lam[r];
    float g[8], a[8], b[8], gl[8], gw[8];
    ld8f<T>(dO + e, g);
    ld8f<T>(oL + e, a);
    ld8f<T>(oW + e, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gl[i] = c * g[i];
      gw[i] = (1.f - c) * g[i];
    }
    const typename Vec<T>::v8 pl = pack8<T>(gl), pw = pack8<T>(gw);
    st8<T>(dOL + e, pl);
    st8<T>(dOW + e, pw);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dw += to_f<T>(pw[i]) * b[i];
      dl += g[i] * (a[i] - b[i]);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) {
    dw += __shfl_xor(dw, off, 64);
    dl += __shfl_xor(dl, off, 64);
  }
  if (r < nrows && part == 0) {
    const long h = r % H, bt = r / H, t = bt % Tn, b = bt / Tn;
    DW[(b * H + h) * Tn + t] = dw;
    if (dlam) dlam[r] = dl;
  }
}

template <typename T>
hipError_t mix_out(const Shape& s, const void* oL, const void* oW, const float* lam, void* o, hipStream_t st) {
  const long nrows = (long)s.B * s.T * s.H, n8 = nrows * s.d / 8;
  hipLaunchKernelGGL(k_mix_out<T>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, (const T*)oL, (const T*)oW,
                     lam, (T*)o, nrows, s.d);
  return hipGetLastError();
}

template <typename T, int D>
void mix_prep_d(const Shape& s, const WeightedPtrs& p, const MixWs& L, hipStream_t st) {
  const long nrows = (long)s.B * s.T * s.H;
  hipLaunchKernelGGL((k_mix_bwd_prep<T, D>), dim3((unsigned)((nrows * (D / 8) + 255) / 256)), dim3(256), 0, st,
                     (const T*)p.dO, (const T*)(p.ws + L.ol), (const T*)(p.ws + L.ow), p.lam, (T*)(p.ws + L.dol),
                     (T*)(p.ws + L.dow), (float*)(p.ws + L.dw), p.dlam, s.T, s.H, nrows);
}

template <typename T>
void mix_prep(const Shape& s, const WeightedPtrs& p, const MixWs& L, hipStream_t st) {
  switch (s.d) {
    case 32: return mix_prep_d<T, 32>(s, p, L, st);
    case 64: return mix_prep_d<T, 64>(s, p, L, st);
    case 128: return mix_prep_d<T, 128>(s, p, L, st);
  }
}

// The two reads: slot partial -> (ol, lsel), window read -> (ow, lsew); the
// forward's prologue (gates, state scan, RoPE) lands in the workspace where
// the backward's after-forward path reads it.
hipError_t both_reads(const Shape& s, const RopeTheta& th, const WeightedPtrs& p, void* ol, float* lsel, void* ow,
                      float* lsew, hipStream_t st) {
  FwdPtrs f{p.q, p.k, p.v, p.alpha, ow, lsew, nullptr, p.ws, nullptr};
  f.separate = true;
  f.ol_dst = ol;
  f.lsel_dst = lsel;
  return launch_fwd(s, th, f, st);
}

}  // namespace

size_t weighted_ws_bytes(const Shape& s) { return mix_ws_layout(s).total; }

hipError_t launch_fwd_weighted(const Shape& s, const RopeTheta& th, const WeightedPtrs& p, hipStream_t st) {
  const MixWs L = mix_ws_layout(s);
  const size_t bht = (size_t)s.B * s.H * s.T;
  float* lsel = p.lse2 ? p.lse2 : (float*)(p.ws + L.lsel);
  float* lsew = p.lse2 ? p.lse2 + bht : nullptr;
  hipError_t e = both_reads(s, th, p, p.ws + L.ol, lsel, p.ws + L.ow, lsew, st);
  if (e != hipSuccess) return e;
  return s.dtype == NHA_DTYPE_BF16 ? mix_out<bf16>(s, p.ws + L.ol, p.ws + L.ow, p.lam, p.o, st)
                                   : mix_out<float>(s, p.ws + L.ol, p.ws + L.ow, p.lam, p.o, st);
}

hipError_t launch_bwd_weighted(const Shape& s, const RopeTheta& th, const WeightedPtrs& p, hipStream_t st) {
  const MixWs L = mix_ws_layout(s);
  hipError_t e = both_reads(s, th, p, p.ws + L.ol, (float*)(p.ws + L.lsel), p.ws + L.ow, (float*)(p.ws + L.lsew), st);
  if (e != hipSuccess) return e;
  if (s.dtype == NHA_DTYPE_BF16)
    mix_prep<bf16>(s, p, L, st);
  else
    mix_prep<float>(s, p, L, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the slot kernels on (o^L, lse^L, dO^L), the window kernels on (dO^W,
  // lse^W, D^W); the prologue is already in the workspace
  BwdPtrs b{p.q, p.k, p.v, p.alpha, p.ws + L.ol, p.ws + L.dol, (const float*)(p.ws + L.lsel), p.dq, p.dk, p.dv,
            p.dalpha, p.ws, nullptr, true};
  b.win_dO = p.ws + L.dow;
  b.win_lse = (const float*)(p.ws + L.lsew);
  b.win_D = (const float*)(p.ws + L.dw);
  return launch_bwd(s, th, b, st);
}

}  // namespace nha
