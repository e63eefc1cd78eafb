// nha_decode.hip -- one recurrent ("RNN mode") inference step of the NHA layer.
//
// The Paper-Notes page "Native Hybrid Attention for Efficient Sequence
// Modeling" (section 局限与展望) notes that the chunk kernel serves training and
// that recurrent-mode inference is a separate path; the ai.info page ("Why This
// Matters") describes switching one model into that RNN mode at inference.
// At position t (read from the state, per (batch, KV head)) one step:
//   1. if t >= w: absorbs the token leaving the window, k_{t-w} (ring row
//      t mod w; the current k_t when w = 0), with gate alpha_t:
//        S <- Diag(alpha_t) S + (1 - alpha_t) (x) k_{t-w}   (same for V)
//      -- the K^long_t recurrence of section 关键设计 > 层内混合 with its token
//      shift;
//   2. reads the m slots (raw q, no RoPE) and the min(w, t+1) window tokens
//      (RoPE'd q and keys) through one softmax scaled by `scale`;
//   3. pushes (k_t, v_t) into ring row t mod w and advances the position.
// Two launches.  k_dec_split: grid (NS, B*Hkv); workgroup s takes the keys
// s, s + NS, s + 2 NS, ... of the list [m slots; window tokens], absorbs its
// own slot rows (every slot row has one owner, so the state is updated in
// place without races), and leaves per query head a partial softmax (max,
// sum, unnormalised output) in the state's scratch.  k_dec_combine: one
// workgroup per (batch, KV head) merges the NS partials of each head of the
// group (the standard max / sum rescaling), then pushes the token into the
// rings -- after every split has read ring row t mod w -- and advances the
// position.  A key is handled by D/8 lanes, 8 channels each.
#include "nha_common.h"
#include "nha_internal.h"

namespace nha {

__device__ __forceinline__ void dec_angle(double theta, long long pos, float& cs, float& sn) {
  double ang = (double)pos * theta;
  ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
  sincosf((float)ang, &sn, &cs);
}

// Rotate-half RoPE of one lane's 8 channels x[0..7] = row[8 li .. 8 li + 7]
// at position `pos`: the partner channels (i +- D/2) sit in lane li ^ (LPK/2)
// of the same key group.
template <int D>
__device__ __forceinline__ void dec_rope(float (&x)[8], int li, long long pos, const RopeTheta& th) {
  constexpr int LPK = D / 8, HALF = D / 2;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = __shfl_xor(x[e], LPK / 2, 64);
  const bool first = 8 * li < HALF;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int ch = 8 * li + e, i = ch % HALF;
    float cs, sn;
    dec_angle(th.theta[i], pos, cs, sn);
    x[e] = first ? x[e] * cs - y[e] * sn : x[e] * cs + y[e] * sn;
  }
}

template <typename T>
__device__ __forceinline__ void ld8f_row(const T* p, float (&x)[8]) {
  const typename Vec<T>::v8 v = ld8<T>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = to_f<T>(v[e]);
}

// Sum over the LPK lanes of one key group (lanes 16-aligned blocks of LPK).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = 1; o < LPK; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

constexpr int kDecGH = 4;  // query heads per pass

template <typename T, int D>
__global__ __launch_bounds__(256) void k_dec_split(const T* __restrict__ q, const T* __restrict__ kin,
                                                   const T* __restrict__ vin, const T* __restrict__ alpha,
                                                   float* __restrict__ SK, float* __restrict__ SV,
                                                   const T* __restrict__ RK, const T* __restrict__ RV,
                                                   const T* __restrict__ RKR, const long long* __restrict__ pos,
                                                   float* __restrict__ part, int H, int Hkv, int m, int w,
                                                   int NS, float scale, RopeTheta th, int rope) {
  constexpr int LPK = D / 8, NG = 256 / LPK, PP = D + 4;
  __shared__ float lg[kDecGH][kDecodeKeysPerSplit];  // logits of this split's keys (log2 units)
  __shared__ float red[kDecGH][4];
  const int tid = threadIdx.x, grp = tid / LPK, li = tid % LPK;
  const int s = blockIdx.x, unit = blockIdx.y, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  const long long t = pos[unit];
  const long long nwin = (w == 0) ? 0 : (t + 1 < w ? t + 1 : w);
  const int nkeys = m + (int)nwin;
  const long long jfirst = t - nwin + 1;
  const int nmine = nkeys > s ? (nkeys - s + NS - 1) / NS : 0;  // keys of this split
  float* sk = SK + (size_t)unit * m * D;
  float* sv = SV + (size_t)unit * m * D;
  // 1. absorb this split's slot rows (slot i = key index i < m)
  if (t >= w) {
    float kap[8], nu[8];
    if (w > 0) {
      const size_t rr = (size_t)(t % w) * D + 8 * li;
      ld8f_row<T>(RK + (size_t)unit * w * D + rr, kap);
      ld8f_row<T>(RV + (size_t)unit * w * D + rr, nu);
    } else {
      ld8f_row<T>(kin + ((size_t)b * Hkv + hg) * D + 8 * li, kap);
      ld8f_row<T>(vin + ((size_t)b * Hkv + hg) * D + 8 * li, nu);
    }
    const T* al = alpha + ((size_t)b * Hkv + hg) * m;
    for (int j = grp; j < nmine; j += NG) {
      const int e = s + NS * j;
      if (e >= m) break;
      const float a = to_f<T>(al[e]);
      float* rk_ = sk + (size_t)e * D + 8 * li;
      float* rv_ = sv + (size_t)e * D + 8 * li;
      floatx4 k0 = *reinterpret_cast<const floatx4*>(rk_), k1 = *reinterpret_cast<const floatx4*>(rk_ + 4);
      floatx4 v0 = *reinterpret_cast<const floatx4*>(rv_), v1 = *reinterpret_cast<const floatx4*>(rv_ + 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        k0[r] = a * k0[r] + (1.f - a) * kap[r];
        k1[r] = a * k1[r] + (1.f - a) * kap[4 + r];
        v0[r] = a * v0[r] + (1.f - a) * nu[r];
        v1[r] = a * v1[r] + (1.f - a) * nu[4 + r];
      }
      *reinterpret_cast<floatx4*>(rk_) = k0;
      *reinterpret_cast<floatx4*>(rk_ + 4) = k1;
      *reinterpret_cast<floatx4*>(rv_) = v0;
      *reinterpret_cast<floatx4*>(rv_ + 4) = v1;
    }
  }
  // the new token's key (position t), RoPE'd, for the split that owns it
  float knew[8];
  ld8f_row<T>(kin + ((size_t)b * Hkv + hg) * D + 8 * li, knew);
  if (rope) dec_rope<D>(knew, li, t, th);
  const float sl2 = scale * NHA_LOG2E;
  for (int h0 = 0; h0 < G; h0 += kDecGH) {
    const int nh = (G - h0) < kDecGH ? (G - h0) : kDecGH;
    float qs[kDecGH][8], qr[kDecGH][8];
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
      const int h = hg * G + h0 + (hh < nh ? hh : 0);
      ld8f_row<T>(q + ((size_t)b * H + h) * D + 8 * li, qs[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[hh][e] = qs[hh][e];
      if (rope) dec_rope<D>(qr[hh], li, t, th);
    }
    // 2a. logits (log2 units) of this split's keys
    for (int j = grp; j < nmine; j += NG) {
      const int e = s + NS * j;
      float x[8];
      bool slot = e < m;
      if (slot) {
        const float* row = sk + (size_t)e * D + 8 * li;
        const floatx4 a0 = *reinterpret_cast<const floatx4*>(row), a1 = *reinterpret_cast<const floatx4*>(row + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = a0[r];
          x[4 + r] = a1[r];
        }
      } else {
        const long long jp = jfirst + (e - m);
        if (jp == t) {
#pragma unroll
          for (int r = 0; r < 8; ++r) x[r] = knew[r];
        } else {
          const T* ring = (rope ? RKR : RK) + ((size_t)unit * w + (size_t)(jp % w)) * D + 8 * li;
          ld8f_row<T>(ring, x);
        }
      }
#pragma unroll
      for (int hh = 0; hh < kDecGH; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) acc += x[r] * (slot ? qs[hh][r] : qr[hh][r]);
        acc = group_sum<LPK>(acc);
        if (li == 0 && hh < nh) lg[hh][j] = acc * sl2;
      }
    }
    __syncthreads();
    // 2b. max and sum per head over this split's keys
    for (int hh = 0; hh < nh; ++hh) {
      float mx = -INFINITY;
      for (int j = tid; j < nmine; j += 256) mx = fmaxf(mx, lg[hh][j]);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      if ((tid & 63) == 0) red[hh][tid >> 6] = mx;
    }
    __syncthreads();
    float mxh[kDecGH];
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
      mxh[hh] = -INFINITY;
      if (hh < nh)
        for (int x = 0; x < 4; ++x) mxh[hh] = fmaxf(mxh[hh], red[hh][x]);
    }
    __syncthreads();
    // 2c. p = 2^(l - max) and the unnormalised output of this split
    float oa[kDecGH][8];
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh)
#pragma unroll
      for (int r = 0; r < 8; ++r) oa[hh][r] = 0.f;
    float zs[kDecGH] = {0.f, 0.f, 0.f, 0.f};
    for (int j = grp; j < nmine; j += NG) {
      const int e = s + NS * j;
      float x[8];
      if (e < m) {
        const float* row = sv + (size_t)e * D + 8 * li;
        const floatx4 a0 = *reinterpret_cast<const floatx4*>(row), a1 = *reinterpret_cast<const floatx4*>(row + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = a0[r];
          x[4 + r] = a1[r];
        }
      } else {
        const long long jp = jfirst + (e - m);
        if (jp == t)
          ld8f_row<T>(vin + ((size_t)b * Hkv + hg) * D + 8 * li, x);
        else
          ld8f_row<T>(RV + ((size_t)unit * w + (size_t)(jp % w)) * D + 8 * li, x);
      }
#pragma unroll
      for (int hh = 0; hh < kDecGH; ++hh) {
        if (hh < nh) {
          const float p = fast_exp2(lg[hh][j] - mxh[hh]);
          zs[hh] += p;
#pragma unroll
          for (int r = 0; r < 8; ++r) oa[hh][r] += p * x[r];
        }
      }
    }
    // reduce over the key groups: within the wave by shuffles (groups of the
    // same channels are LPK lanes apart), then across the 4 waves in LDS
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) {
        zs[hh] += __shfl_xor(zs[hh], o, 64);
#pragma unroll
        for (int r = 0; r < 8; ++r) oa[hh][r] += __shfl_xor(oa[hh][r], o, 64);
      }
    }
    const int wv = tid >> 6;
    // lanes 0 .. LPK-1 of each wave hold the wave's sums for channels 8 li ..
    __shared__ float wsum[4][kDecGH][D + 1];
    if ((tid & 63) < LPK) {
#pragma unroll
      for (int hh = 0; hh < kDecGH; ++hh) {
#pragma unroll
        for (int r = 0; r < 8; ++r) wsum[wv][hh][8 * li + r] = oa[hh][r];
        if (li == 0) wsum[wv][hh][D] = zs[hh];
      }
    }
    __syncthreads();
    for (int e = tid; e < nh * (D + 1); e += 256) {
      const int hh = e / (D + 1), c = e % (D + 1);
      const float v = wsum[0][hh][c] + wsum[1][hh][c] + wsum[2][hh][c] + wsum[3][hh][c];
      float* dst = part + (((size_t)(b * H + hg * G + h0 + hh)) * kDecodeSplitMax + s) * PP;
      if (c < D) dst[4 + c] = v;
      else {
        dst[0] = mxh[hh];
        dst[1] = v;
      }
    }
    __syncthreads();
  }
}

// One workgroup (D threads) per (batch, KV head): merge the partials of each
// query head of the group, write o_t, push the token into the rings and
// advance the position.
template <typename T, int D>
__global__ __launch_bounds__(128) void k_dec_combine(const float* __restrict__ part, const T* __restrict__ kin,
                                                     const T* __restrict__ vin, T* __restrict__ RK,
                                                     T* __restrict__ RV, T* __restrict__ RKR,
                                                     long long* __restrict__ pos, T* __restrict__ o, int H,
                                                     int Hkv, int w, int NS, RopeTheta th, int rope) {
  constexpr int PP = D + 4;
  const int c = threadIdx.x, unit = blockIdx.x, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  const long long t = pos[unit];
  if (c < D) {
    for (int hh = 0; hh < G; ++hh) {
      const float* pr = part + ((size_t)(b * H + hg * G + hh)) * kDecodeSplitMax * PP;
      float M = -INFINITY;
      for (int s = 0; s < NS; ++s) M = fmaxf(M, pr[s * PP]);
      float z = 0.f, acc = 0.f;
      for (int s = 0; s < NS; ++s) {
        const float f = fast_exp2(pr[s * PP] - M);
        z += f * pr[s * PP + 1];
        acc += f * pr[s * PP + 4 + c];
      }
      o[((size_t)b * H + hg * G + hh) * D + c] = to_t<T>(acc / z);
    }
    if (w > 0) {
      const size_t src = ((size_t)b * Hkv + hg) * D, dst = ((size_t)unit * w + (size_t)(t % w)) * D;
      const float x = to_f<T>(kin[src + c]);
      RK[dst + c] = kin[src + c];
      RV[dst + c] = vin[src + c];
      if (rope) {
        constexpr int HALF = D / 2;
        const int i = c % HALF;
        const float pair = to_f<T>(kin[src + (c < HALF ? c + HALF : c - HALF)]);
        float cs, sn;
        dec_angle(th.theta[i], t, cs, sn);
        RKR[dst + c] = to_t<T>(c < HALF ? x * cs - pair * sn : x * cs + pair * sn);
      }
    }
  }
  __syncthreads();
  if (c == 0) pos[unit] = t + 1;
}

template <typename T, int D>
static hipError_t decode_impl(const Shape& s, const RopeTheta& th, const DecodePtrs& p, hipStream_t st) {
  StateLayout L = state_layout(s);
  char* base = (char*)p.state;
  const int NS = decode_splits(s), units = s.B * s.Hkv;
  hipLaunchKernelGGL((k_dec_split<T, D>), dim3(NS, units), dim3(256), 0, st, (const T*)p.q, (const T*)p.k,
                     (const T*)p.v, (const T*)p.alpha, (float*)(base + L.sk), (float*)(base + L.sv),
                     (const T*)(base + L.rk), (const T*)(base + L.rv), (const T*)(base + L.rkr),
                     (const long long*)(base + L.pos), (float*)(base + L.part), s.H, s.Hkv, s.m, s.w, NS, s.scale,
                     th, s.rope ? 1 : 0);
  hipLaunchKernelGGL((k_dec_combine<T, D>), dim3(units), dim3(128), 0, st, (const float*)(base + L.part),
                     (const T*)p.k, (const T*)p.v, (T*)(base + L.rk), (T*)(base + L.rv), (T*)(base + L.rkr),
                     (long long*)(base + L.pos), (T*)p.o, s.H, s.Hkv, s.w, NS, th, s.rope ? 1 : 0);
  return hipGetLastError();
}

template <typename T>
static hipError_t decode_d(const Shape& s, const RopeTheta& th, const DecodePtrs& p, hipStream_t st) {
  switch (s.d) {
    case 32: return decode_impl<T, 32>(s, th, p, st);
    case 64: return decode_impl<T, 64>(s, th, p, st);
    case 128: return decode_impl<T, 128>(s, th, p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const Shape& s, const RopeTheta& th, const DecodePtrs& p, hipStream_t st) {
  if (s.dtype == NHA_DTYPE_BF16) return decode_d<bf16>(s, th, p, st);
  return decode_d<float>(s, th, p, st);
}

}  // namespace nha
