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
//   2. pushes (k_t, v_t) into ring row t mod w;
//   3. reads the m slots (raw q, no RoPE) and the min(w, t+1) window tokens
//      (RoPE'd q and keys) through one softmax scaled by `scale`;
//   4. advances the position.
// One workgroup per (b, KV head) serves all H/Hkv query heads of the group.
#include "nha_common.h"
#include "nha_internal.h"

namespace nha {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_decode(const T* __restrict__ q, const T* __restrict__ kin,
                                                const T* __restrict__ vin, const T* __restrict__ alpha,
                                                float* __restrict__ SK, float* __restrict__ SV,
                                                T* __restrict__ RK, T* __restrict__ RV,
                                                long long* __restrict__ pos, T* __restrict__ o, int H, int Hkv,
                                                int m, int w, float scale, RopeTheta th, int rope) {
  extern __shared__ float dsm[];  // logits [G][m + w]
  __shared__ float qs[4 * D];    // raw q of up to 4 heads per pass
  __shared__ float qrs[4 * D];   // rotated q
  __shared__ float kap[D], nu[D];
  __shared__ float red[2 * 256];
  __shared__ long long tpos;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  if (tid == 0) tpos = pos[unit];
  __syncthreads();
  const long long t = tpos;
  float* sk = SK + (size_t)unit * m * D;
  float* sv = SV + (size_t)unit * m * D;
  T* rk = RK + (size_t)unit * w * D;
  T* rv = RV + (size_t)unit * w * D;
  const T* kt = kin + ((size_t)b * Hkv + hg) * D;
  const T* vt = vin + ((size_t)b * Hkv + hg) * D;
  // 1. absorb
  if (t >= w) {
    for (int j = tid; j < D; j += blockDim.x) {
      if (w > 0) {
        size_t rr = (size_t)(t % w) * D + j;
        kap[j] = to_f<T>(rk[rr]);
        nu[j] = to_f<T>(rv[rr]);
      } else {
        kap[j] = to_f<T>(kt[j]);
        nu[j] = to_f<T>(vt[j]);
      }
    }
    __syncthreads();
    const T* al = alpha + ((size_t)b * Hkv + hg) * m;
    for (int e = tid; e < m * D; e += blockDim.x) {
      int i = e / D, j = e % D;
      float a = to_f<T>(al[i]);
      sk[e] = a * sk[e] + (1.f - a) * kap[j];
      sv[e] = a * sv[e] + (1.f - a) * nu[j];
    }
  }
  __syncthreads();
  // 2. push
  if (w > 0) {
    for (int j = tid; j < D; j += blockDim.x) {
      size_t rr = (size_t)(t % w) * D + j;
      rk[rr] = kt[j];
      rv[rr] = vt[j];
    }
  }
  __syncthreads();
  const long long nwin = (w == 0) ? 0 : (t + 1 < w ? t + 1 : w);
  const int nkeys = m + (int)nwin;
  const long long jfirst = t - nwin + 1;
  const int KG = 256 / D;  // key groups of the value pass
  for (int h0 = 0; h0 < G; h0 += 4) {
    const int nh = (G - h0) < 4 ? (G - h0) : 4;
    // 3a. queries of this pass (raw and rotated by t)
    for (int e = tid; e < nh * D; e += blockDim.x) {
      int hh = e / D, j = e % D;
      const T* qh = q + ((size_t)b * H + hg * G + h0 + hh) * D;
      float x = to_f<T>(qh[j]);
      qs[e] = x;
      float y = x;
      if (rope) {
        int half = D / 2, i = j % half;
        double ang = (double)t * th.theta[i];
        ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        float pair = to_f<T>(qh[j < half ? j + half : j - half]);
        y = (j < half) ? x * cs - pair * sn : x * cs + pair * sn;
      }
      qrs[e] = y;
    }
    __syncthreads();
    // 3b. logits
    for (int e = tid; e < nkeys; e += blockDim.x) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      if (e < m) {
        const float* row = sk + (size_t)e * D;
        for (int j = 0; j < D; ++j) {
          float x = row[j];
#pragma unroll
          for (int hh = 0; hh < 4; ++hh)
            if (hh < nh) acc[hh] += x * qs[hh * D + j];
        }
      } else {
        long long jp = jfirst + (e - m);
        const T* row = rk + (size_t)(jp % w) * D;
        const int half = D / 2;
        for (int i = 0; i < half; ++i) {
          float a = to_f<T>(row[i]), bb = to_f<T>(row[i + half]);
          float ya = a, yb = bb;
          if (rope) {
            double ang = (double)jp * th.theta[i];
            ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
            float sn, cs;
            sincosf((float)ang, &sn, &cs);
            ya = a * cs - bb * sn;
            yb = bb * cs + a * sn;
          }
#pragma unroll
          for (int hh = 0; hh < 4; ++hh)
            if (hh < nh) acc[hh] += ya * qrs[hh * D + i] + yb * qrs[hh * D + i + half];
        }
      }
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
        if (hh < nh) dsm[(size_t)hh * nkeys + e] = acc[hh] * scale;
    }
    __syncthreads();
    // 3c. softmax + values, one head at a time
    for (int hh = 0; hh < nh; ++hh) {
      float* lg = dsm + (size_t)hh * nkeys;
      float mx = -INFINITY;
      for (int e = tid; e < nkeys; e += blockDim.x) mx = fmaxf(mx, lg[e]);
      red[tid] = mx;
      __syncthreads();
      for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
        __syncthreads();
      }
      mx = red[0];
      __syncthreads();
      float zs = 0.f;
      for (int e = tid; e < nkeys; e += blockDim.x) {
        float pv = __expf(lg[e] - mx);
        lg[e] = pv;
        zs += pv;
      }
      red[tid] = zs;
      __syncthreads();
      for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
      }
      zs = red[0];
      __syncthreads();
      const int col = tid % D, kgp = tid / D;
      float acc = 0.f;
      if (kgp < KG) {
        for (int e = kgp; e < nkeys; e += KG) {
          float pv = lg[e];
          float x;
          if (e < m) x = sv[(size_t)e * D + col];
          else x = to_f<T>(rv[(size_t)((jfirst + (e - m)) % w) * D + col]);
          acc += pv * x;
        }
      }
      red[tid] = acc;
      __syncthreads();
      if (tid < D) {
        float s2 = 0.f;
        for (int x = 0; x < KG; ++x) s2 += red[x * D + tid];
        o[((size_t)b * H + hg * G + h0 + hh) * D + tid] = to_t<T>(s2 / zs);
      }
      __syncthreads();
    }
  }
  if (tid == 0) pos[unit] = t + 1;
}

template <typename T, int D>
static hipError_t decode_impl(const Shape& s, const RopeTheta& th, const DecodePtrs& p, hipStream_t st) {
  StateLayout L = state_layout(s);
  char* base = (char*)p.state;
  size_t dyn = (size_t)4 * (s.m + s.w) * 4;
  hipLaunchKernelGGL((k_decode<T, D>), dim3(s.B * s.Hkv), dim3(256), dyn, st, (const T*)p.q, (const T*)p.k,
                     (const T*)p.v, (const T*)p.alpha, (float*)(base + L.sk), (float*)(base + L.sv),
                     (T*)(base + L.rk), (T*)(base + L.rv), (long long*)(base + L.pos), (T*)p.o, s.H, s.Hkv,
                     s.m, s.w, s.scale, th, s.rope ? 1 : 0);
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
