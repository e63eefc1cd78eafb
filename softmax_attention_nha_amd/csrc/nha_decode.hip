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
//      shift (without the token shift, the ablation: k_t itself at every step);
//   2. reads the m slots (raw q, no RoPE) and the min(w, t+1) window tokens
//      (RoPE'd q and keys) through one softmax scaled by `scale`;
//   3. pushes (k_t, v_t) into ring row t mod w and advances the position.
// Two launches.  k_dec_split, grid (NS, B*Hkv): workgroup s takes the keys
// s, s + NS, s + 2 NS, ... of the list [m slots; window tokens], absorbs its
// own slot rows (every slot row has one owner, so the state is updated in
// place without races), and leaves per query head a partial softmax (max,
// sum, unnormalised output) in the state's scratch.  A key is handled by D/8
// lanes, 8 channels each; all rows a lane needs are loaded before their first
// use (two memory round trips: the position, then the ring rows it selects),
// and the D/8 partial dot products of a lane's D/16 keys are summed by a
// halving butterfly (D/16 lane exchanges per head instead of one log2(D/8)
// reduction per key).  k_dec_merge, one workgroup per (batch, KV head):
// merges the NS partials of each head of the group in split order (the
// standard max / sum rescaling), writes o_t, pushes the token into the rings
// -- after every split has read ring row t mod w -- and advances the
// position.  No atomics: o_t is bitwise reproducible.
#include "nha_common.h"
#include "nha_internal.h"

namespace nha {

__device__ __forceinline__ void dec_angle(double theta, long long pos, float& cs, float& sn) {
  double ang = (double)pos * theta;
  ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
  sincosf((float)ang, &sn, &cs);
}

template <typename T>
__device__ __forceinline__ void ld8f_row(const T* p, float (&x)[8]) {
  const typename Vec<T>::v8 v = ld8<T>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = to_f<T>(v[e]);
}

__device__ __forceinline__ void ld8f_f32(const float* p, float (&x)[8]) {
  const floatx4 a0 = *reinterpret_cast<const floatx4*>(p), a1 = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = a0[r];
    x[4 + r] = a1[r];
  }
}

// A gate's value from its bits in a 32-bit register (bf16: zero-extended; a
// bf16 is the upper half of the float it stands for).
template <typename T>
__device__ __forceinline__ float gate_from_bits(uint32_t r) {
  return __uint_as_float(sizeof(T) == 2 ? r << 16 : r);
}

// The new token's ring entries: thread c < D holds channel c of k_t and v_t,
// the rotate-half partner channel of k_t and the channel's RoPE frequency.
// Loaded at kernel entry (they depend on no other load; a per-thread index
// into the argument block is a memory load too) and stored once every read of
// the ring row they replace is done.
template <typename T, int D>
struct RingPush {
  T kx, vx, kp;
  double th;
  __device__ __forceinline__ void load(const T* __restrict__ kin, const T* __restrict__ vin, size_t src,
                                       const RopeTheta& rt, int tid) {
    constexpr int HALF = D / 2;
    const int c = tid < D ? tid : 0;
    kx = kin[src + c];
    vx = vin[src + c];
    kp = kin[src + (c < HALF ? c + HALF : c - HALF)];
    th = rt.theta[c % HALF];
  }
  // thread tid < D; row dst of the rings, position t
  __device__ __forceinline__ void store(T* __restrict__ RK, T* __restrict__ RV, T* __restrict__ RKR, size_t dst,
                                        long long t, int rope, int tid) const {
    constexpr int HALF = D / 2;
    RK[dst + tid] = kx;
    RV[dst + tid] = vx;
    if (rope) {
      const float x = to_f<T>(kx), pair = to_f<T>(kp);
      float cs, sn;
      dec_angle(th, t, cs, sn);
      RKR[dst + tid] = to_t<T>(tid < HALF ? x * cs - pair * sn : x * cs + pair * sn);
    }
  }
};

// Sum over the LPK lanes of one key group (lanes 16-aligned blocks of LPK).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = 1; o < LPK; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Rotate-half RoPE of one lane's 8 channels with precomputed (cos, sin) of
// their angles; the partner channels (i +- D/2) sit in lane li ^ (LPK/2).
template <int D>
__device__ __forceinline__ void dec_rope_cs(float (&x)[8], int li, const float (&cs)[8], const float (&sn)[8]) {
  constexpr int LPK = D / 8, HALF = D / 2;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = __shfl_xor(x[e], LPK / 2, 64);
  const bool first = 8 * li < HALF;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = first ? x[e] * cs[e] - y[e] * sn[e] : x[e] * cs[e] + y[e] * sn[e];
}

constexpr int kDecGH = 4;  // query heads per pass

template <typename T, int D, int KPG>
__global__ __launch_bounds__(256) void k_dec_split(const T* __restrict__ q, const T* __restrict__ kin,
                                                   const T* __restrict__ vin, const T* __restrict__ alpha,
                                                   float* __restrict__ SK, float* __restrict__ SV,
                                                   const T* __restrict__ RK, const T* __restrict__ RV,
                                                   const T* __restrict__ RKR, const long long* __restrict__ pos,
                                                   float* __restrict__ part, int H, int Hkv, int m, int w, int sh,
                                                   int NS, float scale, RopeTheta th, int rope) {
  // KPG keys per group of LPK lanes; a split takes at most KPG * NG keys
  constexpr int LPK = D / 8, NG = 256 / LPK, PP = D + 4, HALF = D / 2, LPR = LPK / KPG;
  static_assert(KPG >= 1 && LPR >= 2 && KPG * NG <= kDecodeKeysPerSplit, "keys per lane group");
  __shared__ float lg[kDecGH][kDecodeKeysPerSplit];  // logits of this split's keys (log2 units)
  __shared__ float red[kDecGH][4];
  __shared__ float wsum[4][kDecGH][D + 1];
  const int tid = threadIdx.x, grp = tid / LPK, li = tid % LPK, wv = tid >> 6;
  const int s = blockIdx.x, unit = blockIdx.y, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  // Every load that does not depend on the position goes out with the
  // position's, raw (converted only after the last of them is issued), so
  // that the step waits on two memory round trips: these, then the ring rows
  // the position selects.
  const long long t = pos[unit];
  // this lane's RoPE frequencies (a per-lane index into the argument block
  // is a memory load)
  double thv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) thv[e] = th.theta[(8 * li + e) % HALF];
  // the first head group's query rows
  typename Vec<T>::v8 q0[kDecGH];
#pragma unroll
  for (int hh = 0; hh < kDecGH; ++hh)
    q0[hh] = ld8<T>(q + ((size_t)b * H + hg * G + (hh < G ? hh : 0)) * D + 8 * li);
  // the new token, and this group's slot rows and their gates (slot e = key
  // index e < m; address clamped)
  const size_t krow = ((size_t)b * Hkv + hg) * D + 8 * li;  // this lane's channels of k_t / v_t
  const typename Vec<T>::v8 knew8 = ld8<T>(kin + krow), vnew8 = ld8<T>(vin + krow);
  float* sk = SK + (size_t)unit * m * D + 8 * li;
  float* sv = SV + (size_t)unit * m * D + 8 * li;
  // through buffer resources over the unit's slot rows and gates: no branch
  // on m (a branch would place each gate's conversion, and a wait for its
  // load, before the next row's loads); with m = 0 the resources are empty
  // and the loads read zeros without touching memory
  const __amdgpu_buffer_rsrc_t rsk = buf_rsrc(SK + (size_t)unit * m * D, (uint32_t)(m * D * 4));
  const __amdgpu_buffer_rsrc_t rsv = buf_rsrc(SV + (size_t)unit * m * D, (uint32_t)(m * D * 4));
  const __amdgpu_buffer_rsrc_t rga = buf_rsrc(alpha + ((size_t)b * Hkv + hg) * m, (uint32_t)(m * sizeof(T)));
  float xk[KPG][8], xv[KPG][8], ga[KPG];
  uint32_t gar[KPG];  // raw gate bits
#pragma unroll
  for (int kk = 0; kk < KPG; ++kk) {
    const int e = max(min(s + NS * (grp + NG * kk), m - 1), 0);
    const uint32_t off = (uint32_t)(e * D + 8 * li) * 4u;
    const floatx8 rk8 = buf_ld16(rsk, off, (floatx8*)nullptr), rv8 = buf_ld16(rsv, off, (floatx8*)nullptr);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      xk[kk][r] = rk8[r];
      xv[kk][r] = rv8[r];
    }
    gar[kk] = sizeof(T) == 2 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rga, (uint32_t)e * 2u, 0, 0)
                             : __builtin_amdgcn_raw_buffer_load_b32(rga, (uint32_t)e * 4u, 0, 0);
  }
  const long long nwin = (w == 0) ? 0 : (t + 1 < w ? t + 1 : w);
  const int nkeys = m + (int)nwin;
  const long long jfirst = t - nwin + 1;
  const int nmine = nkeys > s ? (nkeys - s + NS - 1) / NS : 0;  // keys of this split
  // the token absorbed at this step: the one leaving the window (ring row
  // t mod w), or k_t itself when w = 0 or without token shift (sh = 0); and
  // this group's window rows (RoPE'd keys when RoPE is on)
  float kap[8], nu[8];
  typename Vec<T>::v8 wk[KPG], wvr[KPG];  // raw rows, converted when selected
  if (w > 0) {
    const T* rk = RK + (size_t)unit * w * D + 8 * li;
    const T* rv = RV + (size_t)unit * w * D + 8 * li;
    const T* rkw = (rope ? RKR : RK) + (size_t)unit * w * D + 8 * li;
    const size_t ra = (size_t)(t % w) * D;
    ld8f_row<T>(rk + ra, kap);
    ld8f_row<T>(rv + ra, nu);
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      const int e = s + NS * (grp + NG * kk);
      // window position jfirst + e - m, clamped into the ring's valid rows
      long long jp = jfirst + (e - m);
      jp = jp < jfirst ? jfirst : (jp > t ? t : jp);
      const size_t rr = (size_t)(jp % w) * D;
      wk[kk] = ld8<T>(rkw + rr);
      wvr[kk] = ld8<T>(rv + rr);
    }
  }
  float knew[8], vnew[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    knew[r] = to_f<T>(knew8[r]);
    vnew[r] = to_f<T>(vnew8[r]);
  }
#pragma unroll
  for (int kk = 0; kk < KPG; ++kk) ga[kk] = gate_from_bits<T>(gar[kk]);
  if (sh == 0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      kap[r] = knew[r];
      nu[r] = vnew[r];
    }
  }
  // this lane's RoPE factors at position t (a channel and its partner share
  // the angle)
  float cs[8], sn[8];
  if (rope) {
#pragma unroll
    for (int e = 0; e < 8; ++e) dec_angle(thv[e], t, cs[e], sn[e]);
  }
  float knr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) knr[r] = knew[r];
  if (rope) dec_rope_cs<D>(knr, li, cs, sn);
  // 1. absorb this group's slot rows and select every key's K and V rows
  bool isslot[KPG];
#pragma unroll
  for (int kk = 0; kk < KPG; ++kk) {
    const int j = grp + NG * kk, e = s + NS * j;
    isslot[kk] = e < m;
    if (j < nmine && e < m) {
      if (t >= sh) {
        const float a = ga[kk];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          xk[kk][r] = a * xk[kk][r] + (1.f - a) * kap[r];
          xv[kk][r] = a * xv[kk][r] + (1.f - a) * nu[r];
        }
        float* rk_ = sk + (size_t)e * D;
        float* rv_ = sv + (size_t)e * D;
        *reinterpret_cast<floatx4*>(rk_) = floatx4{xk[kk][0], xk[kk][1], xk[kk][2], xk[kk][3]};
        *reinterpret_cast<floatx4*>(rk_ + 4) = floatx4{xk[kk][4], xk[kk][5], xk[kk][6], xk[kk][7]};
        *reinterpret_cast<floatx4*>(rv_) = floatx4{xv[kk][0], xv[kk][1], xv[kk][2], xv[kk][3]};
        *reinterpret_cast<floatx4*>(rv_ + 4) = floatx4{xv[kk][4], xv[kk][5], xv[kk][6], xv[kk][7]};
      }
    } else if (jfirst + (e - m) == t) {  // the new token
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        xk[kk][r] = knr[r];
        xv[kk][r] = vnew[r];
      }
    } else if (w > 0) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        xk[kk][r] = to_f<T>(wk[kk][r]);
        xv[kk][r] = to_f<T>(wvr[kk][r]);
      }
    }
  }
  const float sl2 = scale * NHA_LOG2E;
  for (int h0 = 0; h0 < G; h0 += kDecGH) {
    const int nh = (G - h0) < kDecGH ? (G - h0) : kDecGH;
    float qs[kDecGH][8], qr[kDecGH][8];
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
      const int h = hg * G + h0 + (hh < nh ? hh : 0);
      if (h0 == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[hh][e] = to_f<T>(q0[hh][e]);
      } else {
        ld8f_row<T>(q + ((size_t)b * H + h) * D + 8 * li, qs[hh]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[hh][e] = qs[hh][e];
      if (rope && hh < nh) dec_rope_cs<D>(qr[hh], li, cs, sn);
    }
    // 2a. logits (log2 units) of this group's keys: lane li ends up with the
    // full dot product of key li / LPR of its group
    const int kmine = li / LPR, jmine = grp + NG * kmine;
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
      if (hh < nh) {
        float P[KPG];
#pragma unroll
        for (int kk = 0; kk < KPG; ++kk) {
          float acc = 0.f;
#pragma unroll
          for (int r = 0; r < 8; ++r) acc += xk[kk][r] * (isslot[kk] ? qs[hh][r] : qr[hh][r]);
          P[kk] = acc;
        }
        // halving butterfly: at lane bit msk = LPK/2, LPK/4, .., LPR the lane
        // keeps the upper half of its keys if that bit is set, the lower half
        // otherwise, adding its partner's part of the kept half; the lane bits
        // below LPR then sum the one key left
#pragma unroll
        for (int lvl = 0; (KPG >> lvl) > 1; ++lvl) {
          const int n = KPG >> lvl, msk = LPK >> (lvl + 1);
          const bool up = (li & msk) != 0;
#pragma unroll
          for (int i = 0; i < n / 2; ++i) {
            const float snd = up ? P[i] : P[i + n / 2];
            const float rcv = __shfl_xor(snd, msk, 64);
            P[i] = (up ? P[i + n / 2] : P[i]) + rcv;
          }
        }
#pragma unroll
        for (int msk = LPR / 2; msk >= 1; msk >>= 1) P[0] += __shfl_xor(P[0], msk, 64);
        if (li % LPR == 0 && jmine < nmine) lg[hh][jmine] = P[0] * sl2;
      }
    }
    __syncthreads();
    // 2b. max per head over this split's keys
    for (int hh = 0; hh < nh; ++hh) {
      float mx = -INFINITY;
      for (int j = tid; j < nmine; j += 256) mx = fmaxf(mx, lg[hh][j]);
#pragma unroll
      for (int o2 = 1; o2 < 64; o2 <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
      if ((tid & 63) == 0) red[hh][wv] = mx;
    }
    __syncthreads();
    float mxh[kDecGH];
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
      mxh[hh] = -INFINITY;
      if (hh < nh)
        for (int x = 0; x < 4; ++x) mxh[hh] = fmaxf(mxh[hh], red[hh][x]);
    }
    // 2c. p = 2^(l - max) and the unnormalised output of this group's keys
    float oa[kDecGH][8];
    float zs[kDecGH];
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
      zs[hh] = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) oa[hh][r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      const int j = grp + NG * kk;
      if (j < nmine) {
#pragma unroll
        for (int hh = 0; hh < kDecGH; ++hh) {
          if (hh < nh) {
            const float p = fast_exp2(lg[hh][j] - mxh[hh]);
            zs[hh] += p;
#pragma unroll
            for (int r = 0; r < 8; ++r) oa[hh][r] += p * xv[kk][r];
          }
        }
      }
    }
    // reduce over the key groups: within the wave by shuffles (groups of the
    // same channels are LPK lanes apart), then across the 4 waves in LDS
#pragma unroll
    for (int hh = 0; hh < kDecGH; ++hh) {
      if (hh >= nh) continue;
#pragma unroll
      for (int o2 = LPK; o2 < 64; o2 <<= 1) {
        zs[hh] += __shfl_xor(zs[hh], o2, 64);
#pragma unroll
        for (int r = 0; r < 8; ++r) oa[hh][r] += __shfl_xor(oa[hh][r], o2, 64);
      }
    }
    // lanes 0 .. LPK-1 of each wave hold the wave's sums for channels 8 li ..
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
      if (c < D)
        dst[4 + c] = v;
      else {
        dst[0] = mxh[hh];
        dst[1] = v;
      }
    }
    __syncthreads();
  }
}

// One workgroup (256 threads) per (batch, KV head): merge the partials of
// each query head of the group, write o_t, push the token into the rings and
// advance the position.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_dec_merge(const float* __restrict__ part, const T* __restrict__ kin,
                                                   const T* __restrict__ vin, T* __restrict__ RK, T* __restrict__ RV,
                                                   T* __restrict__ RKR, long long* __restrict__ pos,
                                                   T* __restrict__ o, int H, int Hkv, int w, int NS, RopeTheta th,
                                                   int rope) {
  constexpr int PP = D + 4, HALF = D / 2, SG = 256 / D, PER = (kDecodeSplitMax + SG - 1) / SG;
  __shared__ float fs[kDecodeSplitMax];  // per-split factors 2^(max_s - M)
  __shared__ float acc_s[SG * D];
  __shared__ float zred[SG];
  const int tid = threadIdx.x, unit = blockIdx.x, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  const long long t = pos[unit];
  // thread (sp, c) sums channel c over the splits sp, sp + SG, ...: every
  // load first (addresses clamped), then the sums in split order
  const int c = tid % D, sp = tid / D;
  float xo[PER], xz[PER], mx;
  auto load_head = [&](int hh) {
    const float* pr = part + ((size_t)(b * H + hg * G + hh)) * kDecodeSplitMax * PP;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int sx = min(sp + SG * i, NS - 1);
      xo[i] = pr[sx * PP + 4 + c];
      xz[i] = pr[sx * PP + 1];
    }
    mx = pr[min(tid & 63, NS - 1) * PP];
  };
  load_head(0);
  // the ring push's rows after the first head's partials: both in flight
  // together, neither waiting on the other
  RingPush<T, D> rp;
  rp.load(kin, vin, ((size_t)b * Hkv + hg) * D, th, tid);
  for (int hh = 0; hh < G; ++hh) {
    if (hh > 0) load_head(hh);
    if (tid < 64) {
      if (tid >= NS) mx = -INFINITY;
      float M = mx;
#pragma unroll
      for (int o2 = 1; o2 < 64; o2 <<= 1) M = fmaxf(M, __shfl_xor(M, o2, 64));
      if (tid < NS) fs[tid] = fast_exp2(mx - M);
    }
    __syncthreads();
    float acc = 0.f, z = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int sx = sp + SG * i;
      if (sx < NS) {
        acc += fs[sx] * xo[i];
        z += fs[sx] * xz[i];
      }
    }
    // then the SG split groups in a fixed order through LDS
    acc_s[sp * D + c] = acc;
    if (c == 0) zred[sp] = z;
    __syncthreads();
    if (tid < D) {
      float a2 = 0.f, z2 = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < SG; ++g2) {
        a2 += acc_s[g2 * D + tid];
        z2 += zred[g2];
      }
      o[((size_t)b * H + hg * G + hh) * D + tid] = to_t<T>(a2 / z2);
    }
    __syncthreads();
  }
  // push (k_t, v_t) into ring row t mod w (and the key with RoPE at t)
  if (w > 0 && tid < D) rp.store(RK, RV, RKR, ((size_t)unit * w + (size_t)(t % w)) * D, t, rope, tid);
  if (tid == 0) pos[unit] = t + 1;
}

// Single-launch step for many units (B * Hkv at least the compute-unit
// count: one workgroup per unit already fills the chip).  The workgroup walks
// the key list [m slots; window tokens] in passes of KPN keys (the split
// kernel's key-group layout, contiguous keys per pass), keeps each head's
// softmax as a running (max, sum, unnormalised output) in LDS, rescaled when a
// pass raises the maximum, and then writes o_t, pushes the token into the
// rings and advances the position -- after a barrier behind the last read of
// ring row t mod w.  Heads of the group go kDecGH at a time; the slot rows are
// absorbed (in place, each by its one owner lane group) in the first head
// pass only, later head passes read them back.
template <typename T, int D, int KPG, int GH>
__global__ __launch_bounds__(256) void k_dec_fused(const T* __restrict__ q, const T* __restrict__ kin,
                                                   const T* __restrict__ vin, const T* __restrict__ alpha,
                                                   float* __restrict__ SK, float* __restrict__ SV, T* __restrict__ RK,
                                                   T* __restrict__ RV, T* __restrict__ RKR, long long* __restrict__ pos,
                                                   T* __restrict__ o, int H, int Hkv, int m, int w, int sh,
                                                   float scale, RopeTheta th, int rope) {
  constexpr int LPK = D / 8, NG = 256 / LPK, HALF = D / 2, LPR = LPK / KPG, KPN = KPG * NG;
  static_assert(KPG >= 1 && LPR >= 2, "keys per lane group");
  __shared__ float lg[GH][KPN];  // logits of this pass's keys (log2 units)
  __shared__ float red[GH][4];
  __shared__ float wsum[4][GH][D + 1];
  __shared__ float run_o[GH][D];  // running unnormalised output of each head of the pass
  __shared__ float run_m[GH], run_z[GH];
  const int tid = threadIdx.x, grp = tid / LPK, li = tid % LPK, wv = tid >> 6;
  const int unit = blockIdx.x, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  double thv[8];  // this lane's RoPE frequencies, loaded first (as in k_dec_split)
#pragma unroll
  for (int e = 0; e < 8; ++e) thv[e] = th.theta[(8 * li + e) % HALF];
  RingPush<T, D> rp;
  rp.load(kin, vin, ((size_t)b * Hkv + hg) * D, th, tid);
  const size_t krow = ((size_t)b * Hkv + hg) * D + 8 * li;
  float knew[8], vnew[8];
  ld8f_row<T>(kin + krow, knew);
  ld8f_row<T>(vin + krow, vnew);
  float* sk = SK + (size_t)unit * m * D + 8 * li;
  float* sv = SV + (size_t)unit * m * D + 8 * li;
  const long long t = pos[unit];
  const long long nwin = (w == 0) ? 0 : (t + 1 < w ? t + 1 : w);
  const int nkeys = m + (int)nwin;
  const long long jfirst = t - nwin + 1;
  const int npass = (nkeys + KPN - 1) / KPN;
  // the token absorbed at this step (ring row t mod w, or k_t itself)
  float kap[8], nu[8];
  const T* rkw = (rope ? RKR : RK) + (size_t)unit * w * D + 8 * li;
  const T* rvw = RV + (size_t)unit * w * D + 8 * li;
  if (w > 0) {
    const size_t ra = (size_t)(t % w) * D;
    ld8f_row<T>(RK + (size_t)unit * w * D + 8 * li + ra, kap);
    ld8f_row<T>(rvw + ra, nu);
  }
  if (sh == 0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      kap[r] = knew[r];
      nu[r] = vnew[r];
    }
  }
  float cs[8], sn[8];
  if (rope) {
#pragma unroll
    for (int e = 0; e < 8; ++e) dec_angle(thv[e], t, cs[e], sn[e]);
  }
  float knr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) knr[r] = knew[r];
  if (rope) dec_rope_cs<D>(knr, li, cs, sn);
  const float sl2 = scale * NHA_LOG2E;
  for (int h0 = 0; h0 < G; h0 += GH) {
    const int nh = (G - h0) < GH ? (G - h0) : GH;
    float qs[GH][8], qr[GH][8];
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      const int h = hg * G + h0 + (hh < nh ? hh : 0);
      ld8f_row<T>(q + ((size_t)b * H + h) * D + 8 * li, qs[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[hh][e] = qs[hh][e];
      if (rope && hh < nh) dec_rope_cs<D>(qr[hh], li, cs, sn);
    }
    for (int e = tid; e < GH * D; e += 256) run_o[e / D][e % D] = 0.f;
    if (tid < GH) {
      run_m[tid] = -INFINITY;
      run_z[tid] = 0.f;
    }
    // the window rows of a pass go out one pass ahead (raw, converted when
    // the pass starts), so each pass waits on no load of its own
    typename Vec<T>::v8 pk[KPG], pv[KPG];
    auto fetch = [&](int pass) {
#pragma unroll
      for (int kk = 0; kk < KPG; ++kk) {
        long long jp = jfirst + (pass * KPN + grp + NG * kk - m);  // window position, clamped to the valid rows
        jp = jp < jfirst ? jfirst : (jp > t ? t : jp);
        if (w > 0) {
          const size_t rr = (size_t)(jp % w) * D;
          pk[kk] = ld8<T>(rkw + rr);
          pv[kk] = ld8<T>(rvw + rr);
        }
      }
    };
    fetch(0);
    for (int pass = 0; pass < npass; ++pass) {
      const int ebase = pass * KPN, nmine = min(KPN, nkeys - ebase);
      // this group's keys: slot rows (absorbed here in the first head pass)
      // or window rows
      float xk[KPG][8], xv[KPG][8];
      bool isslot[KPG];
#pragma unroll
      for (int kk = 0; kk < KPG; ++kk) {
        const int j = grp + NG * kk, e = ebase + j;
        isslot[kk] = e < m;
        if (e < m) {
          ld8f_f32(sk + (size_t)e * D, xk[kk]);
          ld8f_f32(sv + (size_t)e * D, xv[kk]);
          if (h0 == 0 && j < nmine && t >= sh) {
            const float a = to_f<T>(alpha[((size_t)b * Hkv + hg) * m + e]);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              xk[kk][r] = a * xk[kk][r] + (1.f - a) * kap[r];
              xv[kk][r] = a * xv[kk][r] + (1.f - a) * nu[r];
            }
            float* rk_ = sk + (size_t)e * D;
            float* rv_ = sv + (size_t)e * D;
            *reinterpret_cast<floatx4*>(rk_) = floatx4{xk[kk][0], xk[kk][1], xk[kk][2], xk[kk][3]};
            *reinterpret_cast<floatx4*>(rk_ + 4) = floatx4{xk[kk][4], xk[kk][5], xk[kk][6], xk[kk][7]};
            *reinterpret_cast<floatx4*>(rv_) = floatx4{xv[kk][0], xv[kk][1], xv[kk][2], xv[kk][3]};
            *reinterpret_cast<floatx4*>(rv_ + 4) = floatx4{xv[kk][4], xv[kk][5], xv[kk][6], xv[kk][7]};
          }
        } else if (jfirst + (e - m) == t) {  // the new token
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            xk[kk][r] = knr[r];
            xv[kk][r] = vnew[r];
          }
        } else if (w > 0) {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            xk[kk][r] = to_f<T>(pk[kk][r]);
            xv[kk][r] = to_f<T>(pv[kk][r]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 8; ++r) xk[kk][r] = xv[kk][r] = 0.f;
        }
      }
      if (pass + 1 < npass) fetch(pass + 1);
      // logits: lane li ends with the full dot product of key li / LPR of its group
      const int kmine = li / LPR, jmine = grp + NG * kmine;
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        if (hh < nh) {
          float P[KPG];
#pragma unroll
          for (int kk = 0; kk < KPG; ++kk) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) acc += xk[kk][r] * (isslot[kk] ? qs[hh][r] : qr[hh][r]);
            P[kk] = acc;
          }
#pragma unroll
          for (int lvl = 0; (KPG >> lvl) > 1; ++lvl) {
            const int n = KPG >> lvl, msk = LPK >> (lvl + 1);
            const bool up = (li & msk) != 0;
#pragma unroll
            for (int i = 0; i < n / 2; ++i) {
              const float snd = up ? P[i] : P[i + n / 2];
              const float rcv = __shfl_xor(snd, msk, 64);
              P[i] = (up ? P[i + n / 2] : P[i]) + rcv;
            }
          }
#pragma unroll
          for (int msk = LPR / 2; msk >= 1; msk >>= 1) P[0] += __shfl_xor(P[0], msk, 64);
          if (li % LPR == 0 && jmine < nmine) lg[hh][jmine] = P[0] * sl2;
        }
      }
      __syncthreads();
      for (int hh = 0; hh < nh; ++hh) {
        float mx = -INFINITY;
        for (int j = tid; j < nmine; j += 256) mx = fmaxf(mx, lg[hh][j]);
#pragma unroll
        for (int o2 = 1; o2 < 64; o2 <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
        if ((tid & 63) == 0) red[hh][wv] = mx;
      }
      __syncthreads();
      // the pass's maximum joins the running one
      float mnew[GH], fold[GH];
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        float mp = -INFINITY;
        if (hh < nh)
          for (int x = 0; x < 4; ++x) mp = fmaxf(mp, red[hh][x]);
        const float mr = hh < nh ? run_m[hh] : 0.f;
        mnew[hh] = fmaxf(mr, mp);
        fold[hh] = hh < nh ? fast_exp2(mr - mnew[hh]) : 0.f;  // 0 on the first pass (mr = -inf)
      }
      float oa[GH][8], zs[GH];
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        zs[hh] = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) oa[hh][r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < KPG; ++kk) {
        const int j = grp + NG * kk;
        if (j < nmine) {
#pragma unroll
          for (int hh = 0; hh < GH; ++hh) {
            if (hh < nh) {
              const float p = fast_exp2(lg[hh][j] - mnew[hh]);
              zs[hh] += p;
#pragma unroll
              for (int r = 0; r < 8; ++r) oa[hh][r] += p * xv[kk][r];
            }
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        if (hh >= nh) continue;
#pragma unroll
        for (int o2 = LPK; o2 < 64; o2 <<= 1) {
          zs[hh] += __shfl_xor(zs[hh], o2, 64);
#pragma unroll
          for (int r = 0; r < 8; ++r) oa[hh][r] += __shfl_xor(oa[hh][r], o2, 64);
        }
      }
      if ((tid & 63) < LPK) {
#pragma unroll
        for (int hh = 0; hh < GH; ++hh) {
#pragma unroll
          for (int r = 0; r < 8; ++r) wsum[wv][hh][8 * li + r] = oa[hh][r];
          if (li == 0) wsum[wv][hh][D] = zs[hh];
        }
      }
      __syncthreads();
      // running state <- fold * running + this pass (each element by one thread)
      for (int e = tid; e < nh * (D + 1); e += 256) {
        const int hh = e / (D + 1), c = e % (D + 1);
        const float v = wsum[0][hh][c] + wsum[1][hh][c] + wsum[2][hh][c] + wsum[3][hh][c];
        if (c < D)
          run_o[hh][c] = run_o[hh][c] * fold[hh] + v;
        else
          run_z[hh] = run_z[hh] * fold[hh] + v;
      }
      __syncthreads();
      if (tid < nh) run_m[tid] = mnew[tid];
      __syncthreads();
    }
    for (int e = tid; e < nh * D; e += 256) {
      const int hh = e / D, c = e % D;
      o[((size_t)b * H + hg * G + h0 + hh) * D + c] = to_t<T>(run_o[hh][c] / run_z[hh]);
    }
    __syncthreads();
  }
  // every read of ring row t mod w is behind the barriers above: push (k_t,
  // v_t) there (and the key with RoPE at t) and advance the position
  if (w > 0 && tid < D) rp.store(RK, RV, RKR, ((size_t)unit * w + (size_t)(t % w)) * D, t, rope, tid);
  if (tid == 0) pos[unit] = t + 1;
}

template <typename T, int D>
static hipError_t decode_impl(const Shape& s, const RopeTheta& th, const DecodePtrs& p, hipStream_t st) {
  StateLayout L = state_layout(s);
  char* base = (char*)p.state;
  const int units = s.B * s.Hkv;
  if (units >= device_cu_count()) {
    // one workgroup per unit fills the chip: one launch, no partials
    // one query head per KV head: one head per pass, twice the keys per
    // lane group; else four heads per pass
    auto fused = s.G == 1 ? k_dec_fused<T, D, D / 32 < 1 ? 1 : D / 32, 1> : k_dec_fused<T, D, D / 32 < 1 ? 1 : D / 32, kDecGH>;
    hipLaunchKernelGGL(fused, dim3(units), dim3(256), 0, st, (const T*)p.q, (const T*)p.k, (const T*)p.v,
                       (const T*)p.alpha, (float*)(base + L.sk), (float*)(base + L.sv), (T*)(base + L.rk),
                       (T*)(base + L.rv), (T*)(base + L.rkr), (long long*)(base + L.pos), (T*)p.o, s.H, s.Hkv, s.m,
                       s.w, s.sh, s.scale, th, s.rope ? 1 : 0);
    return hipGetLastError();
  }
  const DecodeSplit sp = decode_splits(s);
  const int NS = sp.ns;
  // half-size key groups (fewer registers, more workgroups per CU) whenever
  // the keys fit them
  auto split = sp.small ? k_dec_split<T, D, D / 32 < 1 ? 1 : D / 32> : k_dec_split<T, D, D / 16>;
  hipLaunchKernelGGL(split, dim3(NS, units), dim3(256), 0, st, (const T*)p.q, (const T*)p.k, (const T*)p.v,
                     (const T*)p.alpha, (float*)(base + L.sk), (float*)(base + L.sv), (const T*)(base + L.rk),
                     (const T*)(base + L.rv), (const T*)(base + L.rkr), (const long long*)(base + L.pos),
                     (float*)(base + L.part), s.H, s.Hkv, s.m, s.w, s.sh, NS, s.scale, th, s.rope ? 1 : 0);
  hipLaunchKernelGGL((k_dec_merge<T, D>), dim3(units), dim3(256), 0, st, (const float*)(base + L.part),
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
