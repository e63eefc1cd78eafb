// nha_slot.h -- device building blocks of the slot (long-term memory) branch,
// shared by the forward and backward kernels.
//
// Per (batch, KV head), with a_t = alpha_t and b_t = 1 - alpha_t for t >= w
// (a_t = 1, b_t = 0 before: nothing is absorbed yet) and key_t the absorbed
// row (k_{t-w}, v_{t-w}: the token shift), the slot state obeys
//     S_t = a_t (.) S_{t-1} + b_t (x) key_t
// -- the K^long_t recurrence of the Paper-Notes page "Native Hybrid Attention
// for Efficient Sequence Modeling", section 关键设计 > 层内混合, with the token
// shift described there.  Inside a chunk starting at t0, with
// G_u = sum_{j=t0..u} log2 a_j (per slot),
//     S_t = 2^{G_t} S_{t0-1} + sum_{u=t0..t} 2^{G_t - G_u} b_u (x) key_u ,
// the cumulative / reverse gate products of the chunkwise form (ibid.,
// Chunkwise 并行计算).  Every factor used is 2^{G_later - G_earlier} <= 1:
// pairs in different 16-row blocks go through a block-boundary reference,
// pairs inside one block through exact running products of a.
#pragma once
#include "nha_common.h"

namespace nha {

// Row pitch (floats) of the fp32 per-chunk slot tiles (log2 cumsum G, source
// weights): odd, so the 16 lanes that read one slot column from 16 different
// rows hit 16 different LDS banks.
template <int MP>
struct SlotPitch {
  static constexpr int PG = MP + 1;
};

// In-place inclusive cumsum over the C rows of an LDS tile g[u * P + i] (fp32)
// for columns i < MP, by NT threads: each thread scans a run of rows of one
// column, then adds the totals of the runs before it.
template <int C, int MP, int P, int NT>
__device__ __forceinline__ void lds_col_cumsum(float* g, int tid) {
  constexpr int PARTS = (NT / MP) < C ? (NT / MP) : C;
  constexpr int RP = C / PARTS;
  const int i = tid % MP, part = tid / MP;
  const bool act = part < PARTS;
  if (act) {
    float acc = 0.f;
#pragma unroll
    for (int u = part * RP; u < (part + 1) * RP; ++u) {
      acc += g[u * P + i];
      g[u * P + i] = acc;
    }
  }
  __syncthreads();
  float off = 0.f;
  if (act)
    for (int pp = 0; pp < part; ++pp) off += g[((pp + 1) * RP - 1) * P + i];
  __syncthreads();
  if (act && part > 0) {
#pragma unroll
    for (int u = part * RP; u < (part + 1) * RP; ++u) g[u * P + i] += off;
  }
  __syncthreads();
}

// A chunk's gates, staged into LDS as la[u][i] = log2 a_u (0 where nothing
// is absorbed: t < w, t >= T or padded slot) and al[u][i] = raw alpha (1
// outside).  load() issues every load of the tile (rows and slots clamped into
// range, so no load is conditional) and stage() consumes them: issuing load()
// before other tiles' loads lets stage() wait for the gates alone.  16-byte
// pieces of the rows when m is a multiple of 8, else one element per load.
template <typename T, int C, int MP, int NT>
struct GateTile {
  static constexpr int PR = MP / 8, NV = C * PR, ITV = (NV + NT - 1) / NT, ITS = (C * MP + NT - 1) / NT;
  typename Vec<T>::v8 xv[ITV];
  T xs[ITS];
  __device__ __forceinline__ void load(const T* __restrict__ alpha, int b, int hg, int t0, int Tn, int Hkv, int m,
                                       int tid) {
    if (m % 8 == 0) {
#pragma unroll
      for (int k = 0; k < ITV; ++k) {
        const int e = tid + k * NT, u = e / PR, i0 = (e % PR) * 8, t = t0 + u;
        xv[k] = ld8<T>(alpha + (((size_t)b * Tn + (t < Tn ? t : Tn - 1)) * Hkv + hg) * m + (i0 < m ? i0 : m - 8));
      }
    } else {
#pragma unroll
      for (int k = 0; k < ITS; ++k) {
        const int e = tid + k * NT, u = e / MP, i = e % MP, t = t0 + u;
        xs[k] = alpha[(((size_t)b * Tn + (t < Tn ? t : Tn - 1)) * Hkv + hg) * m + (i < m ? i : m - 1)];
      }
    }
  }
  template <int PG, int PA>
  __device__ __forceinline__ void stage(float* la, T* al, int t0, int Tn, int m, int w, int tid) const {
    const T one = to_t<T>(1.f);
    if (m % 8 == 0) {
#pragma unroll
      for (int k = 0; k < ITV; ++k) {
        const int e = tid + k * NT, u = e / PR, i0 = (e % PR) * 8, t = t0 + u;
        if (e < NV) {
          const bool real = i0 < m && t < Tn, act = real && t >= w;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const T av = real ? xv[k][j] : one;
            la[u * PG + i0 + j] = act ? fmaxf(__log2f(to_f<T>(av)), NHA_LOG2A_MIN) : 0.f;
            al[u * PA + i0 + j] = av;
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < ITS; ++k) {
        const int e = tid + k * NT, u = e / MP, i = e % MP, t = t0 + u;
        if (e < C * MP) {
          const bool real = i < m && t < Tn;
          const T av = real ? xs[k] : one;
          la[u * PG + i] = (real && t >= w) ? fmaxf(__log2f(to_f<T>(av)), NHA_LOG2A_MIN) : 0.f;
          al[u * PA + i] = av;
        }
      }
    }
  }
};

template <typename T, int C, int MP, int PG, int PA, int NT>
__device__ __forceinline__ void stage_gates(const T* __restrict__ alpha, float* la, T* al, int b, int hg, int t0,
                                            int Tn, int Hkv, int m, int w, int tid) {
  GateTile<T, C, MP, NT> gt;
  gt.load(alpha, b, hg, t0, Tn, Hkv, m, tid);
  gt.template stage<PG, PA>(la, al, t0, Tn, m, w, tid);
}

// ---------------------------------------------------------------- intra-chunk slot products
// The two products every slot kernel needs, for one wave owning chunk rows
// r0 .. r0+15 (I = r0 / 16; lane (g, cc) handles row r0 + cc and slots
// i = 16 mb + 4 g + r).  LDS operands of the chunk:
//   sG[u*PG + i]  log2 cumsum of the effective decay (fp32, PG = MP + 1)
//   sA[u*PM + i]  raw gate (a_u = alpha, b_u = 1 - alpha when t0+u >= w)
//   sB[u*PM + i]  2^{E_J - G_u} b_u,  sBt[i*PC + u] the same (E_J = G at the
//                 last row of u's 16-row block)
// and S_t = 2^{G_t} S0 + sum_{u<=t} 2^{G_t - G_u} b_u (x) key_u.

// Same-block pairs can use the block-end reference too (one more masked MFMA
// instead of per-element running products) when every slot's total decay over
// the block is mild, >= 2^-16: the factors 2^{G_t - E_I}, 2^{E_I - G_u} are
// then within [2^-16, 2^16] and the same-block terms, which dominate the slot
// reads, keep bf16 operand precision relative to their own size.  Stronger
// decays take the exact fp32 running products: there dalpha's
// (A - b F) / alpha form cancels, and the same-block terms must stay fp32.
// Uniform over the wave.
// (Every load is unconditional and the test is a bitwise and: no branch and
// no serialised LDS round trip per slot.)
template <int MP>
__device__ __forceinline__ bool block_factorizable(const float* sG, int r0, float lim = -16.f) {
  constexpr int NB = MP / 16, PG = SlotPitch<MP>::PG;
  const int g = (threadIdx.x & 63) >> 4;
  const float keep = r0 > 0 ? 1.f : 0.f;
  const int rb = r0 > 0 ? r0 - 1 : 0;
  bool ok = true;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * mb + 4 * g + r;
      const float before = keep * sG[rb * PG + i];
      ok &= (sG[(r0 + 15) * PG + i] - before >= lim);
    }
  return __all(ok);
}

// Per-chunk decay factors of the block-referenced form, built once per chunk
// from the log2 cumsum G by build_slot_tab (after G's last barrier; a barrier
// must follow before they are read).  With E_J = G at the last row of 16-row
// block J and E_{-1} = 0 (the chunk start):
//   e[J + 1][i] = E_J
//   f[I][J][i]  = 2^{E_{I-1} - E_J}   (J <= I; <= 1 for J < I; clamped to
//                                      2^64 for J = I, where it is used only
//                                      when the block is factorizable, <= 2^16)
//   z[I][i]     = 2^{E_{I-1}}
// A slot factor 2^{G_t - E_J} of row t in block I is then the lane's
// 2^{G_t - E_{I-1}} (<= 1, computed once) times f[I][J]: one product instead
// of an exponential and two scattered reads per (row, slot, block).
template <int C, int MP>
struct SlotTab {
  static constexpr int NW = C / 16;
  float e[NW + 1][MP];
  float f[NW][NW][MP];
  float z[NW][MP];
};

template <int C, int MP, int NT>
__device__ __forceinline__ void build_slot_tab(SlotTab<C, MP>& tb, const float* sG, int tid) {
  constexpr int NW = C / 16, PG = SlotPitch<MP>::PG;
  for (int x = tid; x < (NW + 1) * MP; x += NT) {
    const int J = x / MP - 1, i = x % MP;
    tb.e[J + 1][i] = J < 0 ? 0.f : sG[(16 * J + 15) * PG + i];
  }
  for (int x = tid; x < NW * NW * MP; x += NT) {
    const int I = x / (NW * MP), J = (x / MP) % NW, i = x % MP;
    const float ep = I > 0 ? sG[(16 * I - 1) * PG + i] : 0.f;
    tb.f[I][J][i] = J <= I ? fast_exp2(fminf(ep - sG[(16 * J + 15) * PG + i], 64.f)) : 0.f;
  }
  for (int x = tid; x < NW * MP; x += NT) {
    const int I = x / MP, i = x % MP;
    tb.z[I][i] = I > 0 ? fast_exp2(sG[(16 * I - 1) * PG + i]) : 1.f;
  }
}

// block_factorizable from the table: E_I - E_{I-1} >= -16 for every slot
template <int C, int MP>
__device__ __forceinline__ bool block_factorizable(const SlotTab<C, MP>& tb, int I) {
  constexpr int NB = MP / 16;
  const int g = (threadIdx.x & 63) >> 4;
  bool ok = true;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(&tb.e[I][16 * mb + 4 * g]);
    const floatx4 b = *reinterpret_cast<const floatx4*>(&tb.e[I + 1][16 * mb + 4 * g]);
#pragma unroll
    for (int r = 0; r < 4; ++r) ok &= (b[r] - a[r] >= -16.f);
  }
  return __all(ok);
}

// out[mb][r] = <x_t, S_t[i]> for the wave's rows.  sS: S0 [i][d] (pitch PD);
// sKey: key rows [u][d] (pitch PD); xf: the rows' vectors as B fragments.
// TR (bf16 only): sBt is the row tile B [u][i] (pitch PM), read transposed
// with ds_read_b64_tr_b16; else the transposed copy [i][u] (pitch PC).
template <typename T, int D, int MP, int C, bool TR = false>
__device__ __forceinline__ void slot_read(const T* sS, const T* sKey, const T* sBt, const float* sG, const T* sA,
                                          const typename Vec<T>::v8* xf, int I, int t0, int w, int Tn,
                                          float (&out)[MP / 16][4], const SlotTab<C, MP>* tb = nullptr) {
  constexpr int NW = C / 16, NB = MP / 16, PD = pitch_of(D), PM = pitch_of(MP), PC = pitch_of(C);
  constexpr int PG = SlotPitch<MP>::PG;
  const int l = threadIdx.x & 63, g = l >> 4, cc = l & 15, r0 = 16 * I, urow = r0 + cc;
  // TR: every factor from the table (out accumulates in units of the lane's
  // F = 2^{G_t - E_{I-1}}, applied at the end); else the exponentials directly
  float F[NB][4];
  if constexpr (TR) {
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      const floatx4 ep = *reinterpret_cast<const floatx4*>(&tb->e[I][16 * mb + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) F[mb][r] = fast_exp2(sG[urow * PG + 16 * mb + 4 * g + r] - ep[r]);
    }
  }
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    floatx4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) acc = mma32(acc, ld8<T>(&sS[(16 * mb + cc) * PD + 32 * ks + 8 * g]), xf[ks]);
    if constexpr (TR) {
      const floatx4 z4 = *reinterpret_cast<const floatx4*>(&tb->z[I][16 * mb + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) out[mb][r] = z4[r] * acc[r];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) out[mb][r] = fast_exp2(sG[urow * PG + 16 * mb + 4 * g + r]) * acc[r];
    }
  }
  // earlier 16-row blocks J < I of the chunk, and (when factorizable) the
  // block itself with the causal mask u <= t; one block per iteration (not
  // unrolled: the blocks are independent and unrolling only multiplies the
  // live registers)
  bool fast;
  if constexpr (TR) fast = block_factorizable<C, MP>(*tb, I);
  else fast = block_factorizable<MP>(sG, r0);
  floatx4 aI = zero4();  // A[u][t] of the wave's own block (exact path)
  auto block = [&](int J) {
    floatx4 av = zero4();  // A[u][t] = key_u . x_t, D layout [u = 16J + 4g + r][t = cc]
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      av = mma32(av, ld8<T>(&sKey[(16 * J + cc) * PD + 32 * ks + 8 * g]), xf[ks]);
    if (J == I) aI = av;
    if (J < I || fast) {
      if (J == I) {
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = (4 * g + r <= cc) ? av[r] : 0.f;
      }
      typename Vec<T>::v4 bfr = pack4<T>(av);
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        typename Vec<T>::v4 bt;
        if constexpr (TR)
          bt = ld_tr4(&sBt[(16 * J + 4 * g + (cc >> 2)) * PM + 16 * mb + 4 * (cc & 3)]);
        else
          bt = ld4<T>(&sBt[(16 * mb + cc) * PC + 16 * J + 4 * g]);
        floatx4 x = mma16(zero4(), bt, bfr);
        if constexpr (TR) {
          const floatx4 f4 = *reinterpret_cast<const floatx4*>(&tb->f[I][J][16 * mb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) out[mb][r] += f4[r] * x[r];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int i = 16 * mb + 4 * g + r;
            out[mb][r] += fast_exp2(sG[urow * PG + i] - sG[(16 * J + 15) * PG + i]) * x[r];
          }
        }
      }
    }
  };
  if constexpr (TR) {
    // (bf16 kernels: registers to spare -- unrolled, so that the blocks'
    // reads and products overlap)
#pragma unroll
    for (int J = 0; J < NW; ++J)
      if (J <= I) block(J);
  } else {
#pragma unroll 1
    for (int J = 0; J <= I; ++J) block(J);
  }
  if constexpr (TR) {
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[mb][r] *= F[mb][r];
  }
  if (fast) return;
  // same block: exact running products
  float Ad[16];
#pragma unroll
  for (int gg = 0; gg < 4; ++gg)
#pragma unroll
    for (int r = 0; r < 4; ++r) Ad[4 * gg + r] = __shfl(aI[r], cc + 16 * gg, 64);
  float Dp[NB][4];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) Dp[mb][r] = 1.f;
#pragma unroll
  for (int uu = 15; uu >= 0; --uu) {
    if (uu <= cc) {
      int u = r0 + uu, t = t0 + u;
      bool absorb = (t >= w) && (t < Tn);
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        typename Vec<T>::v4 al = ld4<T>(&sA[u * PM + 16 * mb + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = to_f<T>(al[r]);
          float be = absorb ? 1.f - a : 0.f;
          out[mb][r] += Ad[uu] * Dp[mb][r] * be;
          Dp[mb][r] *= absorb ? a : 1.f;
        }
      }
    }
  }
}

// accO (O^T[d][t] in D layout) += sum_i wgt_t[i] S_t[i].  sSt: S0 transposed
// [d][i] (pitch PM); sKeyT: key rows transposed [d][u] (pitch PCT).  TR
// (bf16 only): sSt and sKeyT are the row tiles S0 [i][d] and key [u][d]
// (pitch PD), read transposed with ds_read_b64_tr_b16.
template <typename T, int D, int MP, int C, int PCT, bool TR = false>
__device__ __forceinline__ void slot_mix(const T* sSt, const T* sKeyT, const T* sB, const float* sG, const T* sA,
                                         const float (&wgt)[MP / 16][4], int I, int t0, int w, int Tn,
                                         floatx4 (&accO)[D / 16], const SlotTab<C, MP>* tb = nullptr) {
  constexpr int NW = C / 16, NB = MP / 16, PM = pitch_of(MP), PG = SlotPitch<MP>::PG, PD = pitch_of(D);
  const int l = threadIdx.x & 63, g = l >> 4, cc = l & 15, r0 = 16 * I, urow = r0 + cc;
  // TR: wF = wgt * 2^{G_t - E_{I-1}}, the lane's part of every factor (the
  // block parts come from the table)
  float wF[NB][4];
  if constexpr (TR) {
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      const floatx4 ep = *reinterpret_cast<const floatx4*>(&tb->e[I][16 * mb + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        wF[mb][r] = wgt[mb][r] * fast_exp2(sG[urow * PG + 16 * mb + 4 * g + r] - ep[r]);
    }
  }
  {
    float ph[NB][4];
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      if constexpr (TR) {
        const floatx4 z4 = *reinterpret_cast<const floatx4*>(&tb->z[I][16 * mb + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) ph[mb][r] = wF[mb][r] * z4[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) ph[mb][r] = wgt[mb][r] * fast_exp2(sG[urow * PG + 16 * mb + 4 * g + r]);
      }
    }
#pragma unroll
    for (int s = 0; s < NB / 2; ++s) {
      typename Vec<T>::v8 bfr = pack8<T>(floatx4{ph[2 * s][0], ph[2 * s][1], ph[2 * s][2], ph[2 * s][3]},
                                         floatx4{ph[2 * s + 1][0], ph[2 * s + 1][1], ph[2 * s + 1][2],
                                                 ph[2 * s + 1][3]});
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        typename Vec<T>::v8 at;
        if constexpr (TR) {
          const bf16x4 a0 = ld_tr4(&sSt[(32 * s + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
          const bf16x4 a1 = ld_tr4(&sSt[(32 * s + 16 + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            at[e] = a0[e];
            at[4 + e] = a1[e];
          }
        } else {
          at = ld4x2<T>(&sSt[(16 * db + cc) * PM + 32 * s + 4 * g], &sSt[(16 * db + cc) * PM + 32 * s + 16 + 4 * g]);
        }
        accO[db] = mma32(accO[db], at, bfr);
      }
    }
  }
  bool fast;
  if constexpr (TR) fast = block_factorizable<C, MP>(*tb, I);
  else fast = block_factorizable<MP>(sG, r0);
  auto block = [&](int J) {
    if (J < I || fast) {
      floatx4 at = zero4();
#pragma unroll
      for (int s = 0; s < NB / 2; ++s) {
        float f[8];
        if constexpr (TR) {
          const floatx4 fa = *reinterpret_cast<const floatx4*>(&tb->f[I][J][32 * s + 4 * g]);
          const floatx4 fb = *reinterpret_cast<const floatx4*>(&tb->f[I][J][32 * s + 16 + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            f[r] = wF[2 * s][r] * fa[r];
            f[4 + r] = wF[2 * s + 1][r] * fb[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int i0 = 32 * s + 4 * g + r, i1 = i0 + 16;
            f[r] = wgt[2 * s][r] * fast_exp2(sG[urow * PG + i0] - sG[(16 * J + 15) * PG + i0]);
            f[4 + r] = wgt[2 * s + 1][r] * fast_exp2(sG[urow * PG + i1] - sG[(16 * J + 15) * PG + i1]);
          }
        }
        at = mma32(at,
                   ld4x2<T>(&sB[(16 * J + cc) * PM + 32 * s + 4 * g], &sB[(16 * J + cc) * PM + 32 * s + 16 + 4 * g]),
                   pack8<T>(f));
      }
      if (J == I) {
#pragma unroll
        for (int r = 0; r < 4; ++r) at[r] = (4 * g + r <= cc) ? at[r] : 0.f;  // u <= t
      }
      typename Vec<T>::v4 bfr = pack4<T>(at);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        typename Vec<T>::v4 kt;
        if constexpr (TR)
          kt = ld_tr4(&sKeyT[(16 * J + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
        else
          kt = ld4<T>(&sKeyT[(16 * db + cc) * PCT + 16 * J + 4 * g]);
        accO[db] = mma16(accO[db], kt, bfr);
      }
    }
  };
  if constexpr (TR) {
#pragma unroll
    for (int J = 0; J < NW; ++J)
      if (J <= I) block(J);
  } else {
#pragma unroll 1
    for (int J = 0; J <= I; ++J) block(J);
  }
  if (fast) return;
  float Dp[NB][4];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) Dp[mb][r] = 1.f;
  float mine[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int uu = 15; uu >= 0; --uu) {
    float cu = 0.f;
    int u = r0 + uu, t = t0 + u;
    bool absorb = (t >= w) && (t < Tn);
    if (uu <= cc) {
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        typename Vec<T>::v4 al = ld4<T>(&sA[u * PM + 16 * mb + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = to_f<T>(al[r]);
          float be = absorb ? 1.f - a : 0.f;
          cu += wgt[mb][r] * Dp[mb][r] * be;
          Dp[mb][r] *= absorb ? a : 1.f;
        }
      }
    }
    cu = sum_over_g(cu);
    if ((uu >> 2) == g) mine[uu & 3] = cu;
  }
  typename Vec<T>::v4 bfr;
#pragma unroll
  for (int r = 0; r < 4; ++r) bfr[r] = to_t<T>(mine[r]);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    typename Vec<T>::v4 kt;
    if constexpr (TR)
      kt = ld_tr4(&sKeyT[(r0 + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
    else
      kt = ld4<T>(&sKeyT[(16 * db + cc) * PCT + r0 + 4 * g]);
    accO[db] = mma16(accO[db], kt, bfr);
  }
}

}  // namespace nha
