// nha_fwd.hip -- forward kernels of the NHA layer operator (gfx950).
//
// The forward follows the chunkwise-parallel form described on the
// Paper-Notes page "Native Hybrid Attention for Efficient Sequence Modeling",
// section 关键设计 > Chunkwise 并行计算 (and the ai.info page, "Methodology in
// Plain English"): the sequence is cut into chunks of C tokens; inside a chunk
// the linear-channel (slot) logits come from cumulative / reverse gate
// products, the window logits are ordinary shifted-window attention, both
// enter one softmax, and the two value aggregations are summed.  Here the two
// branches meet through the standard merge of two partial softmaxes (the slot
// branch is handed to the window branch as one "super key" with logit lse_L
// and value o_L / Z_L), which is exact: inside one chunk kernel (bf16, C = 64,
// when the state scan has enough waves to fill the chip), or in a window
// kernel and a slot kernel that merges the window partial.
//
// Per (batch b, KV head g), with a_t = alpha_t and b_t = 1 - alpha_t for
// t >= w (a_t = 1, b_t = 0 before: nothing is absorbed yet), kappa_t = k_{t-w},
// nu_t = v_{t-w} (token shift), the slot state obeys
//     S_t = a_t (.) S_{t-1} + b_t (x) kappa_t .
// Within chunk [t0, t0 + C) let G_u = sum_{j=t0..u} log2 a_j (per slot).  Then
//     S_t = 2^{G_t} S_{t0-1} + sum_{u=t0..t} 2^{G_t - G_u} b_u (x) kappa_u .
// Every exponent used below is of the form G_later - G_earlier <= 0, so no
// factor exceeds 1:  the chunk is cut into 16-row blocks J, and a source row u
// of block J is referred to E_J = G at the last row of J:
//     2^{G_t - G_u} = 2^{G_t - E_J} * 2^{E_J - G_u}   (t beyond J, u in J),
// while pairs inside one block use exact running products of a.
//
// Kernels, in launch order:
//   k_rope          q, k -> R_t q, R_t k (rotate-half RoPE, fp64 angle reduction)
//   k_chunk_gates   per chunk: W^T[i][u] = 2^{G_end - G_u} b_u and 2^{G_end}
//   k_state_scan    sequential over chunks: S at every chunk start (MFMA)
//   k_chunk_fwd_b16 both branches of a 128-query tile: the slot partial of
//                   its two chunks, then the window band seeded with it (MFMA)
// or, in place of the chunk kernel,
//   k_win_fwd       band-masked window attention from an empty softmax
//                   (beside the gate products and the scan, on the side stream)
//   k_slot_fwd      slot logits and their partial, merged with the window's (MFMA)
//   k_export_state  ring buffer + position of the decode state (optional)
#include "nha_common.h"
#include "nha_internal.h"
#include "nha_slot.h"

namespace nha {

// ---------------------------------------------------------------- RoPE
// cs[t][i] = (cos, sin)((pos0 + t) theta_i) for t < T, i < d/2; the angle is
// reduced modulo 2 pi in double precision before the single-precision sincos.
__global__ __launch_bounds__(256) void k_rope_cs(float2* __restrict__ cs, int Tn, int half, RopeTheta th) {
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long)Tn * half) return;
  const int t = (int)(e / half), i = (int)(e % half);
  double ang = (double)(th.pos0 + t) * th.theta[i];
  ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
  float sn, cn;
  sincosf((float)ang, &sn, &cn);
  cs[e] = make_float2(cn, sn);
}

// y[r] = R_pos x[r] for the nq rows of q ([B][T][Hq][d]) followed by the nk
// rows of k ([B][T][Hk][d]); pos = (r / heads) % T.  One thread rotates 8
// frequency pairs (i, i + d/2) with the angles of the cs table.
template <typename T>
__global__ __launch_bounds__(256) void k_rope(const T* __restrict__ q, const T* __restrict__ k, T* __restrict__ qo,
                                              T* __restrict__ ko, long nq, long nk, int Hq, int Hk, int Tn, int d,
                                              const float2* __restrict__ cs) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = d / 16;
  long r = gid / per;
  if (r >= nq + nk) return;
  const bool isq = r < nq;
  if (!isq) r -= nq;
  const int heads = isq ? Hq : Hk;
  const int i0 = (int)(gid % per) * 8;
  const int pos = (int)((r / heads) % Tn);
  const T* xr = (isq ? q : k) + r * d;
  T* yr = (isq ? qo : ko) + r * d;
  const float2* c = cs + (size_t)pos * (d / 2) + i0;
  float a[8], b[8], ya[8], yb[8];
  ld8f<T>(xr + i0, a);
  ld8f<T>(xr + i0 + d / 2, b);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 t = c[e];
    ya[e] = a[e] * t.x - b[e] * t.y;
    yb[e] = b[e] * t.x + a[e] * t.y;
  }
  st8<T>(yr + i0, pack8<T>(ya));
  st8<T>(yr + i0 + d / 2, pack8<T>(yb));
}

// ---------------------------------------------------------------- gate prep
// grid (NC, B*Hkv), 256 threads.
// Wt[unit][c][i][u] = 2^{G_end,i - G_u,i} b_u,i   (0 for padded slots / rows)
// aend[unit][c][i]  = 2^{G_end,i}
// Thread (part, i) holds rows part*RP .. part*RP + RP-1 of slot i in
// registers: it sums their log2 gates in row order, the parts' totals meet
// in LDS, and each part adds the totals of the parts before it in part order
// -- the same float additions, in the same order, as the LDS column cumsum
// of the slot kernels -- so its slot row of W^T is RP contiguous elements.
template <typename T, int C, int MP>
__global__ __launch_bounds__(256) void k_chunk_gates(const T* __restrict__ alpha, T* __restrict__ Wt,
                                                     float* __restrict__ aend, int Tn, int Hkv, int m, int w,
                                                     int NC) {
  constexpr int NT = 256, PARTS = (NT / MP) < C ? (NT / MP) : C, RP = C / PARTS;
  static_assert(RP * PARTS == C && (RP == 2 || RP % 4 == 0), "row split");
  __shared__ float tot[PARTS][MP];
  const int tid = threadIdx.x, c = blockIdx.x, unit = blockIdx.y;
  const int b = unit / Hkv, hg = unit % Hkv, t0 = c * C, i = tid % MP, part = tid / MP;
  const bool act = part < PARTS;
  float av[RP], G[RP];
  if (act) {
#pragma unroll
    for (int k = 0; k < RP; ++k) {  // every load first (rows and slots clamped into range)
      const int t = t0 + part * RP + k;
      av[k] = to_f<T>(alpha[(((size_t)b * Tn + (t < Tn ? t : Tn - 1)) * Hkv + hg) * m + (i < m ? i : m - 1)]);
    }
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int t = t0 + part * RP + k;
      const bool act_t = i < m && t < Tn && t >= w;
      acc += act_t ? fmaxf(__log2f(av[k]), NHA_LOG2A_MIN) : 0.f;
      G[k] = acc;
      av[k] = act_t ? 1.f - av[k] : 0.f;  // b_u from here on
    }
    tot[part][i] = acc;
  }
  __syncthreads();
  if (!act) return;
  float off = 0.f, ge = 0.f;
#pragma unroll
  for (int pp = 0; pp < PARTS - 1; ++pp) {
    if (pp < part) off += tot[pp][i];
    ge += tot[pp][i];
  }
  ge = tot[PARTS - 1][i] + ge;  // G_end: the last part's rows plus the parts before it
  T y[RP];
#pragma unroll
  for (int k = 0; k < RP; ++k) y[k] = to_t<T>(fast_exp2(ge - (part > 0 ? G[k] + off : G[k])) * av[k]);
  T* dst = Wt + (((size_t)unit * NC + c) * MP + i) * C + part * RP;
  if constexpr (RP % 8 == 0) {
#pragma unroll
    for (int k = 0; k < RP; k += 8) {
      typename Vec<T>::v8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = y[k + e];
      st8<T>(dst + k, v);
    }
  } else if constexpr (RP % 4 == 0) {
#pragma unroll
    for (int k = 0; k < RP; k += 4) {
      typename Vec<T>::v4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = y[k + e];
      st4<T>(dst + k, v);
    }
  } else {
#pragma unroll
    for (int k = 0; k < RP; ++k) dst[k] = y[k];
  }
  if (part == 0) aend[((size_t)unit * NC + c) * MP + i] = fast_exp2(ge);
}

// ---------------------------------------------------------------- state scan
// grid (d/16, B*Hkv), one wave.  Lane (g, c) keeps S^T[j0 + 4g + r][16 nb + c]
// for K and V.  For every chunk: store S (the state before the chunk; both
// halves in [i][d] layout), then S <- aend (.) S + W^T . kappa  (transposed:
// dS^T = kappa^T W).  The next chunk's rows, weights and decays are loaded
// while the current chunk's products run.
template <typename T, int C, int MP>
struct ScanRegs {
  static constexpr int NB = MP / 16;
  static constexpr bool K16 = (C % 32) != 0;
  static constexpr int KS = K16 ? C / 16 : C / 32;
  typename Vec<T>::v8 k0, k1, v0, v1;                                // kappa / nu row l, cols j0..j0+15
  typename std::conditional<K16, typename Vec<T>::v4, typename Vec<T>::v8>::type wf[NB][KS];
  float ae[NB];
};

template <typename T, int C, int MP>
__device__ __forceinline__ void scan_load(ScanRegs<T, C, MP>& R, const T* __restrict__ kk, const T* __restrict__ vv,
                                          const T* __restrict__ Wt, const float* __restrict__ aend, int c, int unit,
                                          int b, int hg, int j0, int Tn, int Hkv, int d, int w, int NC, int l) {
  constexpr int NB = ScanRegs<T, C, MP>::NB, KS = ScanRegs<T, C, MP>::KS;
  const int g = l >> 4, cc = l & 15;
  R.k0 = R.k1 = R.v0 = R.v1 = zero8<T>();
  int t = c * C + l;
  if (l < C && t >= w && t < Tn) {
    size_t row = (((size_t)b * Tn + (t - w)) * Hkv + hg) * d + j0;
    R.k0 = ld8<T>(kk + row);
    R.k1 = ld8<T>(kk + row + 8);
    R.v0 = ld8<T>(vv + row);
    R.v1 = ld8<T>(vv + row + 8);
  }
  const T* wsrc = Wt + ((size_t)unit * NC + c) * MP * C;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    R.ae[nb] = aend[((size_t)unit * NC + c) * MP + 16 * nb + cc];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (ScanRegs<T, C, MP>::K16)
        R.wf[nb][s] = ld4<T>(wsrc + (size_t)(16 * nb + cc) * C + 16 * s + 4 * g);
      else
        R.wf[nb][s] = ld8<T>(wsrc + (size_t)(16 * nb + cc) * C + 32 * s + 8 * g);
    }
  }
}

template <typename T, int C, int MP>
__global__ __launch_bounds__(64) void k_state_scan(const T* __restrict__ kk, const T* __restrict__ vv,
                                                   const T* __restrict__ Wt, const float* __restrict__ aend,
                                                   T* __restrict__ sst, float* __restrict__ skout,
                                                   float* __restrict__ svout, const float* __restrict__ s0k,
                                                   const float* __restrict__ s0v, int Tn, int Hkv, int d, int m,
                                                   int w, int NC) {
  using R_t = ScanRegs<T, C, MP>;
  constexpr int NB = R_t::NB, KS = R_t::KS;
  constexpr int PC = pitch_of(C);
  __shared__ T sKt[16 * PC];
  __shared__ T sVt[16 * PC];
  const int l = threadIdx.x, g = l >> 4, cc = l & 15;
  // the d/16 column blocks of one unit share W^T: keep them on one XCD's L2
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int j0 = (L % gridDim.x) * 16, unit = L / gridDim.x;
  const int b = unit / Hkv, hg = unit % Hkv;
  floatx4 SK[NB], SV[NB];
  init_slot_state<NB>(SK, SV, s0k, s0v, unit, m, d, j0, g, cc);
  const size_t chunk_elems = 2 * (size_t)MP * d;
  R_t cur, nxt;
  scan_load<T, C, MP>(cur, kk, vv, Wt, aend, 0, unit, b, hg, j0, Tn, Hkv, d, w, NC, l);
  for (int c = 0; c < NC; ++c) {
    // state at the chunk start, [i][d] layout for both halves
    T* dst = sst + ((size_t)unit * NC + c) * chunk_elems;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int i = 16 * nb + cc;
      st4<T>(dst + (size_t)i * d + j0 + 4 * g, pack4<T>(SK[nb]));
      st4<T>(dst + (size_t)MP * d + (size_t)i * d + j0 + 4 * g, pack4<T>(SV[nb]));
    }
    if (l < C) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sKt[e * PC + l] = cur.k0[e];
        sKt[(8 + e) * PC + l] = cur.k1[e];
        sVt[e * PC + l] = cur.v0[e];
        sVt[(8 + e) * PC + l] = cur.v1[e];
      }
    }
    __syncthreads();
    if (c + 1 < NC) scan_load<T, C, MP>(nxt, kk, vv, Wt, aend, c + 1, unit, b, hg, j0, Tn, Hkv, d, w, NC, l);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      SK[nb] *= cur.ae[nb];
      SV[nb] *= cur.ae[nb];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (R_t::K16) {
        typename Vec<T>::v4 ak = ld4<T>(&sKt[cc * PC + 16 * s + 4 * g]);
        typename Vec<T>::v4 av = ld4<T>(&sVt[cc * PC + 16 * s + 4 * g]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          SK[nb] = mma16(SK[nb], ak, cur.wf[nb][s]);
          SV[nb] = mma16(SV[nb], av, cur.wf[nb][s]);
        }
      } else {
        typename Vec<T>::v8 ak = ld8<T>(&sKt[cc * PC + 32 * s + 8 * g]);
        typename Vec<T>::v8 av = ld8<T>(&sVt[cc * PC + 32 * s + 8 * g]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          SK[nb] = mma32(SK[nb], ak, cur.wf[nb][s]);
          SV[nb] = mma32(SV[nb], av, cur.wf[nb][s]);
        }
      }
    }
    __syncthreads();
    cur = nxt;
  }
  if (skout) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int i = 16 * nb + cc;
      if (i < m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          skout[((size_t)unit * m + i) * d + j0 + 4 * g + r] = SK[nb][r];
          svout[((size_t)unit * m + i) * d + j0 + 4 * g + r] = SV[nb][r];
        }
      }
    }
  }
}

// bf16 variant: the chunk operands of the wave's 16 columns (kappa and nu
// rows, W^T, aend) stream into an LDS ring NS chunks ahead with direct-to-LDS
// loads, so that a step only waits for loads issued NS - 1 steps earlier.
// Every step issues the same number of vector-memory operations (the state
// stores, then the loads of chunk c + NS, clamped to the last chunk past the
// end), and vector-memory operations complete in issue order, so one counter
// wait covers exactly the loads of the current chunk.
template <int C, int MP>
struct ScanStage {
  static constexpr int KB = C * 32;           // kappa / nu rows: [u][16 columns]
  static constexpr int WB = MP * C * 2;       // W^T [i][u], 16-byte chunks XOR-swizzled by i
  static constexpr int NK = (KB + 1023) / 1024, NWI = WB / 1024;
  static constexpr int OPS = 2 * NK + NWI + 1;  // direct loads per chunk (+1: aend)
  bf16 k[C * 16];
  bf16 v[C * 16];
  bf16 wt[MP * C];
  float ae[64];
};

// Segments: blockIdx.y = unit * nseg + p walks chunks [p segc, (p+1) segc)
// from the state s0 of row (unit * nseg + p) (null: zero) and leaves its end
// state in row (unit * nseg + p) of skout / svout (null: not kept) and, from
// the workgroup of columns 0-15, the segment's decay, the product of
// 2^{G_end} over its chunks, in row (unit * nseg + p) of dec [.][MP] (null:
// not kept); STORE writes the state at every chunk start.  One segment
// (nseg = 1, segc = NC) is the whole walk.
template <int C, int MP, int NS, bool STORE>
__global__ __launch_bounds__(64) void k_state_scan_b16(const bf16* __restrict__ kk, const bf16* __restrict__ vv,
                                                       const bf16* __restrict__ Wt, const float* __restrict__ aend,
                                                       bf16* __restrict__ sst, float* __restrict__ skout,
                                                       float* __restrict__ svout, float* __restrict__ dec,
                                                       const float* __restrict__ s0k, const float* __restrict__ s0v,
                                                       int Tn, int Hkv, int d, int m, int w, int NC, int nseg,
                                                       int segc) {
  using St = ScanStage<C, MP>;
  constexpr int NB = MP / 16, CPR = C / 8;  // W^T 16-byte chunks per row
  __shared__ St ring[NS];
  const int l = threadIdx.x, g = l >> 4, cc = l & 15;
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int j0 = __builtin_amdgcn_readfirstlane((L % gridDim.x) * 16),
            useg = __builtin_amdgcn_readfirstlane(L / gridDim.x);
  const int unit = useg / nseg, c0 = (useg % nseg) * segc, c1 = min(NC, c0 + segc);
  const int b = unit / Hkv, hg = unit % Hkv;
  const size_t ld = (size_t)Hkv * d;
  const bf16* kbase = kk + ((size_t)b * Tn * Hkv + hg) * d + j0;
  const bf16* vbase = vv + ((size_t)b * Tn * Hkv + hg) * d + j0;
  // issue the direct loads of chunk c (clamped to the segment) into ring slot s
  auto issue = [&](int c, int s) {
    c = min(c, c1 - 1);
    const uint32_t base = lds_addr(&ring[s]);
#pragma unroll
    for (int i = 0; i < St::NK; ++i) {
      // 32 rows per instruction, two 16-byte halves per row; absorbed row
      // t - w of chunk row u (rows outside [0, T) are clamped: their weight is 0)
      const int e = i * 64 + l, u = e >> 1;
      const int tr = min(max(c * C + u - w, 0), Tn - 1);
      const uint32_t off = (uint32_t)((size_t)tr * ld * 2 + 16 * (e & 1));
      const bool act = e * 16 < St::KB;
      const uint32_t mk = __builtin_amdgcn_readfirstlane(base + (uint32_t)offsetof(St, k) + i * 1024);
      const uint32_t mv = __builtin_amdgcn_readfirstlane(base + (uint32_t)offsetof(St, v) + i * 1024);
      if (act) {  // (C = 16: half a wave; still one instruction each)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(mk), "v"(off), "s"(sgpr_ptr(kbase))
                     : "memory", "m0");
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(mv), "v"(off), "s"(sgpr_ptr(vbase))
                     : "memory", "m0");
      }
    }
    const bf16* wsrc = Wt + ((size_t)unit * NC + c) * MP * C;
#pragma unroll
    for (int i = 0; i < St::NWI; ++i) {
      const int e = i * 64 + l, r = e / CPR, p = e % CPR;
      const uint32_t off = (uint32_t)(16 * (r * CPR + (p ^ (r & (CPR - 1)))));
      const uint32_t mw = __builtin_amdgcn_readfirstlane(base + (uint32_t)offsetof(St, wt) + i * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(mw), "v"(off), "s"(sgpr_ptr(wsrc))
                   : "memory", "m0");
    }
    {
      const uint32_t off = (uint32_t)(4 * min(l, MP - 1));
      const uint32_t ma = __builtin_amdgcn_readfirstlane(base + (uint32_t)offsetof(St, ae));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                   :
                   : "s"(ma), "v"(off), "s"(sgpr_ptr(aend + ((size_t)unit * NC + c) * MP))
                   : "memory", "m0");
    }
  };
  floatx4 SK[NB], SV[NB];
  init_slot_state<NB>(SK, SV, s0k, s0v, useg, m, d, j0, g, cc);
  float dk[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dk[nb] = 1.f;
  const size_t chunk_elems = 2 * (size_t)MP * d;
  for (int s = 0; s < NS; ++s) issue(c0 + s, s);
  for (int c = c0; c < c1; ++c) {
    const int s = (c - c0) % NS;
    // loads of chunk c done: the later chunks' loads (St::OPS each) and the
    // state stores of the steps since (2 NB each) may still be in flight
    vm_wait_steps<NS, St::OPS, STORE ? 2 * NB : 0>(c - c0);
    const St& R = ring[s];
    if constexpr (STORE) {
      // state at the chunk start, both halves in column blocks [d/16][i][16]:
      // this wave's block is one contiguous 2 KB piece of each half
      bf16* dst = sst + ((size_t)unit * NC + c) * chunk_elems + (size_t)j0 * MP;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int i = 16 * nb + cc;
        st4<bf16>(dst + i * 16 + 4 * g, pack4<bf16>(SK[nb]));
        st4<bf16>(dst + (size_t)MP * d + i * 16 + 4 * g, pack4<bf16>(SV[nb]));
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float a = R.ae[16 * nb + cc];
      SK[nb] *= a;
      SV[nb] *= a;
      if constexpr (!STORE) dk[nb] *= a;
    }
    // dS^T[col][i] += sum_u kappa^T[col][u] W^T[i][u]: A = kappa^T (transposed
    // reads of the row-major tile), B = W^T rows
    if constexpr (C % 32 != 0) {
      // C = 16: one K=16 step
      const bf16x4 ak = ld_tr4(R.k + (4 * g + (cc >> 2)) * 16 + 4 * (cc & 3));
      const bf16x4 av = ld_tr4(R.v + (4 * g + (cc >> 2)) * 16 + 4 * (cc & 3));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int i = 16 * nb + cc;
        const bf16x4 wf = *reinterpret_cast<const bf16x4*>(R.wt + i * C + 8 * ((g >> 1) ^ (i & (CPR - 1))) +
                                                           4 * (g & 1));
        SK[nb] = mma16(SK[nb], ak, wf);
        SV[nb] = mma16(SV[nb], av, wf);
      }
    }
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks) {
      const bf16* kp = R.k + (32 * ks + 8 * g + (cc >> 2)) * 16 + 4 * (cc & 3);
      const bf16* vp = R.v + (32 * ks + 8 * g + (cc >> 2)) * 16 + 4 * (cc & 3);
      const bf16x4 k0 = ld_tr4(kp), k1 = ld_tr4(kp + 4 * 16), v0 = ld_tr4(vp), v1 = ld_tr4(vp + 4 * 16);
      bf16x8 ak, av;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ak[e] = k0[e];
        ak[4 + e] = k1[e];
        av[e] = v0[e];
        av[4 + e] = v1[e];
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int i = 16 * nb + cc, q = 4 * ks + g;
        const bf16x8 wf = *reinterpret_cast<const bf16x8*>(R.wt + i * C + 8 * (q ^ (i & (CPR - 1))));
        SK[nb] = mma32(SK[nb], ak, wf);
        SV[nb] = mma32(SV[nb], av, wf);
      }
    }
    // slot s is free again once its reads have completed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(c + NS, s);
  }
  if constexpr (!STORE) {
    if (dec && j0 == 0 && g == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dec[(size_t)useg * MP + 16 * nb + cc] = dk[nb];
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (skout) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int i = 16 * nb + cc;
      if (i < m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          skout[((size_t)useg * m + i) * d + j0 + 4 * g + r] = SK[nb][r];
          svout[((size_t)useg * m + i) * d + j0 + 4 * g + r] = SV[nb][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- slot branch
// The end of a slot-branch row: lane (g, cc) of a wave holds, for query row
// tq, the unnormalised slot read accO (channels 16 db + 4 g .. + 3), its sum
// zs and maximum mx (log2 units).  Without the window branch (o_w null) it
// stores the normalised partial o_L / Z_L and lse_L; with it, the window
// branch's normalised read o_W and lse_W (loaded by load(), early) are merged
// as two partial softmaxes:  o = (Z_L o_L/Z_L + Z_W o_W/Z_W) / (Z_L + Z_W)
// with Z = 2^{lse log2 e} referred to their common maximum, and lse = ln(Z_L
// + Z_W).
template <typename T, int D>
struct WinPartial {
  typename Vec<T>::v4 ow[D / 16];
  float lw;
  bool on;
  __device__ __forceinline__ void load(const T* o_w, const float* lse_w, int b, int h, int row, int Tn, int H,
                                       int g) {
    on = o_w != nullptr;
    if (!on) return;
    const T* src = o_w + (((size_t)b * Tn + row) * H + h) * D + 4 * g;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) ow[db] = ld4<T>(src + 16 * db);
    lw = lse_w[((size_t)b * H + h) * Tn + row];
  }
  __device__ __forceinline__ void store(const floatx4 (&accO)[D / 16], float zs, float mx, T* out, float* lse_out,
                                        int b, int h, int tq, int Tn, int H, int g) const {
    T* dst = out + (((size_t)b * Tn + tq) * H + h) * D + 4 * g;
    const float a = mx + __log2f(zs);  // slot lse, log2 units
    if (!on) {
      const float inv = 1.f / zs;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) st4<T>(dst + 16 * db, pack4<T>(accO[db] * inv));
      if (g == 0 && lse_out) lse_out[((size_t)b * H + h) * Tn + tq] = a * NHA_LN2;
      return;
    }
    const float bw = lw * NHA_LOG2E, M = fmaxf(a, bw);
    const float wl = fast_exp2(a - M), ww = fast_exp2(bw - M), inv = 1.f / (wl + ww);
    const float cl = wl * inv / zs, cw = ww * inv;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      floatx4 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = accO[db][r] * cl + to_f<T>(ow[db][r]) * cw;
      st4<T>(dst + 16 * db, pack4<T>(y));
    }
    if (g == 0 && lse_out) lse_out[((size_t)b * H + h) * Tn + tq] = (M + __log2f(wl + ww)) * NHA_LN2;
  }
};

// grid (NC, B*H), C/16 waves; wave I owns chunk rows 16I .. 16I+15 (queries
// are the N = 16 columns of every product).  Outputs the normalised slot
// partial o_L / Z_L and lse_L = ln(sum_i exp(l_i)) over the m slot logits.
template <typename T, int D, int MP, int C>
struct SlotFwdSmem {
  static constexpr int PD = pitch_of(D), PM = pitch_of(MP), PC = pitch_of(C);
  T sSK[MP * PD];   // S^K_{t0-1} [i][d]
  T sSVt[D * PM];   // S^V_{t0-1}^T [d][i]
  T sK[C * PD];     // kappa rows [u][d]
  T sVt[D * PC];    // nu^T [d][u]
  T sA[C * PM];     // alpha [u][i] (raw gate; a/b derived with the row's t >= w)
  T sB[C * PM];     // 2^{E_J - G_u} b_u  [u][i]
  T sBt[MP * PC];   // same, [i][u]
  float sG[C * SlotPitch<MP>::PG]; // log2 cumsum [u][i]
};

// Operands of one (chunk, head) item held in registers between their global
// loads and their LDS stores, so that the next item's loads run while the
// current item is computed.
template <typename T, int D, int MP, int C, int NT>
struct SlotFwdRegs {
  static constexpr int NG = (C * MP + NT - 1) / NT;
  RowTile<T, D, NT, MP> tsk;
  PairTileT<T, D, NT, MP> tsv;
  RowTile<T, D, NT, C> tkap;
  PairTileT<T, D, NT, C> tnu;
  T al[NG];
};

// grid: a persistent set of workgroups (about one per compute unit), C/16
// waves each, looping over the items (chunk c, head b*H + h); wave I owns
// chunk rows 16I .. 16I+15 (queries are the N = 16 columns of every product).
// Without oW: outputs the normalised slot partial o_L / Z_L and lse_L =
// ln(sum_i exp(l_i)) over the m slot logits.  With oW (the window branch's
// normalised read and its lse, computed first): merges the two partial
// softmaxes -- weights e^{lse_L}, e^{lse_W} -- and outputs o and lse.
template <typename T, int D, int MP, int C>
__global__ __launch_bounds__(C / 16 * 64) void k_slot_fwd(
    const T* __restrict__ q, const T* __restrict__ kk, const T* __restrict__ vv, const T* __restrict__ alpha,
    const T* __restrict__ sst, const T* __restrict__ oW, const float* __restrict__ lseW, T* __restrict__ oL,
    float* __restrict__ lseL, int Tn, int H, int Hkv, int m, int w, int NC, int nitems, float scale) {
  using S = SlotFwdSmem<T, D, MP, C>;
  constexpr int NW = C / 16, NT = NW * 64, NB = MP / 16, PD = S::PD, PM = S::PM, PC = S::PC;
  constexpr int PG = SlotPitch<MP>::PG;
  using R_t = SlotFwdRegs<T, D, MP, C, NT>;
  __shared__ S sm;
  const int tid = threadIdx.x, I = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  const int G = H / Hkv;
  R_t R;
  // item n: chunk n % NC of head n / NC
  auto load = [&](int n) {
    const int c = n % NC, bh = n / NC, b = bh / H, hg = (bh % H) / G, unit = b * Hkv + hg, t0 = c * C;
    const T* src = sst + ((size_t)unit * NC + c) * 2 * MP * D;
    R.tsk.load(src, D, 0, MP, tid);
    R.tsv.load(src + (size_t)MP * D, D, 0, MP, tid);
    // chunk row u <-> token t0 + u, absorbing key row t0 + u - w when t0 + u >= w
    const long rbase = ((long)b * Tn + (t0 - w)) * Hkv + hg;
    R.tkap.load(kk + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
    R.tnu.load(vv + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
#pragma unroll
    for (int k = 0; k < R_t::NG; ++k) {
      const int e = tid + k * NT, u = e / MP, i = e % MP, t = t0 + u;
      R.al[k] = (e < C * MP && i < m && t < Tn) ? alpha[(((size_t)b * Tn + t) * Hkv + hg) * m + i] : to_t<T>(1.f);
    }
  };
  if ((int)blockIdx.x < nitems) load(blockIdx.x);
  for (int n = blockIdx.x; n < nitems; n += gridDim.x) {
    const int c = n % NC, bh = n / NC, b = bh / H, h = bh % H, t0 = c * C;
    __syncthreads();  // the previous item's LDS reads are done
    R.tsk.template store<PD>(sm.sSK, tid);
    R.tsv.template store<PM>(sm.sSVt, tid);
    R.tkap.template store<PD>(sm.sK, tid);
    R.tnu.template store<PC>(sm.sVt, tid);
    // gates: la[u][i] = log2 a_u (0 where nothing is absorbed), raw alpha
#pragma unroll
    for (int k = 0; k < R_t::NG; ++k) {
      const int e = tid + k * NT, u = e / MP, i = e % MP, t = t0 + u;
      if (e < C * MP) {
        sm.sA[u * PM + i] = R.al[k];
        sm.sG[u * PG + i] =
            (i < m && t < Tn && t >= w) ? fmaxf(__log2f(to_f<T>(R.al[k])), NHA_LOG2A_MIN) : 0.f;
      }
    }
    __syncthreads();
    if (n + (int)gridDim.x < nitems) load(n + gridDim.x);  // in flight during this item
    lds_col_cumsum<C, MP, PG, NT>(sm.sG, tid);
    // B^(J)[u][i] = 2^{E_J - G_u} b_u, E_J = G at the last row of u's block
    for (int e = tid; e < C * MP; e += NT) {
      int u = e / MP, i = e % MP, t = t0 + u;
      int last = (u | 15);
      float be = (i < m && t < Tn && t >= w) ? 1.f - to_f<T>(sm.sA[u * PM + i]) : 0.f;
      float val = fast_exp2(sm.sG[last * PG + i] - sm.sG[u * PG + i]) * be;
      T tv = to_t<T>(val);
      sm.sB[u * PM + i] = tv;
      sm.sBt[i * PC + u] = tv;
    }
    __syncthreads();

    // ---- per-wave work: query rows r0 .. r0+15 of the chunk
    const int r0 = 16 * I;
    const int tq = t0 + r0 + cc;  // this lane's query
    const bool qvalid = tq < Tn;
    typename Vec<T>::v8 qf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[ks] = ld8_sel<T>(q + (((size_t)b * Tn + (qvalid ? tq : Tn - 1)) * H + h) * D + 32 * ks + 8 * g, qvalid);
    float lg[NB][4];
    slot_read<T, D, MP, C>(sm.sSK, sm.sK, sm.sBt, sm.sG, sm.sA, qf, I, t0, w, Tn, lg);
    WinPartial<T, D> wp;
    wp.load(oW, lseW, b, h, qvalid ? tq : Tn - 1, Tn, H, g);
    // softmax partial over the m slots (log2 domain)
    const float sl2 = scale * NHA_LOG2E;
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int i = 16 * mb + 4 * g + r;
        lg[mb][r] = (i < m) ? lg[mb][r] * sl2 : -INFINITY;
        mx = fmaxf(mx, lg[mb][r]);
      }
    mx = max_over_g(mx);
    float zs = 0.f;
    float p[NB][4];
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mb][r] = fast_exp2(lg[mb][r] - mx);
        zs += p[mb][r];
      }
    zs = sum_over_g(zs);
    floatx4 accO[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) accO[db] = zero4();
    slot_mix<T, D, MP, C, PC>(sm.sSVt, sm.sVt, sm.sB, sm.sG, sm.sA, p, I, t0, w, Tn, accO);
    // normalised partial + its lse, or merged with the window branch
    if (qvalid) wp.store(accO, zs, mx, oL, lseL, b, h, tq, Tn, H, g);
  }
}

// bf16 variant: grid (NC, B*H), C/16 waves, two workgroups per compute unit.
// The chunk's two tile pairs go through one pair of LDS row tiles in turn --
// S0^K and kappa for the logits, then S0^V and nu for the output, whose
// loads are in flight while the logits are computed -- and the transposed
// operands are read from the row tiles with ds_read_b64_tr_b16.
template <int D, int MP, int C>
struct SlotFwdSmemB16 {
  static constexpr int PD = pitch_of(D), PM = pitch_of(MP);
  bf16 tS[MP * PD];  // S0^K, then S0^V  [i][d]
  bf16 tK[C * PD];   // kappa, then nu    [u][d]
  bf16 sA[C * PM];   // alpha [u][i]
  bf16 sB[C * PM];   // 2^{E_J - G_u} b_u [u][i]
  float sG[C * SlotPitch<MP>::PG];
  SlotTab<C, MP> tab;
};

// One chunk's slot branch for the calling wave's 16 rows (chunk c of head
// bh, LDS in sm): accO (unnormalised read, O^T layout [16 db + 4 g + r][row
// cc]), its sum zs and maximum mx (log2 units).  mid() runs right after the
// logits (its loads then overlap the softmax and the output phase).
template <int D, int MP, int C, typename Mid>
__device__ __forceinline__ void slot_chunk_b16(SlotFwdSmemB16<D, MP, C>& sm, const bf16* __restrict__ q,
                                               const bf16* __restrict__ kk, const bf16* __restrict__ vv,
                                               const bf16* __restrict__ alpha, const bf16* __restrict__ sst, int c,
                                               int bh, int Tn, int H, int Hkv, int m, int w, int NC, float scale,
                                               Mid mid, floatx4 (&accO)[D / 16], float& zs, float& mx) {
  using S = SlotFwdSmemB16<D, MP, C>;
  constexpr int NW = C / 16, NT = NW * 64, NB = MP / 16, PD = S::PD, PM = S::PM;
  constexpr int PG = SlotPitch<MP>::PG;
  const int tid = threadIdx.x, I = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  const int b = bh / H, h = bh % H, G = H / Hkv, hg = h / G;
  const int unit = b * Hkv + hg, t0 = c * C;
  const bf16* src = sst + ((size_t)unit * NC + c) * 2 * MP * D;
  // chunk row u <-> token t0 + u, absorbing key row t0 + u - w when t0 + u >= w
  const long rbase = ((long)b * Tn + (t0 - w)) * Hkv + hg;
  const int r0 = 16 * I;
  const int tq = t0 + r0 + cc;  // this lane's query
  const bool qvalid = tq < Tn;
  // this lane's query row goes out with the first tiles: the logits then
  // wait on no global load, and the output phase's tiles (issued after the
  // first barrier) stay in flight while they are computed
  bf16x8 qf[D / 32];
  {
    GateTile<bf16, C, MP, NT> gt;
    BlockedTile<bf16, D, NT, MP> ts;
    RowTile<bf16, D, NT, C> tk;
    gt.load(alpha, b, hg, t0, Tn, Hkv, m, tid);
    ts.load(src, tid);
    tk.load(kk + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[ks] = ld8_sel<bf16>(q + (((size_t)b * Tn + (qvalid ? tq : Tn - 1)) * H + h) * D + 32 * ks + 8 * g, qvalid);
    gt.template stage<PG, PM>(sm.sG, sm.sA, t0, Tn, m, w, tid);
    ts.template store<PD>(sm.tS, tid);
    tk.template store<PD>(sm.tK, tid);
  }
  __syncthreads();
  lds_col_cumsum<C, MP, PG, NT>(sm.sG, tid);
  for (int e = tid; e < C * MP; e += NT) {
    const int u = e / MP, i = e % MP, t = t0 + u;
    const float be = (i < m && t < Tn && t >= w) ? 1.f - (float)sm.sA[u * PM + i] : 0.f;
    sm.sB[u * PM + i] = (bf16)(fast_exp2(sm.sG[(u | 15) * PG + i] - sm.sG[u * PG + i]) * be);
  }
  build_slot_tab<C, MP, NT>(sm.tab, sm.sG, tid);
  __syncthreads();
  // the output phase's tiles: loads in flight during the logits
  BlockedTile<bf16, D, NT, MP> tsv;
  RowTile<bf16, D, NT, C> tnu;
  tsv.load(src + (size_t)MP * D, tid);
  tnu.load(vv + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
  float lg[NB][4];
  slot_read<bf16, D, MP, C, true>(sm.tS, sm.tK, sm.sB, sm.sG, sm.sA, qf, I, t0, w, Tn, lg, &sm.tab);
  mid();
  // softmax partial over the m slots (log2 domain)
  const float sl2 = scale * NHA_LOG2E;
  mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * mb + 4 * g + r;
      lg[mb][r] = (i < m) ? lg[mb][r] * sl2 : -INFINITY;
      mx = fmaxf(mx, lg[mb][r]);
    }
  mx = max_over_g(mx);
  zs = 0.f;
  float p[NB][4];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[mb][r] = fast_exp2(lg[mb][r] - mx);
      zs += p[mb][r];
    }
  zs = sum_over_g(zs);
  __syncthreads();  // every wave is done with S0^K and kappa
  tsv.template store<PD>(sm.tS, tid);
  tnu.template store<PD>(sm.tK, tid);
  __syncthreads();
#pragma unroll
  for (int db = 0; db < D / 16; ++db) accO[db] = zero4();
  slot_mix<bf16, D, MP, C, PD, true>(sm.tS, sm.tK, sm.sB, sm.sG, sm.sA, p, I, t0, w, Tn, accO, &sm.tab);
}

template <int D, int MP, int C>
__global__ __launch_bounds__(C / 16 * 64, 2) void k_slot_fwd_b16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ vv,
    const bf16* __restrict__ alpha, const bf16* __restrict__ sst, const bf16* __restrict__ oW,
    const float* __restrict__ lseW, bf16* __restrict__ oL, float* __restrict__ lseL, int Tn, int H, int Hkv, int m,
    int w, int NC, float scale) {
  __shared__ SlotFwdSmemB16<D, MP, C> sm;
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int c = L % NC, bh = L / NC, b = bh / H, h = bh % H;
  const int g = (threadIdx.x & 63) >> 4, tq = c * C + 16 * (threadIdx.x >> 6) + (threadIdx.x & 15);
  const bool qvalid = tq < Tn;
  // the window branch's read for this lane's row, issued after the logits
  // (the query row registers are free then): in flight during the slot
  // softmax and the output phase
  WinPartial<bf16, D> wp;
  floatx4 accO[D / 16];
  float zs, mx;
  slot_chunk_b16<D, MP, C>(sm, q, kk, vv, alpha, sst, c, bh, Tn, H, Hkv, m, w, NC, scale,
                           [&]() { wp.load(oW, lseW, b, h, qvalid ? tq : Tn - 1, Tn, H, g); }, accO, zs, mx);
  if (qvalid) wp.store(accO, zs, mx, oL, lseL, b, h, tq, Tn, H, g);
}

// ---------------------------------------------------------------- window branch
// grid (ceil(T / (32 NWV)), B*H), NWV waves; wave W owns queries q0 + 32W ..
// +31 and works on 32x32 tiles with the query index as the column:
// S^T = K Q^T (key rows), O^T += V^T P^T, so every lane holds one query's
// scores and output column and the softmax bookkeeping stays in the lane
// (plus its partner lane l ^ 32 for the maximum and the sum).  Online softmax
// in log2 units, seeded with the slot partial as one key of logit lse_L and
// value o_L / Z_L; the running maximum is only moved (and O rescaled) when a
// tile raises it by more than 2^kLazy, which keeps every exponent <= kLazy.
// One 64-row K / V tile is staged in LDS at a time and serves all 32 NWV
// queries; the next tile's global loads are in flight (in registers) while
// the current one is used.  A wave skips tiles outside its rows' band and
// masks only the tiles that cross the band's edges.  Writes o and lse.
constexpr int kWinWaves = 4;
constexpr float kLazy = 8.f;
// running maximum (log2 units) of an empty softmax: finite, so that
// 2^(score - max) of a masked score is 0, and below every real logit
constexpr float kEmptyMax = -1e30f;

template <typename T, int D>
struct WinFwdSmem {
  // row pitches of 4 (mod 32) dwords: 8 lanes reading 16 bytes each at the
  // same column of 8 consecutive rows cover the 32 banks once
  static constexpr int PD = pitch_of(D), PK = 64 + 16 / (int)sizeof(T);
  T k[64 * PD];  // RoPE'd keys [key][d]
  T vt[D * PK];  // values, transposed [d][kswz(key)]
};

template <typename T, int D, int NWV>
__global__ __launch_bounds__(NWV * 64, 2) void k_win_fwd(const T* __restrict__ qr, const T* __restrict__ kr,
                                                      const T* __restrict__ vv, const T* __restrict__ oL,
                                                      const float* __restrict__ lseL, T* __restrict__ o,
                                                      float* __restrict__ lse, int Tn, int H, int Hkv, int w,
                                                      float scale) {
  using S = WinFwdSmem<T, D>;
  constexpr int PD = S::PD, PK = S::PK, NT = NWV * 64, QT = 32 * NWV;
  __shared__ S sm[2];
  const int tid = threadIdx.x, W = tid >> 6, l = tid & 63, hf = l >> 5, c = l & 31;
  // logical tile = (query tile, b*H + h), XCD-contiguous
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int q0 = (L % gridDim.x) * QT, bh = L / gridDim.x, b = bh / H, h = bh % H, hg = h / (H / Hkv);
  const int wl = q0 + 32 * W;  // first query of this wave
  const int tq = wl + c;
  const bool qvalid = tq < Tn;
  const int tqc = qvalid ? tq : Tn - 1;  // clamped row: loads stay unconditional
  const size_t qrow = (((size_t)b * Tn + tqc) * H + h) * D;
  typename Vec<T>::v8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = ld8_sel<T>(qr + qrow + 16 * ks + 8 * hf, qvalid);
  // seed with the slot partial (no slots, oL null: an empty softmax, whose
  // running maximum is a finite floor that the query's own key raises)
  const bool seeded = oL != nullptr;
  const float lse_l = seeded ? lseL[(size_t)bh * Tn + tqc] : 0.f;  // unconditional load (clamped row)
  float mu = qvalid ? (seeded ? lse_l * NHA_LOG2E : kEmptyMax) : 0.f;
  float zl = (hf == 0 && seeded) ? 1.f : 0.f;  // lane-partial normaliser
  floatx16 acc[D / 32];                        // O^T: rows d = 32 dt + 8 i + 4 hf + rr, column = query
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    acc[dt] = zero16();
    if (seeded) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        typename Vec<T>::v4 x = ld4<T>(oL + qrow + 32 * dt + 8 * i + 4 * hf);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[dt][4 * i + rr] = qvalid ? to_f<T>(x[rr]) : 0.f;
      }
    }
  }
  const float sl2 = scale * NHA_LOG2E;
  if (w > 0) {
    int kmin = q0 - w + 1;
    if (kmin < 0) kmin = 0;
    int kmax = q0 + QT - 1;
    if (kmax > Tn - 1) kmax = Tn - 1;
    const int jfirst = (kmin / 64) * 64;
    const int ntiles = (kmax - jfirst) / 64 + 1;
    const size_t ld = (size_t)Hkv * D;
    const T* kbase = kr + ((size_t)b * Tn * Hkv + hg) * D;
    const T* vbase = vv + ((size_t)b * Tn * Hkv + hg) * D;
    RowTile<T, D, NT> tk;
    PairTileT<T, D, NT, 64, true> tv;
    tk.load(kbase + (size_t)jfirst * ld, ld, 0, Tn - jfirst, tid);
    tv.load(vbase + (size_t)jfirst * ld, ld, 0, Tn - jfirst, tid);
    tk.template store<PD>(sm[0].k, tid);
    tv.template store<PK>(sm[0].vt, tid);
    if (ntiles > 1) {
      int jn = jfirst + 64;
      tk.load(kbase + (size_t)jn * ld, ld, 0, Tn - jn, tid);
      tv.load(vbase + (size_t)jn * ld, ld, 0, Tn - jn, tid);
    }
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int j0 = jfirst + 64 * it;
      // stage tile it+1 into the other buffer (last read before the previous
      // barrier) and start the global loads of tile it+2
      if (it + 1 < ntiles) {
        tk.template store<PD>(sm[(it + 1) & 1].k, tid);
        tv.template store<PK>(sm[(it + 1) & 1].vt, tid);
        if (it + 2 < ntiles) {
          int jn = j0 + 128;
          tk.load(kbase + (size_t)jn * ld, ld, 0, Tn - jn, tid);
          tv.load(vbase + (size_t)jn * ld, ld, 0, Tn - jn, tid);
        }
      }
      const S& cur = sm[it & 1];
      // does this tile meet the band of the wave's rows [wl, wl + 31]?
      const bool useful = wl < Tn && j0 <= wl + 31 && j0 + 63 > wl - w;
      if (useful) {
        const bool full = (j0 + 63 <= wl) && (j0 > wl + 31 - w) && (j0 + 63 < Tn);
        // S^T = K Q^T; the K fragments of step ks+1 are read while step ks runs
        floatx16 s[2];
        s[0] = zero16();
        s[1] = zero16();
        typename Vec<T>::v8 kfr[2][2];
        kfr[0][0] = ld8<T>(&cur.k[c * PD + 8 * hf]);
        kfr[0][1] = ld8<T>(&cur.k[(32 + c) * PD + 8 * hf]);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          if (ks + 1 < D / 16) {
            kfr[(ks + 1) & 1][0] = ld8<T>(&cur.k[c * PD + 16 * (ks + 1) + 8 * hf]);
            kfr[(ks + 1) & 1][1] = ld8<T>(&cur.k[(32 + c) * PD + 16 * (ks + 1) + 8 * hf]);
          }
          s[0] = mma32x32(s[0], kfr[ks & 1][0], qf[ks]);
          s[1] = mma32x32(s[1], kfr[ks & 1][1], qf[ks]);
        }
        // V^T fragments of the first step, read while the softmax runs
        typename Vec<T>::v8 vfr[2][D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) vfr[0][dt] = ld8<T>(&cur.vt[(32 * dt + c) * PK + 8 * hf]);
        if (!full) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
              bool ok = key <= tq && key > tq - w && key < Tn;
              s[kb][r] = ok ? s[kb][r] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_halves(mx) * sl2;
        const bool raise = mx > mu + kLazy;
        if (__any(raise)) {
          float mnew = raise ? mx : mu;
          float resc = fast_exp2(mu - mnew);
          mu = mnew;
          zl *= resc;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= resc;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float pv = fast_exp2(fmaf(s[kb][r], sl2, -mu));
            s[kb][r] = pv;
            zl += pv;
          }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (st + 1 < 4) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
              vfr[(st + 1) & 1][dt] = ld8<T>(&cur.vt[(32 * dt + c) * PK + 16 * (st + 1) + 8 * hf]);
          }
          typename Vec<T>::v8 bfr = pack8_at<T>(s[st >> 1], 8 * (st & 1));
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mma32x32(acc[dt], vfr[st & 1][dt], bfr);
        }
      }  // useful
      __syncthreads();
    }
  }
  const float z = sum_halves(zl);
  if (qvalid) {
    const float inv = 1.f / z;
    T* dst = o + qrow;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st4<T>(dst + 32 * dt + 8 * i + 4 * hf,
               pack4<T>(floatx4{acc[dt][4 * i] * inv, acc[dt][4 * i + 1] * inv, acc[dt][4 * i + 2] * inv,
                                acc[dt][4 * i + 3] * inv}));
    if (hf == 0 && lse) lse[(size_t)bh * Tn + tq] = (mu + __log2f(z)) * NHA_LN2;
  }
}

// bf16 variant of the same kernel, software-pipelined: K and V tiles go
// straight from global memory to LDS (no staging registers; K triple-, V
// double-buffered) and the transposed V operand is read with
// ds_read_b64_tr_b16 from the row-major tile.  While the softmax of tile i
// runs on the vector ALUs, the matrix cores already compute the scores of
// tile i+1; masks enter as -inf in the initial value of the score
// accumulators, so only the tiles that cross the band's edges pay for them.
// The band of the workgroup's QT = 32 NWV queries q0 .. of head bh, with
// its K / V tiles in kbuf (3 tiles) and vbuf (2 tiles) of LDS; seed(acc, mu,
// zl, qrow, tqc, qvalid) starts each lane's online softmax (an empty one, or
// a partial softmax of the same row).  SYNC: a barrier between the seed and
// the first tile loads (the seed may then sit in the tile buffers).
template <int D, int NWV, bool SYNC, typename Seed>
__device__ __forceinline__ void win_band_b16(bf16 (*kbuf)[64 * D], bf16 (*vbuf)[64 * D], const bf16* __restrict__ qr,
                                             const bf16* __restrict__ kr, const bf16* __restrict__ vv,
                                             bf16* __restrict__ o, float* __restrict__ lse, int q0, int bh, int Tn,
                                             int H, int Hkv, int w, float scale, Seed seed) {
  constexpr int NT = NWV * 64, QT = 32 * NWV;
  // wave-uniform quantities are pinned to scalar registers (integer division
  // is expanded on the vector ALUs otherwise)
  const int tid = threadIdx.x, W = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, hf = l >> 5, c = l & 31,
            jj = l & 15;
  const int b = __builtin_amdgcn_readfirstlane(bh / H), h = __builtin_amdgcn_readfirstlane(bh % H),
            hg = __builtin_amdgcn_readfirstlane(h / (H / Hkv));
  const int wl = q0 + 32 * W;
  const int tq = wl + c;
  const bool qvalid = tq < Tn;
  const int tqc = qvalid ? tq : Tn - 1;  // clamped row: loads stay unconditional
  const size_t qrow = (((size_t)b * Tn + tqc) * H + h) * D;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = ld8_sel<bf16>(qr + qrow + 16 * ks + 8 * hf, qvalid);
  float mu, zl;
  floatx16 acc[D / 32];
  seed(acc, mu, zl, qrow, tqc, qvalid);
  if constexpr (SYNC) __syncthreads();
  // per-lane LDS element offsets of the K fragments (row c, logical chunk
  // 2 ks + hf) and of the transposed V reads (rows 4 hf + jj / 4 (+8) of each
  // 16-row step, columns 32 dt + 16 (c / 16) + 4 (jj % 4) ..)
  // byte offsets: K fragment of step ks at koff[ks] (+ 64 D for the second
  // 32-key block), transposed V reads of column block dt at voff[dt]
  uint32_t koff[D / 16], voff[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = 2 * (c * D + 8 * ((2 * ks + hf) ^ chunk_swz<D, 0>(c)));
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int r = 4 * hf + (jj >> 2), d0 = 32 * dt + 16 * (c >> 4) + 4 * (jj & 3);
    voff[dt] = 2 * (r * D + 8 * ((d0 >> 3) ^ chunk_swz<D, 1>(r)) + (d0 & 7));
  }
  const float sl2 = scale * NHA_LOG2E;
  if (w > 0) {
    int kmin = q0 - w + 1;
    if (kmin < 0) kmin = 0;
    int kmax = q0 + QT - 1;
    if (kmax > Tn - 1) kmax = Tn - 1;
    const int jfirst = (kmin / 64) * 64;
    const int ntiles = (kmax - jfirst) / 64 + 1;
    // key tiles in a rotated order (step it takes the tile X = it mod
    // ntiles): the workgroups of neighbouring query tiles, resident together
    // on one XCD, then read each key tile at the same step, and all but the
    // first hit the XCD's L2
    const int rot = (ntiles - (jfirst / 64) % ntiles) % ntiles;
    auto tile_j0 = [&](int it) {
      const int jr = it + rot >= ntiles ? it + rot - ntiles : it + rot;
      return jfirst + 64 * jr;
    };
    const size_t ld = (size_t)Hkv * D;
    const bf16* kbase = kr + ((size_t)b * Tn * Hkv + hg) * D;
    const bf16* vbase = vv + ((size_t)b * Tn * Hkv + hg) * D;
    const uint32_t kl = lds_addr(&kbuf[0][0]), vl = lds_addr(&vbuf[0][0]);
    const uint32_t kdo = dma_lane_off<D, NT, 0>(tid, ld), vdo = dma_lane_off<D, NT, 1>(tid, ld);
    constexpr uint32_t TB = 64 * D * 2;  // bytes per tile

    auto useful = [&](int j0) { return wl < Tn && j0 <= wl + 31 && j0 + 63 > wl - w; };
    // scores of the tile at j0 outside the band (or of a tile the wave does
    // not need at all) -> -inf; skipped for tiles inside the band
    auto mask_tile = [&](floatx16(&x)[2], int j0, bool use) {
      if (!use || !((j0 + 63 <= wl) && (j0 > wl + 31 - w) && (j0 + 63 < Tn))) {
        // key - tq = rel + (32 kb + 8 (r / 4) + r % 4) must lie in (-w, hi];
        // an unused tile takes rel = 1, span = 0, which rejects every key
        // (one code path keeps the scores in place, without copies)
        const int rel = use ? j0 + 4 * hf - tq + w - 1 : 1;
        const uint32_t span = use ? (uint32_t)(min(0, Tn - 1 - tq) + w - 1) : 0u;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((uint32_t)(rel + 32 * kb + 8 * (r >> 2) + (r & 3)) > span) x[kb][r] = -INFINITY;
      }
    };
    // One pass over the next tile's scores and/or this tile's softmax, cut
    // into 2 D/16 short regions (sched_barrier: nothing moves across) of one
    // score MFMA, the K read RA steps ahead and a slice of the softmax, so
    // the vector ALUs work while the matrix core runs and no region hoists
    // more reads than registers allow.  kt: LDS byte address of the next K
    // tile (kept opaque so that one address per step is formed).
    constexpr int NG = 2 * (D / 16), RA = 4;
    auto main_pass = [&](auto do_s, auto do_sm, floatx16(&nx)[2], uint32_t kt, floatx16(&x)[2], bf16x8(&pf)[4],
                         float& resc, bool& any_raise) {
      bf16x8 kr[RA];
      if constexpr (do_s.value) {
#pragma unroll
        for (int g = 0; g < RA; ++g) kr[g] = ld8_at(kt + koff[g >> 1] + (g & 1) * 64 * D);
      }
      float mx = -INFINITY, zs = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if constexpr (do_s.value) {
          nx[g & 1] = mma32x32(g < 2 ? zero16() : nx[g & 1], kr[g % RA], qf[g >> 1]);
          if (g + RA < NG) kr[g % RA] = ld8_at(kt + koff[(g + RA) >> 1] + ((g + RA) & 1) * 64 * D);
        }
        if constexpr (do_sm.value) {
          constexpr int NMAX = NG / 4;                                  // regions computing the maximum
          constexpr int PER = (32 + NG - NMAX - 2) / (NG - NMAX - 1);  // exponentials per region
          if (g < NMAX) {
#pragma unroll
            for (int e = 0; e < 32 / NMAX; ++e) {
              const int k = g * (32 / NMAX) + e;
              mx = fmaxf(mx, x[k >> 4][k & 15]);
            }
          } else if (g == NMAX) {
            mx = max_halves(mx) * sl2;
            const bool raise = mx > mu + kLazy;
            const float mnew = raise ? mx : mu;
            resc = fast_exp2(mu - mnew);
            mu = mnew;
            any_raise = __any(raise);
          } else {
#pragma unroll
            for (int e0 = 0; e0 < PER; ++e0) {
              const int e = (g - NMAX - 1) * PER + e0;
              if (e < 32) {
                const float pv = fast_exp2(fmaf(x[e >> 4][e & 15], sl2, -mu));
                x[e >> 4][e & 15] = pv;
                zs += pv;
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (do_sm.value) {
        zl = zl * resc + zs;
#pragma unroll
        for (int st = 0; st < 4; ++st) pf[st] = pack8_at<bf16>(x[st >> 1], 8 * (st & 1));
      }
    };
    // O^T += V^T P^T: 4 (D/32) MFMAs, each one's transposed reads issued VA
    // MFMAs ahead
    constexpr int NP = 4 * (D / 32), VA = 3;
    auto pv = [&](const bf16x8(&pf)[4], uint32_t vt) {
      bf16x8 vr[VA];
      auto vload = [&](int g) {
        const uint32_t p = vt + voff[g % (D / 32)] + 32 * (g / (D / 32)) * D;
        const bf16x4 a0 = ld_tr4_at(p), a1 = ld_tr4_at(p + 16 * D);
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = a0[e];
          f[4 + e] = a1[e];
        }
        return f;
      };
#pragma unroll
      for (int g = 0; g < VA; ++g) vr[g] = vload(g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < NP; ++g) {
        acc[g % (D / 32)] = mma32x32(acc[g % (D / 32)], vr[g % VA], pf[g / (D / 32)]);
        if (g + VA < NP) vr[g % VA] = vload(g + VA);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;

    dma_tile_async<D, NT, 0>(kbase, ld, tile_j0(0), Tn, kl, kdo, tid);
    dma_tile_async<D, NT, 1>(vbase, ld, tile_j0(0), Tn, vl, vdo, tid);
    if (ntiles > 1) dma_tile_async<D, NT, 0>(kbase, ld, tile_j0(1), Tn, kl + TB, kdo, tid);
    wait_vmem();
    __syncthreads();
    floatx16 sa[2], sb[2];
    bool use_c = useful(tile_j0(0));
    {
      bf16x8 pf0[4];
      float r0;
      bool a0;
      main_pass(T_{}, F_{}, sa, __builtin_amdgcn_readfirstlane(kl), sb, pf0, r0, a0);
    }
    auto step = [&](floatx16(&cur)[2], floatx16(&nxt)[2], int it) {
      const int j0 = tile_j0(it);
      if (it + 2 < ntiles)
        dma_tile_async<D, NT, 0>(kbase, ld, tile_j0(it + 2), Tn, kl + ((it + 2) % 3) * TB, kdo, tid);
      if (it + 1 < ntiles)
        dma_tile_async<D, NT, 1>(vbase, ld, tile_j0(it + 1), Tn, vl + ((it + 1) & 1) * TB, vdo, tid);
      const bool use_n = it + 1 < ntiles && useful(tile_j0(it + 1));
      if (use_c || use_n) {
        // one code path for every case (separate variants would each need
        // their own registers): a tile this wave does not need is masked to
        // -inf when it becomes the current one, and past the last tile the
        // pass reads a stale buffer whose scores are never used
        const uint32_t ktn = __builtin_amdgcn_readfirstlane(kl + ((it + 1) % 3) * TB);
        bool any_raise = false;
        float resc = 1.f;
        bf16x8 pf[4];
        mask_tile(cur, j0, use_c);
        main_pass(T_{}, T_{}, nxt, ktn, cur, pf, resc, any_raise);
        if (any_raise) {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= resc;
        }
        pv(pf, __builtin_amdgcn_readfirstlane(vl + (it & 1) * TB));
      }
      use_c = use_n;
      wait_vmem();
      __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
      step(sa, sb, it);
      if (it + 1 < ntiles) step(sb, sa, it + 1);
    }
  }
  const float z = sum_halves(zl);
  // o in whole rows through the K tile buffers (free after the last barrier;
  // unused when w = 0)
  {
    const float inv = 1.f / z;
    static_assert(NWV * 32 * (D + 4) * 2 <= 3 * 64 * D * 2, "staging fits the K tile buffers");
    bf16* stg = &kbuf[0][0] + W * 32 * (D + 4);
    auto roff = [&](int row) { return (((size_t)b * Tn + (wl + row)) * H + h) * D; };
    store_tile_rows<D>([&](int dt, int e) { return acc[dt][e] * inv; }, stg, o, (const bf16*)nullptr, roff,
                       [](int) { return false; }, min(32, Tn - wl));
  }
  if (qvalid && hf == 0 && lse) lse[(size_t)bh * Tn + tq] = (mu + __log2f(z)) * NHA_LN2;
}

template <int D, int NWV>
__global__ __launch_bounds__(NWV * 64, 2) void k_win_fwd_b16(const bf16* __restrict__ qr, const bf16* __restrict__ kr,
                                                             const bf16* __restrict__ vv, const bf16* __restrict__ oL,
                                                             const float* __restrict__ lseL, bf16* __restrict__ o,
                                                             float* __restrict__ lse, int Tn, int H, int Hkv, int w,
                                                             float scale) {
  constexpr int QT = 32 * NWV;
  __shared__ bf16 kbuf[3][64 * D];
  __shared__ bf16 vbuf[2][64 * D];
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int q0 = __builtin_amdgcn_readfirstlane((L % gridDim.x) * QT), bh = __builtin_amdgcn_readfirstlane(L / gridDim.x);
  // seed with the slot partial (o_L / Z_L and lse_L in the workspace), or (no
  // slots) an empty softmax
  auto seed = [&](floatx16(&acc)[D / 32], float& mu, float& zl, size_t qrow, int tqc, bool qvalid) {
    const int hf = (threadIdx.x & 63) >> 5;
    const bool seeded = oL != nullptr;
    const float lse_l = seeded ? lseL[(size_t)bh * Tn + tqc] : 0.f;  // unconditional load (clamped row)
    mu = qvalid ? (seeded ? lse_l * NHA_LOG2E : kEmptyMax) : 0.f;
    zl = (hf == 0 && seeded) ? 1.f : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      acc[dt] = zero16();
      if (seeded) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 x = ld4<bf16>(oL + qrow + 32 * dt + 8 * i + 4 * hf);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[dt][4 * i + rr] = qvalid ? (float)x[rr] : 0.f;
        }
      }
    }
  };
  win_band_b16<D, NWV, false>(kbuf, vbuf, qr, kr, vv, o, lse, q0, bh, Tn, H, Hkv, w, scale, seed);
}

// ---------------------------------------------------------------- forward chunk kernel
// Both branches of a query tile in one workgroup (bf16, C = 64; the chunk
// computation of the Paper-Notes page, section 关键设计 > Chunkwise 并行计算:
// the slot logits and the window logits of a chunk's queries under one
// softmax, then both aggregations).  grid (ceil(T / 128), B*H), 4 waves.
// The tile's two chunks first run the slot branch (one after the other, the
// first chunk's partial kept in registers); both partials -- o_L / Z_L in
// bf16 and lse_L -- then go into LDS, and the window band starts its online
// softmax from them (the partial as one key of logit lse_L and value
// o_L / Z_L) and writes o and lse.  The slot and window phases share the
// LDS (80 KB, two workgroups per CU); the chunk-start states come from the
// state scan and the RoPE'd q / k from the RoPE pass.  Co-resident
// workgroups in different phases overlap the slot branch's memory traffic
// with the window branch's products, and the window partial makes no HBM
// round trip.
template <int D, int MP>
struct ChunkFwdLds {
  static constexpr int C = 64, QT = 32 * kWinWaves, SP = D + 8;
  static_assert(QT == 2 * C, "a window tile is two chunks");
  static constexpr size_t SLOT = sizeof(SlotFwdSmemB16<D, MP, C>), WIN = 5 * 64 * D * 2,
                          SEED = (size_t)QT * SP * 2 + QT * 4;
  static constexpr size_t BYTES = SLOT > WIN ? (SLOT > SEED ? SLOT : SEED) : (WIN > SEED ? WIN : SEED);
};

template <int D, int MP>
__global__ __launch_bounds__(kWinWaves * 64, 2) void k_chunk_fwd_b16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ vv,
    const bf16* __restrict__ alpha, const bf16* __restrict__ sst, const bf16* __restrict__ qr,
    const bf16* __restrict__ kr, bf16* __restrict__ o, float* __restrict__ lse, int Tn, int H, int Hkv, int m,
    int w, int sh, int NC, float scale) {
  using Lay = ChunkFwdLds<D, MP>;
  constexpr int C = Lay::C, QT = Lay::QT, SP = Lay::SP;
  __shared__ __align__(16) unsigned char smem[Lay::BYTES];
  auto& sm = *reinterpret_cast<SlotFwdSmemB16<D, MP, C>*>(smem);
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int tile = __builtin_amdgcn_readfirstlane(L % gridDim.x), bh = __builtin_amdgcn_readfirstlane(L / gridDim.x);
  const int q0 = tile * QT, tid = threadIdx.x, I = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  // slot branch of the two chunks (the second one may lie past the end)
  floatx4 a0[D / 16], a1[D / 16];
  float z0, m0, z1 = 1.f, m1 = 0.f;
  slot_chunk_b16<D, MP, C>(sm, q, kk, vv, alpha, sst, 2 * tile, bh, Tn, H, Hkv, m, sh, NC, scale, []() {}, a0, z0,
                           m0);
  const bool two = 2 * tile + 1 < NC;
  if (two) {
    __syncthreads();  // every wave is done with the first chunk's tiles
    slot_chunk_b16<D, MP, C>(sm, q, kk, vv, alpha, sst, 2 * tile + 1, bh, Tn, H, Hkv, m, sh, NC, scale, []() {},
                             a1, z1, m1);
  }
  __syncthreads();
  // the partials into LDS: rows [QT][SP] of o_L / Z_L (bf16), then lse_L
  // (log2 units) per row
  bf16* so = reinterpret_cast<bf16*>(smem);
  float* sl = reinterpret_cast<float*>(smem + (size_t)QT * SP * 2);
  auto put = [&](int ch, const floatx4(&a)[D / 16], float z, float mxv) {
    const int row = ch * C + 16 * I + cc;
    const float inv = 1.f / z;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) st4<bf16>(so + row * SP + 16 * db + 4 * g, pack4<bf16>(a[db] * inv));
    if (g == 0) sl[row] = mxv + __log2f(z);
  };
  put(0, a0, z0, m0);
  if (two) put(1, a1, z1, m1);
  __syncthreads();
  // each lane's row of the window tile (wave W, lane c: query q0 + 32 W + c)
  auto seed = [&](floatx16(&acc)[D / 32], float& mu, float& zl, size_t, int, bool qvalid) {
    const int hf = (threadIdx.x & 63) >> 5, row = 32 * (threadIdx.x >> 6) + (threadIdx.x & 31);
    mu = qvalid ? sl[row] : 0.f;
    zl = hf == 0 ? 1.f : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x4 x = *reinterpret_cast<const bf16x4*>(so + row * SP + 32 * dt + 8 * i + 4 * hf);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[dt][4 * i + rr] = qvalid ? (float)x[rr] : 0.f;
      }
  };
  bf16(*kb)[64 * D] = reinterpret_cast<bf16(*)[64 * D]>(smem);
  win_band_b16<D, kWinWaves, true>(kb, kb + 3, qr, kr, vv, o, lse, q0, bh, Tn, H, Hkv, w, scale, seed);
}

// ---------------------------------------------------------------- decode-state export
// Ring rows for positions max(0, T-w) .. T-1 (raw keys, values and, with
// RoPE, the RoPE'd keys the forward computed) and the position counter; row j
// of the sequence is absolute position pos0 + j (pos0 > 0 for a continued
// segment).
template <typename T>
__global__ void k_export_state(const T* __restrict__ kk, const T* __restrict__ vv, const T* __restrict__ kr,
                               T* __restrict__ rk, T* __restrict__ rv, T* __restrict__ rkr,
                               long long* __restrict__ pos, int Tn, int Hkv, int d, int w, long long pos0) {
  int unit = blockIdx.y, b = unit / Hkv, hg = unit % Hkv;
  int first = Tn - w > 0 ? Tn - w : 0;
  int nrows = w > 0 ? Tn - first : 0;
  for (int e = (blockIdx.x * blockDim.x + threadIdx.x) * 8; e < nrows * d; e += gridDim.x * blockDim.x * 8) {
    int j = first + e / d, x = e % d;
    size_t src = (((size_t)b * Tn + j) * Hkv + hg) * d + x;
    size_t dst = ((size_t)unit * w + (size_t)((pos0 + j) % w)) * d + x;
    st8<T>(rk + dst, ld8<T>(kk + src));
    st8<T>(rv + dst, ld8<T>(vv + src));
    if (kr) st8<T>(rkr + dst, ld8<T>(kr + src));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) pos[unit] = pos0 + Tn;
}

// ---------------------------------------------------------------- segmented scan: start states
// In place over the segment rows (unit * nseg + p) of segk / segv [.][m][d]:
// they hold each segment's end state from a zero start and receive its start
// state, start(0) = s0 (null: zero), start(p + 1) = D_p (.) start(p) + end(p),
// where D_p[i] = dec[unit * nseg + p][i] is the product of 2^{G_end,i} over
// the segment's chunks (the recurrence is linear, with one decay per slot
// row).  The state after the last segment goes to skout / svout when not null.
// grid (ceil(m d / 256), B*Hkv), 256 threads.
__global__ __launch_bounds__(256) void k_scan_combine(const float* __restrict__ dec, float* __restrict__ segk,
                                                      float* __restrict__ segv, const float* __restrict__ s0k,
                                                      const float* __restrict__ s0v, float* __restrict__ skout,
                                                      float* __restrict__ svout, int m, int d, int MP, int nseg) {
  const int unit = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= m * d) return;
  const int i = e / d;
  const size_t u0 = (size_t)unit * m * d + e;
  float sk = s0k ? s0k[u0] : 0.f, sv = s0v ? s0v[u0] : 0.f;
  for (int p = 0; p < nseg; ++p) {
    const size_t r = ((size_t)unit * nseg + p) * m * d + e;
    const float ek = segk[r], ev = segv[r], D = dec[((size_t)unit * nseg + p) * MP + i];
    segk[r] = sk;
    segv[r] = sv;
    sk = D * sk + ek;
    sv = D * sv + ev;
  }
  if (skout) {
    skout[u0] = sk;
    svout[u0] = sv;
  }
}

// ---------------------------------------------------------------- host launcher
template <typename T, int C, int MP>
static void launch_gates(const Shape& s, const T* alpha, const ProloguePtrs& pp, hipStream_t st) {
  hipLaunchKernelGGL((k_chunk_gates<T, C, MP>), dim3(s.NC, s.B * s.Hkv), dim3(256), 0, st, alpha, (T*)pp.wt, pp.aend,
                     s.T, s.Hkv, s.m, s.sh, s.NC);
}

template <typename T, int D, int C, int MP>
static void launch_scan(const Shape& s, const T* k, const T* v, const ProloguePtrs& pp, Marks& mk,
                        hipStream_t st) {
  const int units = s.B * s.Hkv;
  if constexpr (sizeof(T) == 2) {
    const ScanSegs sg = scan_segments(s);
    if (sg.n > 1) {
      // three launches: segment end states, segment start states, the walk
      float* sk = pp.seg;
      float* sv = sk + (size_t)units * sg.n * s.m * D;
      float* dc = sv + (size_t)units * sg.n * s.m * D;
      hipLaunchKernelGGL((k_state_scan_b16<C, MP, 4, false>), dim3(D / 16, units * sg.n), dim3(64), 0, st, k, v,
                         (const T*)pp.wt, (const float*)pp.aend, (T*)pp.sst, sk, sv, dc, (const float*)nullptr,
                         (const float*)nullptr, s.T, s.Hkv, D, s.m, s.sh, s.NC, sg.n, sg.len);
      mk.mark(st);
      hipLaunchKernelGGL(k_scan_combine, dim3((s.m * D + 255) / 256, units), dim3(256), 0, st, (const float*)dc,
                         sk, sv, pp.s0k, pp.s0v, pp.skout, pp.svout, s.m, D, MP, sg.n);
      mk.mark(st);
      hipLaunchKernelGGL((k_state_scan_b16<C, MP, 4, true>), dim3(D / 16, units * sg.n), dim3(64), 0, st, k, v,
                         (const T*)pp.wt, (const float*)pp.aend, (T*)pp.sst, (float*)nullptr, (float*)nullptr,
                         (float*)nullptr, (const float*)sk, (const float*)sv, s.T, s.Hkv, D, s.m, s.sh, s.NC, sg.n,
                         sg.len);
    } else {
      hipLaunchKernelGGL((k_state_scan_b16<C, MP, 4, true>), dim3(D / 16, units), dim3(64), 0, st, k, v,
                         (const T*)pp.wt, (const float*)pp.aend, (T*)pp.sst, pp.skout, pp.svout, (float*)nullptr,
                         pp.s0k, pp.s0v, s.T, s.Hkv, D, s.m, s.sh, s.NC, 1, s.NC);
    }
  } else
    hipLaunchKernelGGL((k_state_scan<T, C, MP>), dim3(D / 16, units), dim3(64), 0, st, k, v, (const T*)pp.wt,
                       (const float*)pp.aend, (T*)pp.sst, pp.skout, pp.svout, pp.s0k, pp.s0v, s.T, s.Hkv, D, s.m,
                       s.sh, s.NC);
}

// RoPE table, then the RoPE'd q and k rows (two launches)
template <typename T>
static void launch_rope(const Shape& s, const RopeTheta& th, const T* q, const T* k, const ProloguePtrs& pp,
                        Marks& mk, hipStream_t rs) {
  const long nq = (long)s.B * s.T * s.H, nk = (long)s.B * s.T * s.Hkv;
  const long ncs = (long)s.T * (s.d / 2), thr = (nq + nk) * (s.d / 16);
  mk.mark(rs);
  hipLaunchKernelGGL(k_rope_cs, dim3((unsigned)((ncs + 255) / 256)), dim3(256), 0, rs, pp.rcs, s.T, s.d / 2, th);
  mk.mark(rs);
  hipLaunchKernelGGL(k_rope<T>, dim3((unsigned)((thr + 255) / 256)), dim3(256), 0, rs, q, k, (T*)pp.qrot,
                     (T*)pp.krot, nq, nk, s.H, s.Hkv, s.T, s.d, (const float2*)pp.rcs);
}

template <typename T, int D, int MP, int C>
static void prologue_impl(const Shape& s, const RopeTheta& th, const T* q, const T* k, const T* v, const T* alpha,
                          const ProloguePtrs& pp, Marks& mk, hipStream_t st, const Fork& fk) {
  if (s.m > 0) {  // (no slots: no gates and no states)
    mk.mark(st);
    launch_gates<T, C, MP>(s, alpha, pp, st);
  }
  if (s.rope && s.win) fk.record(st);
  if (s.m > 0) {
    mk.mark(st);
    launch_scan<T, D, C, MP>(s, k, v, pp, mk, st);
  }
  if (s.rope && s.win) {
    // RoPE (HBM-bound, no LDS) on the side stream beside the state scan (bound
    // by its chain of dependent steps; the gate products, HBM-bound too, run
    // before both), enqueued after the scan so that the scan's workgroups are
    // placed first; joined at the end
    launch_rope<T>(s, th, q, k, pp, mk, fk.follow(st));
    fk.join(st);
  }
}

template <typename T, int D, int MP, int C>
static hipError_t fwd_impl(const Shape& s, const RopeTheta& th, const FwdPtrs& p, hipStream_t st) {
  if constexpr (sizeof(SlotFwdSmem<T, D, MP, C>) > kMaxLds) {
    return hipErrorInvalidConfiguration;
  } else {
    FwdWs L = fwd_ws_layout(s);
    const T* q = (const T*)p.q;
    const T* k = (const T*)p.k;
    const T* v = (const T*)p.v;
    const T* alpha = (const T*)p.alpha;
    const int units = s.B * s.Hkv;
    Marks mk;
    mk.ev = p.events;
    StateLayout SL{};
    ProloguePtrs pp{p.ws + L.sst, p.ws + L.wt, (float*)(p.ws + L.aend), nullptr, nullptr, nullptr, nullptr, nullptr};
    pp.seg = (float*)(p.ws + L.seg);
    pp.s0k = p.s0k;
    pp.s0v = p.s0v;
    if (s.rope && s.win) {
      pp.qrot = p.ws + L.qrot;
      pp.krot = p.ws + L.krot;
      pp.rcs = (float2*)(p.ws + L.rcs);
    }
    if (p.state_out) {
      SL = state_layout(s);
      pp.skout = (float*)((char*)p.state_out + SL.sk);
      pp.svout = (float*)((char*)p.state_out + SL.sv);
    }
    const Fork fk = side_fork(p.events == nullptr && !p.one_stream);
    const T* qr = pp.qrot ? (const T*)pp.qrot : q;
    const T* kr = pp.krot ? (const T*)pp.krot : k;
    // slot branch: its normalised partial and lse (o_w null), or the final
    // output merged with the window branch's partial (o_w, lse_w)
    auto slot = [&](const T* o_w, const float* lse_w, T* out, float* lse_out) {
      mk.mark(st);
      if constexpr (sizeof(T) == 2) {
        hipLaunchKernelGGL((k_slot_fwd_b16<D, MP, C>), dim3(s.NC, s.B * s.H), dim3(C / 16 * 64), 0, st, q, k, v,
                           alpha, (const T*)pp.sst, o_w, lse_w, out, lse_out, s.T, s.H, s.Hkv, s.m, s.sh, s.NC,
                           s.scale);
      } else {
        const int nitems = s.NC * s.B * s.H;
        const int nwg = nitems < device_cu_count() ? nitems : device_cu_count();
        hipLaunchKernelGGL((k_slot_fwd<T, D, MP, C>), dim3(nwg), dim3(C / 16 * 64), 0, st, q, k, v, alpha,
                           (const T*)pp.sst, o_w, lse_w, out, lse_out, s.T, s.H, s.Hkv, s.m, s.sh, s.NC, nitems,
                           s.scale);
      }
    };
    // window branch, started from the slot partial (seed) or an empty softmax
    auto window = [&](hipStream_t ws_, const T* seed, const float* seed_lse, T* out, float* lse_out) {
      mk.mark(ws_);
      if constexpr (sizeof(T) == 2) {
        hipLaunchKernelGGL((k_win_fwd_b16<D, kWinWaves>),
                           dim3((s.T + 32 * kWinWaves - 1) / (32 * kWinWaves), s.B * s.H), dim3(kWinWaves * 64), 0,
                           ws_, qr, kr, v, seed, seed_lse, out, lse_out, s.T, s.H, s.Hkv, s.w, s.scale);
      } else {
        hipLaunchKernelGGL((k_win_fwd<T, D, kWinWaves>),
                           dim3((s.T + 32 * kWinWaves - 1) / (32 * kWinWaves), s.B * s.H), dim3(kWinWaves * 64), 0,
                           ws_, qr, kr, v, seed, seed_lse, out, lse_out, s.T, s.H, s.Hkv, s.w, s.scale);
      }
    };
    if (s.m > 0 && s.win && !p.separate && chunk_fused(s)) {
      // both branches in the chunk kernel, after RoPE, the gate products and
      // the slot-state scan, all in order on the caller's stream: the scan is
      // a latency-bound walk over the chunks, and RoPE beside it on the side
      // stream slowed it by more than RoPE takes alone (RoPE first: the
      // chunk-start states the scan writes last are the freshest in the
      // memory-side cache when the chunk kernel reads them)
      if constexpr (sizeof(T) == 2 && C == 64) {
        if (s.rope) launch_rope<T>(s, th, q, k, pp, mk, st);
        mk.mark(st);
        launch_gates<T, C, MP>(s, alpha, pp, st);
        mk.mark(st);
        launch_scan<T, D, C, MP>(s, k, v, pp, mk, st);
        mk.mark(st);
        hipLaunchKernelGGL((k_chunk_fwd_b16<D, MP>), dim3((s.T + 32 * kWinWaves - 1) / (32 * kWinWaves), s.B * s.H),
                           dim3(kWinWaves * 64), 0, st, q, k, v, alpha, (const T*)pp.sst, qr, kr, (T*)p.o, p.lse,
                           s.T, s.H, s.Hkv, s.m, s.w, s.sh, s.NC, s.scale);
      }
    } else if (s.m > 0 && s.win && !p.separate) {
      // both branches: the window branch (RoPE, then band attention from an
      // empty softmax into the workspace) on the side stream, beside the gate
      // products and the slot-state scan it does not depend on; the slot
      // kernel then merges the two partial softmaxes into o and lse
      T* ow = (T*)(p.ws + L.ol);
      float* lw = (float*)(p.ws + L.lsel);
      fk.record(st);
      mk.mark(st);
      launch_gates<T, C, MP>(s, alpha, pp, st);
      mk.mark(st);
      launch_scan<T, D, C, MP>(s, k, v, pp, mk, st);
      const hipStream_t rs = fk.follow(st);
      if (s.rope) launch_rope<T>(s, th, q, k, pp, mk, rs);
      window(rs, nullptr, nullptr, ow, lw);
      fk.join(st);
      slot(ow, lw, (T*)p.o, p.lse);
    } else if (s.m > 0 && !s.win && !p.separate) {
      // no window: the slot branch is the whole softmax
      prologue_impl<T, D, MP, C>(s, th, q, k, v, alpha, pp, mk, st, fk);
      slot(nullptr, nullptr, (T*)p.o, p.lse);
    } else {
      // no slots (the window alone), or the weighted-fusion ablation (the
      // slot partial to ol_dst, the window's own read to o)
      prologue_impl<T, D, MP, C>(s, th, q, k, v, alpha, pp, mk, st, fk);
      if (s.m > 0)
        slot(nullptr, nullptr, p.ol_dst ? (T*)p.ol_dst : (T*)(p.ws + L.ol),
             p.lsel_dst ? p.lsel_dst : (float*)(p.ws + L.lsel));
      window(st, nullptr, nullptr, (T*)p.o, p.lse);
    }
    if (p.state_out) {
      char* base = (char*)p.state_out;
      mk.mark(st);
      if (s.w > 0)
        hipLaunchKernelGGL(k_export_state<T>, dim3(32, units), dim3(256), 0, st, k, v,
                           s.rope ? (const T*)pp.krot : (const T*)nullptr, (T*)(base + SL.rk), (T*)(base + SL.rv),
                           (T*)(base + SL.rkr), (long long*)(base + SL.pos), s.T, s.Hkv, s.d, s.w, th.pos0);
      else
        hipLaunchKernelGGL(k_export_state<T>, dim3(1, units), dim3(64), 0, st, k, v, (const T*)nullptr,
                           (T*)nullptr, (T*)nullptr, (T*)nullptr, (long long*)(base + SL.pos), s.T, s.Hkv, s.d, 0,
                           th.pos0);
    }
    mk.mark(st);
    return hipGetLastError();
  }
}

template <typename T, int MP, int C>
static void prologue_d(const Shape& s, const RopeTheta& th, const void* q, const void* k, const void* v,
                       const void* alpha, const ProloguePtrs& pp, Marks& mk, hipStream_t st, const Fork& fk) {
  switch (s.d) {
    case 32:
      return prologue_impl<T, 32, MP, C>(s, th, (const T*)q, (const T*)k, (const T*)v, (const T*)alpha, pp, mk, st, fk);
    case 64:
      return prologue_impl<T, 64, MP, C>(s, th, (const T*)q, (const T*)k, (const T*)v, (const T*)alpha, pp, mk, st, fk);
    case 128:
      return prologue_impl<T, 128, MP, C>(s, th, (const T*)q, (const T*)k, (const T*)v, (const T*)alpha, pp, mk, st,
                                          fk);
  }
}
template <typename T, int MP>
static void prologue_c(const Shape& s, const RopeTheta& th, const void* q, const void* k, const void* v,
                       const void* alpha, const ProloguePtrs& pp, Marks& mk, hipStream_t st, const Fork& fk) {
  switch (s.C) {
    case 16: return prologue_d<T, MP, 16>(s, th, q, k, v, alpha, pp, mk, st, fk);
    case 32: return prologue_d<T, MP, 32>(s, th, q, k, v, alpha, pp, mk, st, fk);
    case 64: return prologue_d<T, MP, 64>(s, th, q, k, v, alpha, pp, mk, st, fk);
  }
}
hipError_t launch_prologue(const Shape& s, const RopeTheta& th, const void* q, const void* k, const void* v,
                           const void* alpha, const ProloguePtrs& pp, Marks& mk, hipStream_t st, const Fork& fk) {
  if (s.dtype == NHA_DTYPE_BF16) {
    if (s.mp == 32) prologue_c<bf16, 32>(s, th, q, k, v, alpha, pp, mk, st, fk);
    else prologue_c<bf16, 64>(s, th, q, k, v, alpha, pp, mk, st, fk);
  } else {
    if (s.mp == 32) prologue_c<float, 32>(s, th, q, k, v, alpha, pp, mk, st, fk);
    else prologue_c<float, 64>(s, th, q, k, v, alpha, pp, mk, st, fk);
  }
  return hipGetLastError();
}

template <typename T, int MP, int C>
static hipError_t fwd_d(const Shape& s, const RopeTheta& th, const FwdPtrs& p, hipStream_t st) {
  switch (s.d) {
    case 32: return fwd_impl<T, 32, MP, C>(s, th, p, st);
    case 64: return fwd_impl<T, 64, MP, C>(s, th, p, st);
    case 128: return fwd_impl<T, 128, MP, C>(s, th, p, st);
  }
  return hipErrorInvalidValue;
}
template <typename T, int MP>
static hipError_t fwd_c(const Shape& s, const RopeTheta& th, const FwdPtrs& p, hipStream_t st) {
  switch (s.C) {
    case 16: return fwd_d<T, MP, 16>(s, th, p, st);
    case 32: return fwd_d<T, MP, 32>(s, th, p, st);
    case 64: return fwd_d<T, MP, 64>(s, th, p, st);
  }
  return hipErrorInvalidValue;
}
template <typename T>
static hipError_t fwd_m(const Shape& s, const RopeTheta& th, const FwdPtrs& p, hipStream_t st) {
  if (s.mp == 32) return fwd_c<T, 32>(s, th, p, st);
  return fwd_c<T, 64>(s, th, p, st);
}

hipError_t launch_fwd(const Shape& s, const RopeTheta& th, const FwdPtrs& p, hipStream_t st) {
  if (s.dtype == NHA_DTYPE_BF16) return fwd_m<bf16>(s, th, p, st);
  return fwd_m<float>(s, th, p, st);
}

int fwd_stages(const Shape& s, bool with_state, const char** names, int max) {
  const char* all[12];
  int n = 0;
  const bool fused = s.m > 0 && s.win && chunk_fused(s);
  if (fused && s.rope) {  // the one-kernel form runs RoPE first
    all[n++] = "rope_cs";
    all[n++] = "rope";
  }
  if (s.m > 0) {
    all[n++] = "chunk_gates";
    if (scan_segments(s).n > 1) {
      all[n++] = "state_scan_seg";
      all[n++] = "scan_combine";
    }
    all[n++] = "state_scan";
  }
  if (s.rope && s.win && !fused) {
    all[n++] = "rope_cs";
    all[n++] = "rope";
  }
  if (fused) {
    all[n++] = "chunk_fwd";
  } else {
    if (s.win) all[n++] = "win_fwd";  // (first: the slot kernel merges it)
    if (s.m > 0) all[n++] = "slot_fwd";
  }
  if (with_state) all[n++] = "export_state";
  for (int i = 0; i < n && i < max && names; ++i) names[i] = all[i];
  return n;
}

size_t slot_fwd_lds_bytes(const Shape& s) {
  size_t e = s.esz;
  size_t PD = pitch_of(s.d), PM = pitch_of(s.mp), PC = pitch_of(s.C);
  return e * (s.mp * PD + s.d * PM + s.C * PD + s.d * PC + 2 * s.C * PM + s.mp * PC) + 4 * (size_t)s.C * s.mp;
}

}  // namespace nha
