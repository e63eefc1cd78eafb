// nha_bwd.hip -- backward kernels of the NHA layer operator (gfx950).
//
// Gradients of the forward in nha_fwd.hip: one softmax over the m slot logits
// and the window logits (Paper-Notes page "Native Hybrid Attention for
// Efficient Sequence Modeling", section 关键设计 > 层内混合: the unified softmax
// couples the gradients of the long- and short-term memories).  With p the
// joint probabilities (recomputed from the forward's lse) and D_t = <dO_t, o_t>:
//     dl = p (dp - D_t)
// Window branch (band attention with RoPE):
//     dq_t += R_t^T s sum_j dl_tj R_j k_j,  dk_j += R_j^T s sum_t dl_tj R_t q_t,
//     dv_j += sum_t p_tj dO_t.
// Slot branch, per (batch, KV head): the slot states receive the direct
// sources dSK_t[i] = s dl_ti q_t, dSV_t[i] = p_ti dO_t (summed over the query
// heads of the group), and their adjoint runs backwards in time,
//     Lam_t = dS_t + a_{t+1} Lam_{t+1},
// which is a slot state in reversed time.  Then, for t >= w,
//     dk_{t-w} += sum_i b_t[i] LamK_t[i]        (dv likewise)
//     F_t[i]   = <LamK_t[i], k_{t-w}> + <LamV_t[i], v_{t-w}>
//     A_t[i]   = sum_h dl_ti l_ti + p_ti dp_ti     (l: scaled slot logit)
//     dalpha_t = (sum_{u>=t} (A_u - b_u F_u)) / alpha_t - F_t
// (from <Lam_t, S_t> = A_t + <Lam_{t+1}, S_{t+1}> - b_{t+1} F_{t+1}), and
// dalpha_t = 0 for t < w.  Chunkwise: the adjoint entering chunk c from the
// right obeys Lin_{c-1} = 2^{G_end} Lin_c + sum_{u in c} 2^{G_u} dS_u.
//
// Kernels, in launch order (after the shared prologue: RoPE, gates, state scan):
//   k_bwd_prep      D_t = <dO_t, o_t> (fp32; bf16 computes it in slot pass A)
//   k_bwd_slot_a    per (b, h, chunk): slot p, dp, dl; dq's slot part; A_t
//                   parts; the chunk's adjoint sources sum_u 2^{G_u} dS_u
//                   (fp32: the weights 2^{G_u} s dl_u, 2^{G_u} p_u instead)
//   k_adj_scan      reverse over chunks: Lin_c for every chunk (bf16:
//                   elementwise on pass A's products; fp32: MFMA)
//   k_bwd_slot_b    per (b, g, chunk): dk/dv slot parts, F, local dalpha
//   k_dalpha_tail   dalpha += (sum of the later chunks' (A - b F)) / alpha
//   k_win_bwd_dq    window dq (+ slot part) -> dq
//   k_win_bwd_dkdv  window dk, dv (+ slot parts at the shifted rows) -> dk, dv
#include "nha_common.h"
#include "nha_internal.h"
#include "nha_slot.h"

namespace nha {

// ---------------------------------------------------------------- workspace
struct BwdWs {
  size_t sst, wt, aend, seg, qrot, krot, rcs;  // prologue (same meaning as the forward's)
  size_t dt;                         // D_t: [B][H][T] float
  size_t dqs;                        // slot part of dq: [B][T][H][d] dtype
  size_t wp;                         // fp32: adjoint weights [B*H][NC][2][mp][C]; bf16: the chunk
                                     // products M [B*H][NC][2][d/16][mp][16]
  size_t sdl, pp, acon;              // [B*H][NC*C][mp] float (bf16 inputs: sdl and pp hold
                                     // only the rows of blocks on the exact same-block path)
  size_t sdlh, pph;                  // bf16 inputs: s dl and p as fp16 [B*H][NC*C][mp], every row
  size_t lin;                        // adjoint entering each chunk: [B*Hkv][NC][2][mp x d] dtype
                                     // (fp32 [i][d] rows, bf16 column blocks [d/16][i][16])
  size_t dkap, dnu;                  // slot parts of dk, dv at the key row: [B][T][Hkv][d] dtype
  size_t csum;                       // [B*Hkv][NC][mp] float
  size_t xck;                        // bf16: exact carries at the checkpoint chunks [B*Hkv][(NC-1)/16][mp] float
  size_t total;
};

static BwdWs bwd_ws_layout(const Shape& s) {
  BwdWs L;
  FwdWs F = fwd_ws_layout(s);
  L.sst = F.sst;
  L.wt = F.wt;
  L.aend = F.aend;
  L.seg = F.seg;
  L.qrot = F.qrot;
  L.krot = F.krot;
  L.rcs = F.rcs;
  size_t off = F.ol;  // the forward's partial-output region is not needed here
  const size_t BH = (size_t)s.B * s.H, units = (size_t)s.B * s.Hkv, TT = (size_t)s.NC * s.C;
  L.dt = off;
  off += align256(BH * s.T * 4);
  L.dqs = off;
  off += align256((size_t)s.B * s.T * s.H * s.d * s.esz);
  L.wp = off;
  off += align256(BH * s.NC * 2 * (size_t)s.mp * (s.esz == 2 ? s.d : s.C) * s.esz);
  L.sdl = off;
  off += align256(BH * TT * s.mp * 4);
  L.pp = off;
  off += align256(BH * TT * s.mp * 4);
  L.acon = off;
  off += align256(BH * TT * s.mp * 4);
  L.sdlh = off;
  off += s.esz == 2 ? align256(BH * TT * s.mp * 2) : 0;
  L.pph = off;
  off += s.esz == 2 ? align256(BH * TT * s.mp * 2) : 0;
  L.lin = off;
  off += align256(units * s.NC * 2 * (size_t)s.mp * s.d * s.esz);
  L.dkap = off;
  off += align256((size_t)s.B * s.T * s.Hkv * s.d * s.esz);
  L.dnu = off;
  off += align256((size_t)s.B * s.T * s.Hkv * s.d * s.esz);
  L.csum = off;
  off += align256(units * s.NC * s.mp * 4);
  L.xck = off;
  off += align256(units * (size_t)carry_ckpts(s) * s.mp * 4);
  L.total = off;
  return L;
}

size_t bwd_ws_bytes(const Shape& s) { return bwd_ws_layout(s).total; }

// ---------------------------------------------------------------- D_t
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_prep(const T* __restrict__ o, const T* __restrict__ dO,
                                                  float* __restrict__ Dt, int Tn, int H, long nrows) {
  constexpr int TPR = D / 8;  // threads per row (4, 8 or 16), a divisor of 64
  long gid = (long)blockIdx.x * 256 + threadIdx.x;
  long r = gid / TPR;
  int part = (int)(gid % TPR);
  float acc = 0.f;
  if (r < nrows) {
    float a[8], b[8];
    ld8f<T>(o + r * D + part * 8, a);
    ld8f<T>(dO + r * D + part * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += a[e] * b[e];
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (r < nrows && part == 0) {
    long h = r % H, bt = r / H, t = bt % Tn, b = bt / Tn;
    Dt[(b * H + h) * Tn + t] = acc;
  }
}

// ---------------------------------------------------------------- reverse-time slot products
// For one wave owning chunk rows r0 .. r0+15 (lane: row t = t0 + r0 + cc,
// slots i = 16 mb + 4 g + r) and one query head's sources W[u][i] on rows
// vec_u (sW fp32 [u][i]; sVec [u][d]; sVecT [d][u]), with
//     Lam_t[i] = sum_{u>=t in chunk} 2^{G_u - G_t}[i] W_u[i] vec_u   (+ the
//     incoming adjoint, handled by the caller):
//   accO (O^T[d][t]) += sum_i bt_t[i] Lam_t[i]
//   F[mb][r]         += <Lam_t[i], key_t>
// Cross-block pairs refer to F_I = G at the last row of the wave's block.
//
// With a pair table pf (bf16), sW holds the block-referenced weights
// W_u[i] 2^{G_u - E_{J-1}} (u in block J; E_J = G at the last row of block J,
// E_{-1} = 0; <= 1) and pf[pair_index(I, J)][i] = 2^{E_{J-1} - E_I}, so the
// factor 2^{G_u - E_I} of a source row is one product of two LDS values; the
// exact same-block path then reads the unscaled weights from wg (rows of MP
// floats in global memory).  Without it (fp32) sW holds W itself.
template <int NW>
__host__ __device__ constexpr int pair_index(int I, int J) {
  return I * NW - I * (I - 1) / 2 + (J - I);
}

template <typename T, int D, int MP, int C>
__device__ __forceinline__ void slot_rev(const T* sVec, const T* sVecT, const float* sW, const float* sG,
                                         const T* sA, const float* pf, const float* wg,
                                         const typename Vec<T>::v8* keyf,
                                         const float (&bwI)[MP / 16][4], const float (&bt)[MP / 16][4], int I,
                                         int t0, int w, int Tn, floatx4 (&accO)[D / 16], float (&F)[MP / 16][4]) {
  constexpr int NW = C / 16, NB = MP / 16, PD = pitch_of(D), PM = pitch_of(MP), PC = pitch_of(C);
  constexpr int PG = SlotPitch<MP>::PG;
  constexpr bool TAB = sizeof(T) == 2;
  const int l = threadIdx.x & 63, g = l >> 4, cc = l & 15, r0 = 16 * I, urow = r0 + cc, rl = r0 + 15;
  // later blocks J > I, and (when factorizable) the block itself with u >= t;
  // one block per iteration (not unrolled: the blocks are independent and
  // unrolling only multiplies the live registers)
  const bool fast = block_factorizable<MP>(sG, r0);
  floatx4 aI = zero4();  // A[u][t] = vec_u . key_t for the wave's own block (exact path)
  // sum over the blocks of Y^T A; its factor 2^{G_rl - G_t} does not depend on
  // the block and is applied once after the loop
  floatx4 xs[NB];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) xs[mb] = zero4();
#pragma unroll 1
  for (int J = I; J < NW; ++J) {
    floatx4 aJ = zero4();  // D layout [u = 16J + 4g + r][t = cc]
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      aJ = mma32(aJ, ld8<T>(&sVec[(16 * J + cc) * PD + 32 * ks + 8 * g]), keyf[ks]);
    if (J == I) aI = aJ;
    if (J > I || fast) {
      const int uA = 16 * J + cc;  // A-fragment row of this lane
      const float* pj = TAB ? pf + pair_index<NW>(I, J) * MP : nullptr;
      floatx4 mt = zero4();        // M^T[u][t] = sum_i Y[u][i] bwI[t][i]
#pragma unroll
      for (int s = 0; s < NB / 2; ++s) {
        float f[8];
        if constexpr (TAB) {
          const floatx4 p0 = *reinterpret_cast<const floatx4*>(&pj[32 * s + 4 * g]);
          const floatx4 p1 = *reinterpret_cast<const floatx4*>(&pj[32 * s + 16 + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int i0 = 32 * s + 4 * g + r, i1 = i0 + 16;
            f[r] = sW[uA * PG + i0] * p0[r];
            f[4 + r] = sW[uA * PG + i1] * p1[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int i0 = 32 * s + 4 * g + r, i1 = i0 + 16;
            f[r] = sW[uA * PG + i0] * fast_exp2(sG[uA * PG + i0] - sG[rl * PG + i0]);
            f[4 + r] = sW[uA * PG + i1] * fast_exp2(sG[uA * PG + i1] - sG[rl * PG + i1]);
          }
        }
        typename Vec<T>::v8 bfr = pack8<T>(floatx4{bwI[2 * s][0], bwI[2 * s][1], bwI[2 * s][2], bwI[2 * s][3]},
                                           floatx4{bwI[2 * s + 1][0], bwI[2 * s + 1][1], bwI[2 * s + 1][2],
                                                   bwI[2 * s + 1][3]});
        mt = mma32(mt, pack8<T>(f), bfr);
      }
      if (J == I) {
#pragma unroll
        for (int r = 0; r < 4; ++r) mt[r] = (4 * g + r >= cc) ? mt[r] : 0.f;  // u >= t
      }
      typename Vec<T>::v4 mfr = pack4<T>(mt);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        typename Vec<T>::v4 at;
        if constexpr (sizeof(T) == 2)
          at = ld_tr4(&sVec[(16 * J + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
        else
          at = ld4<T>(&sVecT[(16 * db + cc) * PC + 16 * J + 4 * g]);
        accO[db] = mma16(accO[db], at, mfr);
      }
      floatx4 av = aJ;
      if (J == I) {
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = (4 * g + r >= cc) ? av[r] : 0.f;  // u >= t
      }
      typename Vec<T>::v4 afr = pack4<T>(av);
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        const int iA = 16 * mb + cc;
        floatx4 y;
        if constexpr (TAB) {
          const float pa = pj[iA];
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = sW[(16 * J + 4 * g + r) * PG + iA] * pa;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int u = 16 * J + 4 * g + r;
            y[r] = sW[u * PG + iA] * fast_exp2(sG[u * PG + iA] - sG[rl * PG + iA]);
          }
        }
        xs[mb] = mma16(xs[mb], pack4<T>(y), afr);
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * mb + 4 * g + r;
      F[mb][r] += fast_exp2(sG[rl * PG + i] - sG[urow * PG + i]) * xs[mb][r];
    }
  if (fast) return;
  // same block: u >= t, exact running products D'_{t,u} = prod_{j=t+1..u} a_j
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
  float mine[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int uu = 0; uu < 16; ++uu) {
    float mp = 0.f;
    if (uu >= cc) {
      const int u = r0 + uu;
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        floatx4 w4;
        if constexpr (TAB) {
          w4 = *reinterpret_cast<const floatx4*>(wg + (size_t)u * MP + 16 * mb + 4 * g);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) w4[r] = sW[u * PG + 16 * mb + 4 * g + r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          F[mb][r] += Dp[mb][r] * w4[r] * Ad[uu];
          mp += bt[mb][r] * Dp[mb][r] * w4[r];
        }
      }
      if (uu < 15) {
        const int u1 = u + 1, t1 = t0 + u1;
        const bool ab1 = (t1 >= w) && (t1 < Tn);
#pragma unroll
        for (int mb = 0; mb < NB; ++mb) {
          typename Vec<T>::v4 al = ld4<T>(&sA[u1 * PM + 16 * mb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) Dp[mb][r] *= ab1 ? to_f<T>(al[r]) : 1.f;
        }
      }
    }
    mp = sum_over_g(mp);
    if ((uu >> 2) == g) mine[uu & 3] = mp;
  }
  typename Vec<T>::v4 bfr;
#pragma unroll
  for (int r = 0; r < 4; ++r) bfr[r] = to_t<T>(mine[r]);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    typename Vec<T>::v4 at;
    if constexpr (sizeof(T) == 2)
      at = ld_tr4(&sVec[(r0 + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
    else
      at = ld4<T>(&sVecT[(16 * db + cc) * PC + r0 + 4 * g]);
    accO[db] = mma16(accO[db], at, bfr);
  }
}

// In-place reverse inclusive cumsum over the C rows of an LDS tile (fp32).
template <int C, int MP, int P, int NT>
__device__ __forceinline__ void lds_col_rcumsum(float* g, int tid) {
  constexpr int PARTS = (NT / MP) < C ? (NT / MP) : C;
  constexpr int RP = C / PARTS;
  const int i = tid % MP, part = tid / MP;
  const bool act = part < PARTS;
  if (act) {
    float acc = 0.f;
#pragma unroll
    for (int u = (part + 1) * RP - 1; u >= part * RP; --u) {
      acc += g[u * P + i];
      g[u * P + i] = acc;
    }
  }
  __syncthreads();
  float off = 0.f;
  if (act)
    for (int pp = part + 1; pp < PARTS; ++pp) off += g[(pp * RP) * P + i];
  __syncthreads();
  if (act && part + 1 < PARTS) {
#pragma unroll
    for (int u = part * RP; u < (part + 1) * RP; ++u) g[u * P + i] += off;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- slot pass A
template <typename T, int D, int MP, int C>
struct SlotBwdASmem {
  static constexpr int PD = pitch_of(D), PM = pitch_of(MP), PC = pitch_of(C);
  T sSK[MP * PD];   // S^K_{t0-1} [i][d]
  T sSKt[D * PM];   // S^K_{t0-1}^T [d][i]
  T sSV[MP * PD];   // S^V_{t0-1} [i][d]
  T sK[C * PD];     // kappa rows [u][d]
  T sKt[D * PC];    // kappa^T [d][u]
  T sV[C * PD];     // nu rows [u][d]
  T sA[C * PM];
  T sB[C * PM];
  T sBt[MP * PC];
  float sG[C * SlotPitch<MP>::PG];
};

template <typename T, int D, int MP, int C, int NT>
struct SlotBwdARegs {
  static constexpr int NG = (C * MP + NT - 1) / NT;
  RowTile<T, D, NT, MP> tsk, tsv;
  PairTileT<T, D, NT, MP> tskt;
  RowTile<T, D, NT, C> tk, tv;
  PairTileT<T, D, NT, C> tkt;
  T al[NG];
};

// grid: a persistent set of workgroups (about one per compute unit), C/16
// waves each, looping over the items (chunk c, head b*H + h) with the next
// item's operands loaded while the current one is computed.
template <typename T, int D, int MP, int C>
__global__ __launch_bounds__(C / 16 * 64) void k_bwd_slot_a(
    const T* __restrict__ q, const T* __restrict__ kk, const T* __restrict__ vv, const T* __restrict__ alpha,
    const T* __restrict__ dO, const T* __restrict__ sst, const float* __restrict__ lse,
    const float* __restrict__ Dt, T* __restrict__ dqs, T* __restrict__ wp, float* __restrict__ sdl,
    float* __restrict__ pp, float* __restrict__ acon, int Tn, int H, int Hkv, int m, int w, int NC, int nitems,
    float scale) {
  using S = SlotBwdASmem<T, D, MP, C>;
  constexpr int NT = C / 16 * 64, NB = MP / 16, PD = S::PD, PM = S::PM, PC = S::PC;
  constexpr int PG = SlotPitch<MP>::PG;
  using R_t = SlotBwdARegs<T, D, MP, C, NT>;
  __shared__ S sm;
  const int tid = threadIdx.x, I = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  const int G = H / Hkv;
  R_t R;
  auto load = [&](int n) {
    const int c = n % NC, bh = n / NC, b = bh / H, hg = (bh % H) / G, unit = b * Hkv + hg, t0 = c * C;
    const T* src = sst + ((size_t)unit * NC + c) * 2 * MP * D;
    R.tsk.load(src, D, 0, MP, tid);
    R.tskt.load(src, D, 0, MP, tid);
    R.tsv.load(src + (size_t)MP * D, D, 0, MP, tid);
    const long rbase = ((long)b * Tn + (t0 - w)) * Hkv + hg;
    R.tk.load(kk + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
    R.tkt.load(kk + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
    R.tv.load(vv + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
#pragma unroll
    for (int k = 0; k < R_t::NG; ++k) {
      const int e = tid + k * NT, u = e / MP, i = e % MP, t = t0 + u;
      R.al[k] = (e < C * MP && i < m && t < Tn) ? alpha[(((size_t)b * Tn + t) * Hkv + hg) * m + i] : to_t<T>(1.f);
    }
  };
  if ((int)blockIdx.x < nitems) load(blockIdx.x);
  for (int n = blockIdx.x; n < nitems; n += gridDim.x) {
  const int c = n % NC, bh = n / NC, b = bh / H, h = bh % H;
  const int t0 = c * C;
  __syncthreads();  // the previous item's LDS reads are done
  R.tsk.template store<PD>(sm.sSK, tid);
  R.tskt.template store<PM>(sm.sSKt, tid);
  R.tsv.template store<PD>(sm.sSV, tid);
  R.tk.template store<PD>(sm.sK, tid);
  R.tkt.template store<PC>(sm.sKt, tid);
  R.tv.template store<PD>(sm.sV, tid);
#pragma unroll
  for (int k = 0; k < R_t::NG; ++k) {
    const int e = tid + k * NT, u = e / MP, i = e % MP, t = t0 + u;
    if (e < C * MP) {
      sm.sA[u * PM + i] = R.al[k];
      sm.sG[u * PG + i] = (i < m && t < Tn && t >= w) ? fmaxf(__log2f(to_f<T>(R.al[k])), NHA_LOG2A_MIN) : 0.f;
    }
  }
  __syncthreads();
  if (n + (int)gridDim.x < nitems) load(n + gridDim.x);  // in flight during this item
  lds_col_cumsum<C, MP, PG, NT>(sm.sG, tid);
  for (int e = tid; e < C * MP; e += NT) {
    int u = e / MP, i = e % MP, t = t0 + u;
    float be = (i < m && t < Tn && t >= w) ? 1.f - to_f<T>(sm.sA[u * PM + i]) : 0.f;
    T tv = to_t<T>(fast_exp2(sm.sG[(u | 15) * PG + i] - sm.sG[u * PG + i]) * be);
    sm.sB[u * PM + i] = tv;
    sm.sBt[i * PC + u] = tv;
  }
  __syncthreads();

  const int r0 = 16 * I, urow = r0 + cc, tq = t0 + urow;
  const bool qvalid = tq < Tn;
  const int tqc = qvalid ? tq : Tn - 1;  // clamped row: loads stay unconditional
  typename Vec<T>::v8 qf[D / 32], df[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const size_t off = (((size_t)b * Tn + tqc) * H + h) * D + 32 * ks + 8 * g;
    qf[ks] = ld8_sel<T>(q + off, qvalid);
    df[ks] = ld8_sel<T>(dO + off, qvalid);
  }
  const float lse_r = lse[(size_t)bh * Tn + tqc], lse_t = qvalid ? lse_r : 0.f;
  const float D_r = Dt[(size_t)bh * Tn + tqc], D_t = qvalid ? D_r : 0.f;
  float lg[NB][4], dp[NB][4];
  slot_read<T, D, MP, C>(sm.sSK, sm.sK, sm.sBt, sm.sG, sm.sA, qf, I, t0, w, Tn, lg);
  slot_read<T, D, MP, C>(sm.sSV, sm.sV, sm.sBt, sm.sG, sm.sA, df, I, t0, w, Tn, dp);
  float p[NB][4], dl[NB][4];
  float* sdl_row = sdl + ((size_t)bh * NC * C + urow + t0) * MP;
  float* pp_row = pp + ((size_t)bh * NC * C + urow + t0) * MP;
  float* ac_row = acon + ((size_t)bh * NC * C + urow + t0) * MP;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    floatx4 vs, vp, va;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int i = 16 * mb + 4 * g + r;
      float ls = lg[mb][r] * scale;
      float pv = (i < m && qvalid) ? fast_exp2((ls - lse_t) * NHA_LOG2E) : 0.f;
      float dlv = pv * (dp[mb][r] - D_t);
      p[mb][r] = pv;
      dl[mb][r] = dlv;
      vs[r] = scale * dlv;
      vp[r] = pv;
      va[r] = dlv * ls + pv * dp[mb][r];
    }
    *reinterpret_cast<floatx4*>(sdl_row + 16 * mb + 4 * g) = vs;
    *reinterpret_cast<floatx4*>(pp_row + 16 * mb + 4 * g) = vp;
    *reinterpret_cast<floatx4*>(ac_row + 16 * mb + 4 * g) = va;
  }
  // slot part of dq: s sum_i dl_t[i] SK_t[i]
  floatx4 accO[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) accO[db] = zero4();
  slot_mix<T, D, MP, C, PC>(sm.sSKt, sm.sKt, sm.sB, sm.sG, sm.sA, dl, I, t0, w, Tn, accO);
  if (qvalid) {
    T* dst = dqs + (((size_t)b * Tn + tq) * H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) st4<T>(dst + 16 * db + 4 * g, pack4<T>(accO[db] * scale));
  }
  // adjoint weights 2^{G_u} s dl_u[i] and 2^{G_u} p_u[i], [i][u] layout
  T* wk = wp + (((size_t)bh * NC + c) * 2) * MP * C;
  T* wv = wk + (size_t)MP * C;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int i = 16 * mb + 4 * g + r;
      float e = fast_exp2(sm.sG[urow * PG + i]);
      wk[(size_t)i * C + urow] = to_t<T>(e * scale * dl[mb][r]);
      wv[(size_t)i * C + urow] = to_t<T>(e * p[mb][r]);
    }
  }
}

// bf16 variant: grid (NC, B*H), C/16 waves, two workgroups per compute unit.
// One pair of LDS row tiles holds S0^V and nu (for dp), then S0^K and kappa
// (for the logits and dq's slot part: their transposes are read with
// ds_read_b64_tr_b16); the second pair's loads are in flight during dp.
template <int D, int MP, int C>
struct SlotBwdASmemB16 {
  static constexpr int PD = pitch_of(D), PM = pitch_of(MP);
  bf16 tS[MP * PD];  // S0^V, then S0^K  [i][d]
  bf16 tK[C * PD];   // nu, then kappa   [u][d]
  bf16 sA[C * PM];
  bf16 sB[C * PM];   // 2^{E_J - G_u} b_u [u][i]
  float sG[C * SlotPitch<MP>::PG];
  SlotTab<C, MP> tab;
};

template <int D, int MP, int C>
__global__ __launch_bounds__(C / 16 * 64, 2) void k_bwd_slot_a_b16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ vv,
    const bf16* __restrict__ alpha, const bf16* __restrict__ dO, const bf16* __restrict__ o,
    const bf16* __restrict__ sst, const float* __restrict__ lse, float* __restrict__ Dt, bf16* __restrict__ dqs,
    bf16* __restrict__ madj,
    float* __restrict__ sdl, float* __restrict__ pp, float* __restrict__ acon, f16* __restrict__ sdlh,
    f16* __restrict__ pph, int Tn, int H, int Hkv, int m, int w, int NC, float scale) {
  using S = SlotBwdASmemB16<D, MP, C>;
  constexpr int NT = C / 16 * 64, NB = MP / 16, PD = S::PD, PM = S::PM;
  constexpr int PG = SlotPitch<MP>::PG;
  __shared__ S sm;
  const int tid = threadIdx.x, I = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int c = L % NC, bh = L / NC, b = bh / H, h = bh % H, hg = h / (H / Hkv);
  const int unit = b * Hkv + hg, t0 = c * C;
  const bf16* src = sst + ((size_t)unit * NC + c) * 2 * MP * D;
  const long rbase = ((long)b * Tn + (t0 - w)) * Hkv + hg;
  const int r0 = 16 * I, urow = r0 + cc, tq = t0 + urow;
  const bool qvalid = tq < Tn;
  const int tqc = qvalid ? tq : Tn - 1;  // clamped row: loads stay unconditional
  // this lane's q, dO and o rows and lse go out with the first tiles: the
  // slot reads then wait on no global load, and the second pair of tiles
  // (issued after the first barrier) stays in flight while they run
  bf16x8 qf[D / 32], df[D / 32], of[D / 32];
  float lse_r;
  {
    GateTile<bf16, C, MP, NT> gt;
    BlockedTile<bf16, D, NT, MP> ts;
    RowTile<bf16, D, NT, C> tk;
    gt.load(alpha, b, hg, t0, Tn, Hkv, m, tid);
    ts.load(src + (size_t)MP * D, tid);
    tk.load(vv + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const size_t off = (((size_t)b * Tn + tqc) * H + h) * D + 32 * ks + 8 * g;
      qf[ks] = ld8_sel<bf16>(q + off, qvalid);
      df[ks] = ld8_sel<bf16>(dO + off, qvalid);
      of[ks] = ld8<bf16>(o + off);
    }
    lse_r = lse[(size_t)bh * Tn + tqc];
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
  // this wave's block may go through pass B's exact same-block path (the
  // same test, at -16, on the same cumulative gates there; -15.75 here
  // leaves room for last-bit differences): its rows of s dl and p are also
  // written in fp32, which that path reads
  const bool exact_blk = !block_factorizable<MP>(sm.sG, r0, -15.75f);
  BlockedTile<bf16, D, NT, MP> tsk;
  RowTile<bf16, D, NT, C> tkap;
  tsk.load(src, tid);
  tkap.load(kk + rbase * D, (size_t)Hkv * D, w - t0, Tn - t0, tid);
  const float lse_t = qvalid ? lse_r : 0.f;
  // D_t = <dO_t, o_t>: the four lanes of a query hold a quarter of the row
  // each; written here for the window kernels
  float D_t = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) D_t += (float)df[ks][e] * (float)of[ks][e];
  D_t = sum_over_g(D_t);
  if (qvalid && g == 0) Dt[(size_t)bh * Tn + tq] = D_t;
  float lg[NB][4], dp[NB][4];
  slot_read<bf16, D, MP, C, true>(sm.tS, sm.tK, sm.sB, sm.sG, sm.sA, df, I, t0, w, Tn, dp, &sm.tab);
  __syncthreads();  // every wave is done with S0^V and nu
  tsk.template store<PD>(sm.tS, tid);
  tkap.template store<PD>(sm.tK, tid);
  __syncthreads();
  slot_read<bf16, D, MP, C, true>(sm.tS, sm.tK, sm.sB, sm.sG, sm.sA, qf, I, t0, w, Tn, lg, &sm.tab);
  float p[NB][4], dl[NB][4];
  const size_t wrow = ((size_t)bh * NC * C + urow + t0) * MP;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    floatx4 vs, vp, va;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * mb + 4 * g + r;
      const float ls = lg[mb][r] * scale;
      const float pv = (i < m && qvalid) ? fast_exp2((ls - lse_t) * NHA_LOG2E) : 0.f;
      const float dlv = pv * (dp[mb][r] - D_t);
      p[mb][r] = pv;
      dl[mb][r] = dlv;
      vs[r] = scale * dlv;
      vp[r] = pv;
      va[r] = dlv * ls + pv * dp[mb][r];
    }
    const size_t e = wrow + 16 * mb + 4 * g;
    *reinterpret_cast<f16x4*>(sdlh + e) = __builtin_convertvector(vs, f16x4);
    *reinterpret_cast<f16x4*>(pph + e) = __builtin_convertvector(vp, f16x4);
    if (exact_blk) {
      *reinterpret_cast<floatx4*>(sdl + e) = vs;
      *reinterpret_cast<floatx4*>(pp + e) = vp;
    }
    *reinterpret_cast<floatx4*>(acon + e) = va;
  }
  // slot part of dq: s sum_i dl_t[i] SK_t[i]
  floatx4 accO[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) accO[db] = zero4();
  slot_mix<bf16, D, MP, C, PD, true>(sm.tS, sm.tK, sm.sB, sm.sG, sm.sA, dl, I, t0, w, Tn, accO, &sm.tab);
  if (qvalid) {
    bf16* dst = dqs + (((size_t)b * Tn + tq) * H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) st4<bf16>(dst + 16 * db + 4 * g, pack4<bf16>(accO[db] * scale));
  }
  // The chunk's part of the adjoint recurrence, for the reverse scan:
  //   M^K[i][:] = sum_u 2^{G_u} s dl_u[i] q_u,   M^V[i][:] = sum_u 2^{G_u} p_u[i] dO_u
  // (the weights and this lane's q / dO row go into LDS -- the row tiles are
  // free once every wave is done -- then each wave takes some of the 16 x 16
  // output blocks of M^T, a product over the chunk's rows).  Stored like the
  // adjoint itself: per side, column blocks [d/16][i][16].
  float ew[NB][4];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) ew[mb][r] = fast_exp2(sm.sG[urow * PG + 16 * mb + 4 * g + r]);
  __syncthreads();
  constexpr int PW = C + 8;  // row pitch of the [i][u] weight tiles
  static_assert(2 * MP * PW * sizeof(bf16) + 2 * C * PD * sizeof(bf16) <= sizeof(S),
                "weight and row tiles fit the shared tiles");
  bf16* tw_k = reinterpret_cast<bf16*>(&sm);
  bf16* tw_v = tw_k + MP * PW;
  bf16* tq_ = tw_v + MP * PW;  // q rows [u][d]
  bf16* td_ = tq_ + C * PD;    // dO rows
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * mb + 4 * g + r;
      tw_k[i * PW + urow] = (bf16)(ew[mb][r] * scale * dl[mb][r]);
      tw_v[i * PW + urow] = (bf16)(ew[mb][r] * p[mb][r]);
    }
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    *reinterpret_cast<bf16x8*>(&tq_[urow * PD + 32 * ks + 8 * g]) = qf[ks];
    *reinterpret_cast<bf16x8*>(&td_[urow * PD + 32 * ks + 8 * g]) = df[ks];
  }
  __syncthreads();
  bf16* mout = madj + ((size_t)bh * NC + c) * 2 * MP * D;
  constexpr int NW = C / 16, NTILE = 2 * (D / 16) * NB;
  for (int tt = I; tt < NTILE; tt += NW) {
    const int side = tt / ((D / 16) * NB), db = (tt / NB) % (D / 16), nb = tt % NB;
    const bf16* vec = side ? td_ : tq_;
    const bf16* wt = side ? tw_v : tw_k;
    const int i = 16 * nb + cc;
    floatx4 acc = zero4();  // M^T[16 db + 4 g + r][16 nb + cc]
    if constexpr (C % 32 != 0) {
#pragma unroll
      for (int s16 = 0; s16 < C / 16; ++s16) {
        const bf16x4 a = ld_tr4(&vec[(16 * s16 + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
        acc = mma16(acc, a, *reinterpret_cast<const bf16x4*>(&wt[i * PW + 16 * s16 + 4 * g]));
      }
    } else {
#pragma unroll
      for (int s32 = 0; s32 < C / 32; ++s32) {
        const bf16* ap = &vec[(32 * s32 + 8 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)];
        const bf16x4 a0 = ld_tr4(ap), a1 = ld_tr4(ap + 4 * PD);
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = a0[e];
          a[4 + e] = a1[e];
        }
        acc = mma32(acc, a, *reinterpret_cast<const bf16x8*>(&wt[i * PW + 32 * s32 + 8 * g]));
      }
    }
    st4<bf16>(mout + (size_t)side * MP * D + (size_t)db * MP * 16 + i * 16 + 4 * g, pack4<bf16>(acc));
  }
}

// ---------------------------------------------------------------- adjoint scan
// grid (d/16, B*Hkv), one wave.  Lane keeps Lam^T[j0 + 4g + r][16 nb + c] for
// K and V.  Chunks in reverse: store Lin_c (the adjoint entering chunk c from
// the right, [i][d] layout), then Lam <- aend (.) Lam + sum_h W'_h^T vec_h.
template <typename T, int C, int MP>
__global__ __launch_bounds__(64) void k_adj_scan(const T* __restrict__ q, const T* __restrict__ dO,
                                                 const T* __restrict__ wp, const float* __restrict__ aend,
                                                 T* __restrict__ lin, float* __restrict__ ds0k,
                                                 float* __restrict__ ds0v, int Tn, int H, int Hkv, int d, int m,
                                                 int NC) {
  constexpr int NB = MP / 16;
  constexpr int PC = pitch_of(C);
  constexpr bool K16 = (C % 32) != 0;
  __shared__ T sQt[16 * PC];
  __shared__ T sOt[16 * PC];
  const int l = threadIdx.x, g = l >> 4, cc = l & 15;
  // the d/16 column blocks of one unit share the adjoint weights: one XCD
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int j0 = (L % gridDim.x) * 16, unit = L / gridDim.x, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  floatx4 LK[NB], LV[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) LK[nb] = LV[nb] = zero4();
  for (int c = NC - 1; c >= 0; --c) {
    T* dst = lin + ((size_t)unit * NC + c) * 2 * MP * d;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int i = 16 * nb + cc;
      st4<T>(dst + (size_t)i * d + j0 + 4 * g, pack4<T>(LK[nb]));
      st4<T>(dst + (size_t)MP * d + (size_t)i * d + j0 + 4 * g, pack4<T>(LV[nb]));
      float a = aend[((size_t)unit * NC + c) * MP + i];
      LK[nb] *= a;
      LV[nb] *= a;
    }
    for (int hh = 0; hh < G; ++hh) {
      const int h = hg * G + hh, bh = b * H + h;
      if (l < C) {
        int t = c * C + l;
        typename Vec<T>::v8 q0 = zero8<T>(), q1 = zero8<T>(), o0 = zero8<T>(), o1 = zero8<T>();
        if (t < Tn) {
          size_t row = (((size_t)b * Tn + t) * H + h) * d + j0;
          q0 = ld8<T>(q + row);
          q1 = ld8<T>(q + row + 8);
          o0 = ld8<T>(dO + row);
          o1 = ld8<T>(dO + row + 8);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sQt[e * PC + l] = q0[e];
          sQt[(8 + e) * PC + l] = q1[e];
          sOt[e * PC + l] = o0[e];
          sOt[(8 + e) * PC + l] = o1[e];
        }
      }
      __syncthreads();
      const T* wk = wp + (((size_t)bh * NC + c) * 2) * MP * C;
      const T* wv = wk + (size_t)MP * C;
      if constexpr (K16) {
#pragma unroll
        for (int s = 0; s < C / 16; ++s) {
          typename Vec<T>::v4 aq = ld4<T>(&sQt[cc * PC + 16 * s + 4 * g]);
          typename Vec<T>::v4 ao = ld4<T>(&sOt[cc * PC + 16 * s + 4 * g]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            LK[nb] = mma16(LK[nb], aq, ld4<T>(wk + (size_t)(16 * nb + cc) * C + 16 * s + 4 * g));
            LV[nb] = mma16(LV[nb], ao, ld4<T>(wv + (size_t)(16 * nb + cc) * C + 16 * s + 4 * g));
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < C / 32; ++s) {
          typename Vec<T>::v8 aq = ld8<T>(&sQt[cc * PC + 32 * s + 8 * g]);
          typename Vec<T>::v8 ao = ld8<T>(&sOt[cc * PC + 32 * s + 8 * g]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            LK[nb] = mma32(LK[nb], aq, ld8<T>(wk + (size_t)(16 * nb + cc) * C + 32 * s + 8 * g));
            LV[nb] = mma32(LV[nb], ao, ld8<T>(wv + (size_t)(16 * nb + cc) * C + 32 * s + 8 * g));
          }
        }
      }
      __syncthreads();
    }
  }
  // the adjoint carried to before the first token: the initial states' gradient
  store_slot_state<NB>(LK, LV, ds0k, ds0v, unit, m, d, j0, g, cc);
}

// bf16 variant on the chunk products M of slot pass A: each step is
// elementwise, Lin_{c-1} = aend_c (.) Lin_c + sum_h M_{c,h}, over contiguous
// rows.  grid (ceil(2 mp d / 2048), B*Hkv), 256 threads; a thread keeps 8
// consecutive elements of one (side, column block, slot) row of the adjoint
// in fp32 and walks the chunks in reverse (the group's heads inside a chunk),
// its loads PF steps ahead in registers.
template <int MP>
__global__ __launch_bounds__(256) void k_adj_scan_m(const bf16* __restrict__ madj, const float* __restrict__ aend,
                                                    bf16* __restrict__ lin, float* __restrict__ ds0k,
                                                    float* __restrict__ ds0v, int H, int Hkv, int d, int m, int NC) {
  constexpr int PF = 8;
  const int unit = blockIdx.y, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  const int E = 2 * MP * d;  // adjoint elements per (unit, chunk): [2][d/16][mp][16]
  const int x0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (x0 >= E) return;  // (no barriers below)
  const int side = x0 / (MP * d), rr = x0 % (MP * d), db = rr / (MP * 16), i = (rr / 16) % MP, col = rr % 16;
  const int nsteps = NC * G;
  bf16x8 mr[PF];
  float ar[PF];
  auto load = [&](int n, int k) {
    n = min(n, nsteps - 1);
    const int c = NC - 1 - n / G, hh = n % G;
    mr[k] = ld8<bf16>(madj + ((size_t)(b * H + hg * G + hh) * NC + c) * E + x0);
    ar[k] = aend[((size_t)unit * NC + c) * MP + i];
  };
#pragma unroll
  for (int k = 0; k < PF; ++k) load(k, k);
  float La[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) La[e] = 0.f;
  for (int n0 = 0; n0 < nsteps; n0 += PF) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int n = n0 + k;
      if (n < nsteps) {
        const int c = NC - 1 - n / G;
        if (n % G == 0) {
          // the adjoint entering chunk c from the right
          st8<bf16>(lin + ((size_t)unit * NC + c) * E + x0,
                    pack8<bf16>(floatx4{La[0], La[1], La[2], La[3]}, floatx4{La[4], La[5], La[6], La[7]}));
#pragma unroll
          for (int e = 0; e < 8; ++e) La[e] *= ar[k];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) La[e] += (float)mr[k][e];
        load(n + PF, k);
      }
    }
  }
  // the adjoint carried to before the first token: the initial states' gradient
  if (ds0k && i < m) {
    float* dst = (side ? ds0v : ds0k) + ((size_t)unit * m + i) * d + 16 * db + col;
    *reinterpret_cast<floatx4*>(dst) = floatx4{La[0], La[1], La[2], La[3]};
    *reinterpret_cast<floatx4*>(dst + 4) = floatx4{La[4], La[5], La[6], La[7]};
  }
}

// ---------------------------------------------------------------- slot pass B
template <typename T, int D, int MP, int C>
struct SlotBwdBSmem {
  static constexpr int PD = pitch_of(D), PM = pitch_of(MP), PC = pitch_of(C);
  // bf16 reads the transposed operands straight from the row tiles
  // (ds_read_b64_tr_b16); fp32 keeps transposed copies
  static constexpr bool TR = sizeof(T) == 2;
  T sL[MP * PD];                   // incoming adjoint Lin [i][d]
  T sLt[TR ? 8 : D * PM];          // Lin^T [d][i] (fp32 only)
  T sVec[C * PD];                  // q or dO rows of one head [u][d]
  T sVecT[TR ? 8 : D * PC];        // same, transposed (fp32 only)
  T sA[C * PM];
  float sG[C * SlotPitch<MP>::PG];
  float sW[C * SlotPitch<MP>::PG];  // s dl or p of one head [u][i]; later the (A - bF) tile
  // bf16: the block-pair decay factors 2^{E_{J-1} - E_I} (J >= I) of slot_rev
  alignas(16) float pf[TR ? (C / 16) * (C / 16 + 1) / 2 : 1][MP];
};

// grid (NC, B*Hkv), C/16 waves; all query heads of the KV group.
template <typename T, int D, int MP, int C>
__global__ __launch_bounds__(C / 16 * 64, sizeof(T) == 2 ? 2 : 1) void k_bwd_slot_b(
    const T* __restrict__ q, const T* __restrict__ kk, const T* __restrict__ vv, const T* __restrict__ alpha,
    const T* __restrict__ dO, const T* __restrict__ lin, const float* __restrict__ sdl,
    const float* __restrict__ pp, const float* __restrict__ acon, const f16* __restrict__ sdlh,
    const f16* __restrict__ pph, T* __restrict__ dkap, T* __restrict__ dnu, float* __restrict__ dalpha,
    float* __restrict__ csum, int Tn, int H, int Hkv, int m, int w, int NC) {
  using S = SlotBwdBSmem<T, D, MP, C>;
  constexpr int NT = C / 16 * 64, NB = MP / 16, PD = S::PD, PM = S::PM, PC = S::PC;
  constexpr int PG = SlotPitch<MP>::PG;
  __shared__ S sm;
  const int tid = threadIdx.x, I = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  const int c = blockIdx.x, unit = blockIdx.y, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv, t0 = c * C;
  const int r0 = 16 * I, urow = r0 + cc, tq = t0 + urow;
  const bool absorb = (tq >= w) && (tq < Tn);
  // one query head's source rows (q or dO) and fp32 weights (s dl or p),
  // loaded into registers and then written to LDS
  constexpr int WIT = C * MP / (NT * 4);
  static_assert(WIT * NT * 4 == C * MP, "tile split");
  // with one wave (C = 16) a lane would hold too much of the tiles at once:
  // the first head then loads after the adjoint phase, like the others
  constexpr bool EARLY = NT >= 128;
  struct HeadTile {
    RowTile<T, D, NT, C> tv;
    PairTileT<T, D, NT, C> tvt;  // fp32 only
    floatx4 xw[WIT];
  };
  auto load_head = [&](int side, int hh, HeadTile& ht) {
    const int h = hg * G + hh, bh = b * H + h;
    const T* vb = (side ? dO : q) + (((size_t)b * Tn + t0) * H + h) * D;
    ht.tv.load(vb, (size_t)H * D, 0, Tn - t0, tid);
    if constexpr (!S::TR) ht.tvt.load(vb, (size_t)H * D, 0, Tn - t0, tid);
    const size_t wo = ((size_t)bh * NC * C + t0) * MP;
    if constexpr (S::TR) {  // bf16 inputs: the fp16 copies (every row)
      const f16* wsrc = (side ? pph : sdlh) + wo;
#pragma unroll
      for (int k = 0; k < WIT; ++k)
        ht.xw[k] = __builtin_convertvector(*reinterpret_cast<const f16x4*>(wsrc + (tid + k * NT) * 4), floatx4);
    } else {
      const float* wsrc = (side ? pp : sdl) + wo;
#pragma unroll
      for (int k = 0; k < WIT; ++k) ht.xw[k] = *reinterpret_cast<const floatx4*>(wsrc + (tid + k * NT) * 4);
    }
  };
  auto store_head = [&](const HeadTile& ht) {
#pragma unroll
    for (int k = 0; k < WIT; ++k) {
      const int e = (tid + k * NT) * 4, u = e / MP, i = e % MP, ub = (u & ~15) - 1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (S::TR) {  // block-referenced: W_u 2^{G_u - E_{J-1}}
          const float ep = ub >= 0 ? sm.sG[ub * PG + i + r] : 0.f;
          sm.sW[u * PG + i + r] = ht.xw[k][r] * fast_exp2(sm.sG[u * PG + i + r] - ep);
        } else {
          sm.sW[u * PG + i + r] = ht.xw[k][r];
        }
      }
    }
    ht.tv.template store<PD>(sm.sVec, tid);
    if constexpr (!S::TR) ht.tvt.template store<PC>(sm.sVecT, tid);
  };
  // the loads of one side: this lane's absorbed key row (zero where nothing
  // is absorbed; the address is clamped to a real row either way), the
  // incoming adjoint tile and (two waves or more) the first query head's
  // tiles, all in flight together
  struct SideLoads {
    typename Vec<T>::v8 keyf[D / 32];
    BlockedTile<T, D, NT, MP> tlb;  // bf16 adjoints are stored in column blocks [d/16][i][16]
    RowTile<T, D, NT, MP> tlr;      // fp32: row layout, plus a transposed copy
    PairTileT<T, D, NT, MP> tlt;
    HeadTile ht;
  };
  auto issue = [&](int side, SideLoads& L) {
    const size_t krow = (((size_t)b * Tn + min(max(tq - w, 0), Tn - 1)) * Hkv + hg) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      L.keyf[ks] = ld8_sel<T>((side ? vv : kk) + krow + 32 * ks + 8 * g, absorb);
    const T* lsrc = lin + (((size_t)unit * NC + c) * 2 + side) * MP * D;
    if constexpr (S::TR) {
      L.tlb.load(lsrc, tid);
    } else if constexpr (EARLY) {
      L.tlr.load(lsrc, D, 0, MP, tid);
      L.tlt.load(lsrc, D, 0, MP, tid);
    }
    if constexpr (EARLY) load_head(side, 0, L.ht);
  };
  SideLoads sl[2];
  // (two waves or more) side 0's loads go out right behind the gate loads
  GateTile<T, C, MP, NT> gt;
  gt.load(alpha, b, hg, t0, Tn, Hkv, m, tid);
  if constexpr (EARLY) issue(0, sl[0]);
  gt.template stage<PG, PM>(sm.sG, sm.sA, t0, Tn, m, w, tid);
  __syncthreads();
  lds_col_cumsum<C, MP, PG, NT>(sm.sG, tid);
  if constexpr (S::TR) {
    // pair (I, J >= I): 2^{E_{J-1} - E_I}, clamped to 2^64 for J = I (used
    // only when block I is factorizable, where it is <= 2^16); the side loop's
    // first barrier comes before any read
    constexpr int NW = C / 16;
    for (int x = tid; x < NW * (NW + 1) / 2 * MP; x += NT) {
      int p = x / MP, I0 = 0;
      const int i = x % MP;
      while (p >= NW - I0) p -= NW - I0++;
      const int J0 = I0 + p;
      const float ej = J0 > 0 ? sm.sG[(16 * J0 - 1) * PG + i] : 0.f;
      sm.pf[pair_index<NW>(I0, J0)][i] = fast_exp2(fminf(ej - sm.sG[(16 * I0 + 15) * PG + i], 64.f));
    }
  }
  float bt[NB][4], bwI[NB][4], bwE[NB][4], F[NB][4];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int i = 16 * mb + 4 * g + r;
      float be = (absorb && i < m) ? 1.f - to_f<T>(sm.sA[urow * PM + i]) : 0.f;
      float Gt = sm.sG[urow * PG + i];
      bt[mb][r] = be;
      bwI[mb][r] = be * fast_exp2(sm.sG[(r0 + 15) * PG + i] - Gt);
      bwE[mb][r] = be * fast_exp2(sm.sG[(C - 1) * PG + i] - Gt);
      F[mb][r] = 0.f;
    }
  // with side 0's loads issued early, both sides are unrolled so that each
  // side's loads live in registers of their own only from their issue to
  // their LDS stores; a single wave keeps one set and the loop
#pragma unroll(EARLY ? 2 : 1)
  for (int side = 0; side < 2; ++side) {
    const int li = EARLY ? side : 0;
    if (side == 1 || !EARLY) issue(side, sl[li]);
    SideLoads& L = sl[li];
    const T* lsrc = lin + (((size_t)unit * NC + c) * 2 + side) * MP * D;
    __syncthreads();
    if constexpr (S::TR) {
      L.tlb.template store<PD>(sm.sL, tid);
    } else {  // one wave: one fp32 copy in registers at a time
      if constexpr (!EARLY) L.tlr.load(lsrc, D, 0, MP, tid);
      L.tlr.template store<PD>(sm.sL, tid);
      if constexpr (!EARLY) L.tlt.load(lsrc, D, 0, MP, tid);
      L.tlt.template store<PM>(sm.sLt, tid);
    }
    if constexpr (EARLY) store_head(L.ht);
    __syncthreads();
    floatx4 accO[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) accO[db] = zero4();
    // incoming adjoint: F += 2^{G_end - G_t} <Lin[i], key_t>,  O += sum_i bwE_t[i] Lin[i]
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      floatx4 x = zero4();
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) x = mma32(x, ld8<T>(&sm.sL[(16 * mb + cc) * PD + 32 * ks + 8 * g]), L.keyf[ks]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int i = 16 * mb + 4 * g + r;
        F[mb][r] += fast_exp2(sm.sG[(C - 1) * PG + i] - sm.sG[urow * PG + i]) * x[r];
      }
    }
#pragma unroll
    for (int s = 0; s < NB / 2; ++s) {
      typename Vec<T>::v8 bfr = pack8<T>(floatx4{bwE[2 * s][0], bwE[2 * s][1], bwE[2 * s][2], bwE[2 * s][3]},
                                         floatx4{bwE[2 * s + 1][0], bwE[2 * s + 1][1], bwE[2 * s + 1][2],
                                                 bwE[2 * s + 1][3]});
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        typename Vec<T>::v8 at;
        if constexpr (S::TR) {
          const bf16x4 a0 = ld_tr4(&sm.sL[(32 * s + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
          const bf16x4 a1 = ld_tr4(&sm.sL[(32 * s + 16 + 4 * g + (cc >> 2)) * PD + 16 * db + 4 * (cc & 3)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            at[e] = a0[e];
            at[4 + e] = a1[e];
          }
        } else {
          at = ld4x2<T>(&sm.sLt[(16 * db + cc) * PM + 32 * s + 4 * g],
                        &sm.sLt[(16 * db + cc) * PM + 32 * s + 16 + 4 * g]);
        }
        accO[db] = mma32(accO[db], at, bfr);
      }
    }
#pragma unroll 1
    for (int hh = 0; hh < G; ++hh) {
      if (hh > 0 || !EARLY) {
        HeadTile hn;
        load_head(side, hh, hn);
        __syncthreads();
        store_head(hn);
        __syncthreads();
      }
      const float* wg = (side ? pp : sdl) + ((size_t)(b * H + hg * G + hh) * NC * C + t0) * MP;
      slot_rev<T, D, MP, C>(sm.sVec, sm.sVecT, sm.sW, sm.sG, sm.sA, &sm.pf[0][0], wg, L.keyf, bwI, bt, I, t0, w,
                            Tn, accO, F);
    }
    if (absorb) {
      T* dst = (side ? dnu : dkap) + (((size_t)b * Tn + (tq - w)) * Hkv + hg) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) st4<T>(dst + 16 * db + 4 * g, pack4<T>(accO[db]));
    }
  }
  // X_t = A_t - b_t F_t, its reverse cumsum inside the chunk, local dalpha
  float X[NB][4];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) X[mb][r] = -bt[mb][r] * F[mb][r];
  for (int hh = 0; hh < G; ++hh) {
    const float* ar = acon + ((size_t)(b * H + hg * G + hh) * NC * C + t0 + urow) * MP;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      floatx4 a4 = *reinterpret_cast<const floatx4*>(ar + 16 * mb + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) X[mb][r] += a4[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.sW[urow * PG + 16 * mb + 4 * g + r] = X[mb][r];
  __syncthreads();
  lds_col_rcumsum<C, MP, PG, NT>(sm.sW, tid);
  if (tid < MP) csum[((size_t)unit * NC + c) * MP + tid] = sm.sW[tid];
  if (tq < Tn) {
    float* da = dalpha + (((size_t)b * Tn + tq) * Hkv + hg) * m;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      floatx4 v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * mb + 4 * g + r;
        v4[r] = absorb ? sm.sW[urow * PG + i] / to_f<T>(sm.sA[urow * PM + i]) - F[mb][r] : 0.f;
      }
      const int i0 = 16 * mb + 4 * g;
      if (m % 4 == 0 && i0 + 3 < m) {
        *reinterpret_cast<floatx4*>(da + i0) = v4;  // (rows of m floats: 16-byte aligned)
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (i0 + r < m) da[i0 + r] = v4[r];
      }
    }
  }
}

// Exact carries at the checkpoint chunks c' = q kCarryStride + kCarryStride - 1
// < NC - 1 (bf16): xck[unit][q][i] = <Lin_c'[i], S_{c'+1}[i]> over both halves
// (K and V) -- the adjoint entering chunk c' from the right against the state
// at the start of chunk c' + 1, both stored as bf16 column blocks
// [2][d/16][mp][16].  grid ((NC - 1) / kCarryStride, B*Hkv), 256 threads: slot
// i = tid % MP, its 2 d/16 column blocks split over 256 / MP parts.
template <int D, int MP>
__global__ __launch_bounds__(256) void k_carry_ckpt(const bf16* __restrict__ lin, const bf16* __restrict__ sst,
                                                    float* __restrict__ xck, int NC) {
  constexpr int NP = 256 / MP, NBLK = 2 * (D / 16);
  __shared__ float part[NP][MP];
  const int tid = threadIdx.x, q = blockIdx.x, unit = blockIdx.y, i = tid % MP, pt = tid / MP;
  const int c = q * kCarryStride + kCarryStride - 1;
  const size_t ce = 2 * (size_t)MP * D;
  const bf16* L = lin + ((size_t)unit * NC + c) * ce + i * 16;
  const bf16* S = sst + ((size_t)unit * NC + c + 1) * ce + i * 16;
  float acc = 0.f;
  for (int blk = pt; blk < NBLK; blk += NP) {
    const size_t o = (size_t)blk * MP * 16;  // (side, d/16) block: [mp][16]
    const bf16x8 l0 = ld8<bf16>(L + o), l1 = ld8<bf16>(L + o + 8), s0 = ld8<bf16>(S + o), s1 = ld8<bf16>(S + o + 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)l0[e] * (float)s0[e] + (float)l1[e] * (float)s1[e];
  }
  part[pt][i] = acc;
  __syncthreads();
  if (tid < MP) {
    float x = 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k) x += part[k][tid];
    xck[((size_t)unit * gridDim.x + q) * MP + tid] = x;
  }
}

// dalpha_t[i] += carry_c[i] / alpha_t[i] for the rows t >= w of chunk c, with
// carry_c[i] = sum over the later chunks of their totals of (A - b F).  That
// sum telescopes to <Lin_c[i], S_{c+1}[i]> (the adjoint entering chunk c from
// the right against the state at the next chunk start, both halves), an O(1)
// quantity whose terms mostly cancel: summed over a long sequence, their
// rounding errors would grow with its length.  With checkpoints (xck, bf16
// inputs) the sum runs only up to the next checkpoint chunk c' (the last of
// its group of kCarryStride, c' < NC - 1), whose exact carry xck holds:
// carry_c = sum_{j = c+1 .. c'} total_j + xck[c'].
// grid (NC, B*Hkv), 256 threads: the carry is summed by 256 / MP strided
// parts (a fixed order) and combined through LDS.  Loads are issued in
// batches before their first use (one memory round trip per batch).
template <typename T, int MP, int C>
__global__ __launch_bounds__(256) void k_dalpha_tail(const T* __restrict__ alpha, const float* __restrict__ csum,
                                                     const float* __restrict__ xck, float* __restrict__ dalpha,
                                                     int Tn, int Hkv, int m, int w, int NC) {
  constexpr int NP = 256 / MP, BATCH = 16;
  __shared__ float part[NP][MP];
  __shared__ float carry[MP];
  const int tid = threadIdx.x, c = blockIdx.x, unit = blockIdx.y, b = unit / Hkv, hg = unit % Hkv;
  const int cq = (c / kCarryStride) * kCarryStride + kCarryStride - 1;  // next checkpoint chunk
  const bool ck = xck != nullptr && cq < NC - 1;
  const int cend = ck ? cq + 1 : NC;  // totals of chunks c+1 .. cend-1
  {
    const int i = tid % MP, pt = tid / MP;
    const float* cs = csum + (size_t)unit * NC * MP + i;
    float acc = 0.f;
    for (int c0 = c + 1 + pt; c0 < cend; c0 += BATCH * NP) {
      float x[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const int c2 = c0 + k * NP;
        x[k] = cs[(size_t)(c2 < cend ? c2 : cend - 1) * MP];
      }
#pragma unroll
      for (int k = 0; k < BATCH; ++k) acc += (c0 + k * NP < cend) ? x[k] : 0.f;
    }
    part[pt][i] = acc;
  }
  __syncthreads();
  if (tid < MP) {
    float x = ck ? xck[((size_t)unit * ((NC - 1) / kCarryStride) + cq / kCarryStride) * MP + tid] : 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k) x += part[k][tid];
    carry[tid] = x;
  }
  __syncthreads();
  const int t0 = c * C;
  if (m % 8 == 0) {
    // 8 consecutive slots of one row per thread
    constexpr int PR = MP / 8, NV = C * PR, IT = (NV + 255) / 256;
    floatx4 d0[IT], d1[IT];
    typename Vec<T>::v8 av[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int e = tid + 256 * k, u = e / PR, i0 = (e % PR) * 8, t = t0 + u;
      const int tc = t < Tn ? t : Tn - 1, ic = i0 < m ? i0 : m - 8;
      const size_t idx = (((size_t)b * Tn + tc) * Hkv + hg) * m + ic;
      d0[k] = *reinterpret_cast<const floatx4*>(dalpha + idx);
      d1[k] = *reinterpret_cast<const floatx4*>(dalpha + idx + 4);
      av[k] = ld8<T>(alpha + idx);
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int e = tid + 256 * k, u = e / PR, i0 = (e % PR) * 8, t = t0 + u;
      if (e < NV && i0 < m && t >= w && t < Tn) {
        const size_t idx = (((size_t)b * Tn + t) * Hkv + hg) * m + i0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          d0[k][r] += carry[i0 + r] / to_f<T>(av[k][r]);
          d1[k][r] += carry[i0 + 4 + r] / to_f<T>(av[k][4 + r]);
        }
        *reinterpret_cast<floatx4*>(dalpha + idx) = d0[k];
        *reinterpret_cast<floatx4*>(dalpha + idx + 4) = d1[k];
      }
    }
  } else {
    constexpr int IT = (C * MP + 255) / 256;
    float dv[IT];
    T av[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int e = tid + 256 * k, u = e / MP, i = e % MP, t = t0 + u;
      const int tc = t < Tn ? t : Tn - 1, ic = i < m ? i : m - 1;
      const size_t idx = (((size_t)b * Tn + tc) * Hkv + hg) * m + ic;
      dv[k] = dalpha[idx];
      av[k] = alpha[idx];
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int e = tid + 256 * k, u = e / MP, i = e % MP, t = t0 + u;
      if (e < C * MP && i < m && t >= w && t < Tn)
        dalpha[(((size_t)b * Tn + t) * Hkv + hg) * m + i] = dv[k] + carry[i] / to_f<T>(av[k]);
    }
  }
}

// ---------------------------------------------------------------- window backward: dq
// grid (ceil(T/64), B*H), 4 waves x 16 queries.  dq = R_t^T s sum_j dl_tj R_j k_j
// + the slot part.  Per key tile: S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, and
// dq^T += K^T dS^T.
template <typename T, int D>
struct WinBwdDqSmem {
  static constexpr int PD = pitch_of(D), PK = 64 + 4;
  T k[64 * PD];
  T v[64 * PD];
  T kt[D * PK];
};

__device__ __forceinline__ void rope_cs(double theta, long long pos, float& cs, float& sn) {
  double ang = (double)pos * theta;
  ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
  sincosf((float)ang, &sn, &cs);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_win_bwd_dq(const T* __restrict__ qr, const T* __restrict__ kr,
                                                       const T* __restrict__ vv, const T* __restrict__ dO,
                                                       const float* __restrict__ lse, const float* __restrict__ Dt,
                                                       const T* __restrict__ dqs, T* __restrict__ dq, int Tn,
                                                       int H, int Hkv, int w, float scale, RopeTheta th, int rope) {
  using S = WinBwdDqSmem<T, D>;
  constexpr int PD = S::PD, PK = S::PK;
  __shared__ S sm;
  const int tid = threadIdx.x, W = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int q0 = (L % gridDim.x) * 64, bh = L / gridDim.x, b = bh / H, h = bh % H, hg = h / (H / Hkv);
  const int tq = q0 + 16 * W + cc;
  const bool qvalid = tq < Tn;
  const int tqc = qvalid ? tq : Tn - 1;
  typename Vec<T>::v8 qf[D / 32], df[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const size_t off = (((size_t)b * Tn + tqc) * H + h) * D + 32 * ks + 8 * g;
    qf[ks] = ld8_sel<T>(qr + off, qvalid);
    df[ks] = ld8_sel<T>(dO + off, qvalid);
  }
  const float lse_r = lse[(size_t)bh * Tn + tqc], lse2 = qvalid ? lse_r * NHA_LOG2E : 0.f;
  const float D_r = Dt[(size_t)bh * Tn + tqc], D_t = qvalid ? D_r : 0.f;
  const float sl2 = scale * NHA_LOG2E;
  floatx4 acc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc[db] = zero4();
  if (w > 0) {
    int kmin = q0 - w + 1;
    if (kmin < 0) kmin = 0;
    int kmax = q0 + 63;
    if (kmax > Tn - 1) kmax = Tn - 1;
    const int jfirst = (kmin / 64) * 64;
    const int ntiles = (kmax - jfirst) / 64 + 1;
    const size_t ld = (size_t)Hkv * D;
    const T* kbase = kr + ((size_t)b * Tn * Hkv + hg) * D;
    const T* vbase = vv + ((size_t)b * Tn * Hkv + hg) * D;
    RowTile<T, D, 256> tk, tv;
    PairTileT<T, D, 256> tkt;
    tk.load(kbase + (size_t)jfirst * ld, ld, 0, Tn - jfirst, tid);
    tv.load(vbase + (size_t)jfirst * ld, ld, 0, Tn - jfirst, tid);
    tkt.load(kbase + (size_t)jfirst * ld, ld, 0, Tn - jfirst, tid);
    for (int it = 0; it < ntiles; ++it) {
      const int j0 = jfirst + 64 * it;
      __syncthreads();
      tk.template store<PD>(sm.k, tid);
      tv.template store<PD>(sm.v, tid);
      tkt.template store<PK>(sm.kt, tid);
      __syncthreads();
      if (it + 1 < ntiles) {
        int jn = j0 + 64;
        tk.load(kbase + (size_t)jn * ld, ld, 0, Tn - jn, tid);
        tv.load(vbase + (size_t)jn * ld, ld, 0, Tn - jn, tid);
        tkt.load(kbase + (size_t)jn * ld, ld, 0, Tn - jn, tid);
      }
      float ds[4][4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        floatx4 s4 = zero4(), dp4 = zero4();
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          s4 = mma32(s4, ld8<T>(&sm.k[(16 * mb + cc) * PD + 32 * ks + 8 * g]), qf[ks]);
          dp4 = mma32(dp4, ld8<T>(&sm.v[(16 * mb + cc) * PD + 32 * ks + 8 * g]), df[ks]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int key = j0 + 16 * mb + 4 * g + r;
          bool ok = qvalid && key <= tq && key > tq - w && key < Tn;
          float pv = ok ? fast_exp2(s4[r] * sl2 - lse2) : 0.f;
          ds[mb][r] = pv * (dp4[r] - D_t);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        typename Vec<T>::v8 bfr = pack8<T>(floatx4{ds[2 * st][0], ds[2 * st][1], ds[2 * st][2], ds[2 * st][3]},
                                           floatx4{ds[2 * st + 1][0], ds[2 * st + 1][1], ds[2 * st + 1][2],
                                                   ds[2 * st + 1][3]});
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
          acc[db] = mma32(acc[db],
                          ld4x2<T>(&sm.kt[(16 * db + cc) * PK + 32 * st + 4 * g],
                                   &sm.kt[(16 * db + cc) * PK + 32 * st + 16 + 4 * g]),
                          bfr);
      }
    }
  }
  if (qvalid) {
    // acc[db][r] = dq_rot[d = 16 db + 4 g + r] / scale; rotate back by R_t^T
    constexpr int HB = D / 32;  // d-blocks per half
    float out[D / 16][4];
#pragma unroll
    for (int db = 0; db < HB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int i = 16 * db + 4 * g + r;
        float x1 = acc[db][r] * scale, x2 = acc[db + HB][r] * scale, cs = 1.f, sn = 0.f;
        if (rope) rope_cs(th.theta[i], th.pos0 + tq, cs, sn);
        out[db][r] = x1 * cs + x2 * sn;
        out[db + HB][r] = x2 * cs - x1 * sn;
      }
    const T* sl = dqs + (((size_t)b * Tn + tq) * H + h) * D;  // (null: no slots)
    T* dst = dq + (((size_t)b * Tn + tq) * H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      floatx4 s4 = zero4();
      if (dqs) {
        const typename Vec<T>::v4 x4 = ld4<T>(sl + 16 * db + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) s4[r] = to_f<T>(x4[r]);
      }
      st4<T>(dst + 16 * db + 4 * g,
             pack4<T>(floatx4{out[db][0] + s4[0], out[db][1] + s4[1], out[db][2] + s4[2], out[db][3] + s4[3]}));
    }
  }
}

// bf16 variant: grid (ceil(T / (32 NWV)), B*H), NWV waves x 32 queries on
// 32x32 tiles with the query as the column, as in the forward: per 64-key tile
//   S^T = K Q^T, dP^T = V dO^T, dl^T = P^T (dP^T - D), dq^T += K^T dl^T.
// K and V tiles go straight to LDS (double-buffered); K is read both as row
// fragments and transposed (ds_read_b64_tr_b16), hence the two-pattern
// swizzle (the same for V, so that one set of offsets serves both).
template <int D, int NWV>
__global__ __launch_bounds__(NWV * 64, 2) void k_win_bwd_dq_b16(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ vv,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dt,
    const bf16* __restrict__ dqs, const float2* __restrict__ rcs, bf16* __restrict__ dq, int Tn, int H, int Hkv,
    int w, float scale) {
  constexpr int NT = NWV * 64, QT = 32 * NWV;
  __shared__ bf16 kvbuf[4][64 * D];  // K tiles [0..1], V tiles [2..3]; then the output staging
  const int tid = threadIdx.x, W = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, hf = l >> 5, c = l & 31,
            jj = l & 15;
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int q0 = __builtin_amdgcn_readfirstlane((L % gridDim.x) * QT), bh = __builtin_amdgcn_readfirstlane(L / gridDim.x);
  const int b = __builtin_amdgcn_readfirstlane(bh / H), h = __builtin_amdgcn_readfirstlane(bh % H),
            hg = __builtin_amdgcn_readfirstlane(h / (H / Hkv));
  const int wl = q0 + 32 * W;
  const int tq = wl + c;
  const bool qvalid = tq < Tn;
  const int tqc = qvalid ? tq : Tn - 1;
  const size_t qrow = (((size_t)b * Tn + tqc) * H + h) * D;
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = ld8_sel<bf16>(qr + qrow + 16 * ks + 8 * hf, qvalid);
    df[ks] = ld8_sel<bf16>(dO + qrow + 16 * ks + 8 * hf, qvalid);
  }
  const float lse_r = lse[(size_t)bh * Tn + tqc], lse2 = qvalid ? lse_r * NHA_LOG2E : 0.f;
  const float D_r = Dt[(size_t)bh * Tn + tqc], Dq = qvalid ? D_r : 0.f;
  const float sl2 = scale * NHA_LOG2E;
  floatx16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
  // byte offsets in a tile: row fragments (row c, logical chunk 2 ks + hf) and
  // transposed reads (rows 4 hf + jj / 4 (+8) of each 16-row step, columns
  // 32 dt + 16 (c / 16) + 4 (jj % 4) ..)
  // (toff8: the same 8 rows further on; the swizzle repeats every 16 rows,
  // not every 8)
  uint32_t foff[D / 16], toff[D / 32], toff8[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) foff[ks] = 2 * (c * D + 8 * ((2 * ks + hf) ^ chunk_swz<D, 2>(c)));
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int r = 4 * hf + (jj >> 2), d0 = 32 * dt + 16 * (c >> 4) + 4 * (jj & 3);
    toff[dt] = 2 * (r * D + 8 * ((d0 >> 3) ^ chunk_swz<D, 2>(r)) + (d0 & 7));
    toff8[dt] = 2 * ((r + 8) * D + 8 * ((d0 >> 3) ^ chunk_swz<D, 2>(r + 8)) + (d0 & 7));
  }
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
    const uint32_t kl = lds_addr(&kvbuf[0][0]), vl = lds_addr(&kvbuf[2][0]);
    constexpr uint32_t TB = 64 * D * 2;
    const uint32_t ldo = dma_lane_off<D, NT, 2>(tid, ld);
    dma_tile_async<D, NT, 2>(kbase, ld, tile_j0(0), Tn, kl, ldo, tid);
    dma_tile_async<D, NT, 2>(vbase, ld, tile_j0(0), Tn, vl, ldo, tid);
    wait_vmem();
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int j0 = tile_j0(it), cb = it & 1;
      if (it + 1 < ntiles) {
        const int jn = tile_j0(it + 1);
        dma_tile_async<D, NT, 2>(kbase, ld, jn, Tn, kl + (cb ^ 1) * TB, ldo, tid);
        dma_tile_async<D, NT, 2>(vbase, ld, jn, Tn, vl + (cb ^ 1) * TB, ldo, tid);
      }
      if (wl < Tn && j0 <= wl + 31 && j0 + 63 > wl - w) {
        const uint32_t kt = __builtin_amdgcn_readfirstlane(kl + cb * TB);
        const uint32_t vt = __builtin_amdgcn_readfirstlane(vl + cb * TB);
        floatx16 x[2], dp[2];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            x[kb] = mma32x32(ks == 0 ? zero16() : x[kb], ld8_at(kt + foff[ks] + kb * 64 * D), qf[ks]);
            dp[kb] = mma32x32(ks == 0 ? zero16() : dp[kb], ld8_at(vt + foff[ks] + kb * 64 * D), df[ks]);
          }
        }
        if (!((j0 + 63 <= wl) && (j0 > wl + 31 - w) && (j0 + 63 < Tn))) {
          const int rel = j0 + 4 * hf - tq + w - 1;
          const uint32_t span = (uint32_t)(min(0, Tn - 1 - tq) + w - 1);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if ((uint32_t)(rel + 32 * kb + 8 * (r >> 2) + (r & 3)) > span) x[kb][r] = -INFINITY;
        }
        bf16x8 dsf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) x[kb][r] = fast_exp2(fmaf(x[kb][r], sl2, -lse2)) * (dp[kb][r] - Dq);
#pragma unroll
        for (int st = 0; st < 4; ++st) dsf[st] = pack8_at<bf16>(x[st >> 1], 8 * (st & 1));
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const bf16x4 a0 = ld_tr4_at(kt + toff[dt] + 32 * st * D), a1 = ld_tr4_at(kt + toff8[dt] + 32 * st * D);
            bf16x8 af;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              af[e] = a0[e];
              af[4 + e] = a1[e];
            }
            acc[dt] = mma32x32(acc[dt], af, dsf[st]);
          }
      }
      wait_vmem();
      __syncthreads();
    }
  }
  {
    // acc[dt][4 i + rr] = dq_rot[32 dt + 8 i + 4 hf + rr] / scale; rotate back by R_t^T
    constexpr int HT = D / 64 > 0 ? D / 64 : 1;  // column blocks per half (D >= 64)
    float out[D / 32][16];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) out[dt][e] = acc[dt][e] * scale;
    if (rcs && qvalid) {
      if constexpr (D >= 64) {
        const float2* cs = rcs + (size_t)tq * (D / 2);
#pragma unroll
        for (int dt = 0; dt < HT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float2 t = cs[32 * dt + 8 * (e >> 2) + 4 * hf + (e & 3)];
            const float x1 = out[dt][e], x2 = out[dt + HT][e];
            out[dt][e] = x1 * t.x + x2 * t.y;
            out[dt + HT][e] = x2 * t.x - x1 * t.y;
          }
      } else {
        // D = 32: the partner of column d < 16 is d + 16, held by the same
        // lane at entry e + 8 (8 i + 4 hf + rr with i + 2)
        const float2* cs = rcs + (size_t)tq * (D / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 t = cs[8 * (e >> 2) + 4 * hf + (e & 3)];
          const float x1 = out[0][e], x2 = out[0][e + 8];
          out[0][e] = x1 * t.x + x2 * t.y;
          out[0][e + 8] = x2 * t.x - x1 * t.y;
        }
      }
    }
    // plus the slot part (null: no slots), written in whole rows through the
    // K/V buffers (free after the last barrier; unused when w = 0)
    static_assert(NWV * 32 * (D + 4) * 2 <= 4 * 64 * D * 2, "staging fits the tile buffers");
    bf16* stg = &kvbuf[0][0] + W * 32 * (D + 4);
    auto roff = [&](int row) { return (((size_t)b * Tn + (wl + row)) * H + h) * D; };
    store_tile_rows<D>([&](int dt, int e) { return out[dt][e]; }, stg, dq, dqs, roff, [](int) { return true; },
                       min(32, Tn - wl));
  }
}

// ---------------------------------------------------------------- window backward: dk, dv
// grid (ceil(T/64), B*Hkv), 4 waves x 16 keys.  Loops over the group's query
// heads and the query tiles whose band reaches the keys.  Per query tile:
// S = Q K^T, P, dP = dO V^T, dS; dv^T += dO^T P, dk^T += Q^T dS.
template <typename T, int D>
struct WinBwdKvSmem {
  static constexpr int PD = pitch_of(D), PK = 64 + 4;
  T q[64 * PD];
  T qt[D * PK];
  T o[64 * PD];
  T ot[D * PK];
  float lse2[64];
  float dd[64];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void k_win_bwd_dkdv(
    const T* __restrict__ qr, const T* __restrict__ kr, const T* __restrict__ vv, const T* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Dt, const T* __restrict__ dkap,
    const T* __restrict__ dnu, T* __restrict__ dk, T* __restrict__ dv, int Tn, int H, int Hkv, int w, int sh,
    float scale, RopeTheta th, int rope) {
  using S = WinBwdKvSmem<T, D>;
  constexpr int PD = S::PD, PK = S::PK;
  __shared__ S sm;
  const int tid = threadIdx.x, W = tid >> 6, l = tid & 63, g = l >> 4, cc = l & 15;
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int k0 = (L % gridDim.x) * 64, unit = L / gridDim.x, b = unit / Hkv, hg = unit % Hkv, G = H / Hkv;
  const int key = k0 + 16 * W + cc;
  const bool kvalid = key < Tn;
  typename Vec<T>::v8 kf[D / 32], vf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const size_t off = (((size_t)b * Tn + (kvalid ? key : Tn - 1)) * Hkv + hg) * D + 32 * ks + 8 * g;
    kf[ks] = ld8_sel<T>(kr + off, kvalid);
    vf[ks] = ld8_sel<T>(vv + off, kvalid);
  }
  const float sl2 = scale * NHA_LOG2E;
  floatx4 adk[D / 16], adv[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) adk[db] = adv[db] = zero4();
  if (w > 0) {
    int tmax = k0 + 63 + w - 1;
    if (tmax > Tn - 1) tmax = Tn - 1;
    const int ntiles = k0 <= tmax ? (tmax - k0) / 64 + 1 : 0;
    const size_t ld = (size_t)H * D;
    for (int hh = 0; hh < G; ++hh) {
      const int h = hg * G + hh, bh = b * H + h;
      const T* qbase = qr + ((size_t)b * Tn * H + h) * D;
      const T* obase = dO + ((size_t)b * Tn * H + h) * D;
      RowTile<T, D, 256> tq, to;
      PairTileT<T, D, 256> tqt, tot;
      if (ntiles > 0) {
        tq.load(qbase + (size_t)k0 * ld, ld, 0, Tn - k0, tid);
        tqt.load(qbase + (size_t)k0 * ld, ld, 0, Tn - k0, tid);
        to.load(obase + (size_t)k0 * ld, ld, 0, Tn - k0, tid);
        tot.load(obase + (size_t)k0 * ld, ld, 0, Tn - k0, tid);
      }
      for (int it = 0; it < ntiles; ++it) {
        const int q0 = k0 + 64 * it;
        __syncthreads();
        tq.template store<PD>(sm.q, tid);
        tqt.template store<PK>(sm.qt, tid);
        to.template store<PD>(sm.o, tid);
        tot.template store<PK>(sm.ot, tid);
        if (tid < 64) {
          int t = q0 + tid;
          sm.lse2[tid] = t < Tn ? lse[(size_t)bh * Tn + t] * NHA_LOG2E : 0.f;
          sm.dd[tid] = t < Tn ? Dt[(size_t)bh * Tn + t] : 0.f;
        }
        __syncthreads();
        if (it + 1 < ntiles) {
          int qn = q0 + 64;
          tq.load(qbase + (size_t)qn * ld, ld, 0, Tn - qn, tid);
          tqt.load(qbase + (size_t)qn * ld, ld, 0, Tn - qn, tid);
          to.load(obase + (size_t)qn * ld, ld, 0, Tn - qn, tid);
          tot.load(obase + (size_t)qn * ld, ld, 0, Tn - qn, tid);
        }
        float pm[4][4], ds[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          floatx4 s4 = zero4(), dp4 = zero4();
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            s4 = mma32(s4, ld8<T>(&sm.q[(16 * mb + cc) * PD + 32 * ks + 8 * g]), kf[ks]);
            dp4 = mma32(dp4, ld8<T>(&sm.o[(16 * mb + cc) * PD + 32 * ks + 8 * g]), vf[ks]);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int tl = 16 * mb + 4 * g + r, t = q0 + tl;
            bool ok = kvalid && t < Tn && key <= t && key > t - w;
            float pv = ok ? fast_exp2(s4[r] * sl2 - sm.lse2[tl]) : 0.f;
            pm[mb][r] = pv;
            ds[mb][r] = pv * (dp4[r] - sm.dd[tl]);
          }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          typename Vec<T>::v8 pfr = pack8<T>(floatx4{pm[2 * st][0], pm[2 * st][1], pm[2 * st][2], pm[2 * st][3]},
                                             floatx4{pm[2 * st + 1][0], pm[2 * st + 1][1], pm[2 * st + 1][2],
                                                     pm[2 * st + 1][3]});
          typename Vec<T>::v8 dfr = pack8<T>(floatx4{ds[2 * st][0], ds[2 * st][1], ds[2 * st][2], ds[2 * st][3]},
                                             floatx4{ds[2 * st + 1][0], ds[2 * st + 1][1], ds[2 * st + 1][2],
                                                     ds[2 * st + 1][3]});
#pragma unroll
          for (int db = 0; db < D / 16; ++db) {
            adv[db] = mma32(adv[db],
                            ld4x2<T>(&sm.ot[(16 * db + cc) * PK + 32 * st + 4 * g],
                                     &sm.ot[(16 * db + cc) * PK + 32 * st + 16 + 4 * g]),
                            pfr);
            adk[db] = mma32(adk[db],
                            ld4x2<T>(&sm.qt[(16 * db + cc) * PK + 32 * st + 4 * g],
                                     &sm.qt[(16 * db + cc) * PK + 32 * st + 16 + 4 * g]),
                            dfr);
          }
        }
      }
    }
  }
  if (kvalid) {
    constexpr int HB = D / 32;
    float ok[D / 16][4];
#pragma unroll
    for (int db = 0; db < HB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int i = 16 * db + 4 * g + r;
        float x1 = adk[db][r] * scale, x2 = adk[db + HB][r] * scale, cs = 1.f, sn = 0.f;
        if (rope) rope_cs(th.theta[i], th.pos0 + key, cs, sn);
        ok[db][r] = x1 * cs + x2 * sn;
        ok[db + HB][r] = x2 * cs - x1 * sn;
      }
    const size_t row = (((size_t)b * Tn + key) * Hkv + hg) * D;
    // this key row is also absorbed (at step key + sh); dkap null: no slots
    const bool slot = dkap != nullptr && key + sh < Tn;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      floatx4 sk = zero4(), sv = zero4();
      if (slot) {
        const typename Vec<T>::v4 xk = ld4<T>(dkap + row + 16 * db + 4 * g), xv = ld4<T>(dnu + row + 16 * db + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sk[r] = to_f<T>(xk[r]);
          sv[r] = to_f<T>(xv[r]);
        }
      }
      st4<T>(dk + row + 16 * db + 4 * g,
             pack4<T>(floatx4{ok[db][0] + sk[0], ok[db][1] + sk[1], ok[db][2] + sk[2], ok[db][3] + sk[3]}));
      st4<T>(dv + row + 16 * db + 4 * g, pack4<T>(adv[db] + sv));
    }
  }
}

// bf16 variant: grid (ceil(T / (32 NWV)), B*Hkv), NWV waves x 32 keys on
// 32x32 tiles with the key as the column.  Per 32-query block of each
// 64-query tile of each query head of the group:
//   S' = Q K^T - lse_t / s, dP' = dO V^T - D_t   (the accumulators start at
//        the per-query terms, read from LDS), P = 2^(s log2e S'), dl = P dP'
//   dv^T += dO^T P, dk^T += Q^T dl               (transposed tile reads)
// Q and dO tiles go straight to LDS (double-buffered) with the two-pattern
// swizzle.
template <int D, int NWV>
__global__ __launch_bounds__(NWV * 64, 2) void k_win_bwd_dkdv_b16(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ vv,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dt,
    const bf16* __restrict__ dkap, const bf16* __restrict__ dnu, const float2* __restrict__ rcs,
    bf16* __restrict__ dk, bf16* __restrict__ dv, int Tn, int H, int Hkv, int w, int sh, float scale) {
  constexpr int NT = NWV * 64, KT = 32 * NWV;
  __shared__ bf16 qobuf[4][64 * D];  // Q tiles [0..1], dO tiles [2..3]; then the output staging
  __shared__ float nlb[2][64], ndb[2][64];  // -lse_t / s and -D_t of the tile's queries
  const int tid = threadIdx.x, W = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, hf = l >> 5, c = l & 31,
            jj = l & 15;
  const int L = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int k0 = __builtin_amdgcn_readfirstlane((L % gridDim.x) * KT),
            unit = __builtin_amdgcn_readfirstlane(L / gridDim.x);
  const int b = __builtin_amdgcn_readfirstlane(unit / Hkv), hg = __builtin_amdgcn_readfirstlane(unit % Hkv),
            G = H / Hkv;
  const int kl = k0 + 32 * W;  // first key of this wave
  const int key = kl + c;
  const bool kvalid = key < Tn;
  const size_t krow = (((size_t)b * Tn + (kvalid ? key : Tn - 1)) * Hkv + hg) * D;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    kf[ks] = ld8_sel<bf16>(kr + krow + 16 * ks + 8 * hf, kvalid);
    vf[ks] = ld8_sel<bf16>(vv + krow + 16 * ks + 8 * hf, kvalid);
  }
  const float sl2 = scale * NHA_LOG2E, inv_s = 1.f / scale;
  floatx16 accK[D / 32], accV[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) accK[dt] = accV[dt] = zero16();
  // (the kind-3 swizzle repeats every 8 rows: rows r + 8 are 16 D bytes on)
  // LDS byte offsets of the row fragment of step ks (row c, chunk 2 ks + hf
  // under the swizzle) and of the transposed reads of column block dt: the
  // swizzle is an XOR, which splits into a per-lane base and the step index
  // XORed with the swizzle's upper bits -- two registers instead of one per
  // step (this kernel has none to spare)
  const int swc = chunk_swz<D, 3>(c), fs = swc >> 1;
  const uint32_t fb = 2 * (c * D + 8 * (hf ^ (swc & 1)));
  auto foff = [&](int ks) { return fb + 32u * (uint32_t)(ks ^ fs); };
  const int tr_ = 4 * hf + (jj >> 2), swr = chunk_swz<D, 3>(tr_), ts = swr >> 2;
  const uint32_t tb = 2 * (tr_ * D + 8 * ((2 * (c >> 4) + ((jj & 3) >> 1)) ^ (swr & 3)) + 4 * (jj & 1));
  uint32_t toffa[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) toffa[dt] = tb + 64u * (uint32_t)(dt ^ ts);
  auto toff = [&](int dt) { return toffa[dt]; };
  int tmax = k0 + KT - 1 + w - 1;
  if (tmax > Tn - 1) tmax = Tn - 1;
  const int qfirst = (k0 / 64) * 64;
  const int ntiles = (w > 0 && k0 <= tmax) ? (tmax - qfirst) / 64 + 1 : 0;
  const int total = G * ntiles;
  // query tiles in a rotated order: step j takes the tile X of the band with
  // X = j (mod ntiles), so the workgroups of neighbouring key tiles (same
  // XCD, same time) read each query tile at the same step and all but the
  // first find it in L2 (in band order a tile came back only after every
  // resident workgroup had streamed ~2 tiles, the size of the L2)
  const int rot = ntiles > 0 ? (ntiles - (qfirst / 64) % ntiles) % ntiles : 0;
  auto tile_q0 = [&](int jt) {
    const int jr = jt + rot >= ntiles ? jt + rot - ntiles : jt + rot;
    return qfirst + 64 * jr;
  };
  if (total > 0) {
    const size_t ld = (size_t)H * D;
    const uint32_t ql = lds_addr(&qobuf[0][0]), ol = lds_addr(&qobuf[2][0]);
    constexpr uint32_t TB = 64 * D * 2;
    const uint32_t ldo = dma_lane_off<D, NT, 3>(tid, ld);
    // stage: the tile's lse / D_t values go into registers first (clamped
    // rows: unconditional loads), then the Q and dO tiles into LDS; commit,
    // after the current tile's work, writes the values to LDS -- written
    // right away they would make the wave wait for the tile loads issued
    // before them (the memory counter counts in issue order)
    float lse_n = 0.f, dt_n = 0.f;
    auto stage = [&](int n, int buf) {
      const int hh = n / ntiles, q0 = tile_q0(n - hh * ntiles), h = hg * G + hh;
      const size_t base = ((size_t)b * Tn * H + h) * D;
      if (tid < 64) {
        const size_t e = ((size_t)b * H + h) * Tn + min(q0 + tid, Tn - 1);
        lse_n = lse[e];
        dt_n = Dt[e];
      }
      dma_tile_async<D, NT, 3>(qr + base, ld, q0, Tn, ql + buf * TB, ldo, tid);
      dma_tile_async<D, NT, 3>(dO + base, ld, q0, Tn, ol + buf * TB, ldo, tid);
    };
    auto commit = [&](int n, int buf) {
      if (tid < 64) {
        const int hh = n / ntiles, t = tile_q0(n - hh * ntiles) + tid;
        nlb[buf][tid] = t < Tn ? -lse_n * inv_s : 0.f;
        ndb[buf][tid] = t < Tn ? -dt_n : 0.f;
      }
    };
    stage(0, 0);
    commit(0, 0);
    wait_vmem();
    __syncthreads();
    for (int n = 0; n < total; ++n) {
      const int cb = n & 1;
      if (n + 1 < total) stage(n + 1, cb ^ 1);
      const int hh = n / ntiles, q0 = tile_q0(n - hh * ntiles);
      const uint32_t qt = __builtin_amdgcn_readfirstlane(ql + cb * TB);
      const uint32_t ot = __builtin_amdgcn_readfirstlane(ol + cb * TB);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qb0 = q0 + 32 * qb;
        if (kl < Tn && qb0 < Tn && qb0 + 31 >= kl && qb0 <= kl + 31 + w - 1) {
          floatx16 x, dp;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const floatx4 a = *reinterpret_cast<const floatx4*>(&nlb[cb][32 * qb + 8 * i + 4 * hf]);
            const floatx4 d4 = *reinterpret_cast<const floatx4*>(&ndb[cb][32 * qb + 8 * i + 4 * hf]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              x[4 * i + rr] = a[rr];
              dp[4 * i + rr] = d4[rr];
            }
          }
          if (!((qb0 >= kl + 31) && (qb0 + 31 <= kl + w - 1) && (qb0 + 31 < Tn))) {
            // query - key = rel + 8 i + rr must lie in [0, min(w - 1, Tn - 1 - key)]
            const int rel = qb0 + 4 * hf - key;
            const int span = min(w - 1, Tn - 1 - key);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int dlt = rel + 8 * (e >> 2) + (e & 3);
              if (dlt < 0 || dlt > span) x[e] = -INFINITY;
            }
          }
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            x = mma32x32(x, ld8_at(qt + foff(ks) + qb * 64 * D), kf[ks]);
            dp = mma32x32(dp, ld8_at(ot + foff(ks) + qb * 64 * D), vf[ks]);
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(x[e] * sl2);
            x[e] = p;
            dp[e] *= p;
          }
          const bf16x8 pf0 = pack8_at<bf16>(x, 0), pf1 = pack8_at<bf16>(x, 8);
          const bf16x8 lf0 = pack8_at<bf16>(dp, 0), lf1 = pack8_at<bf16>(dp, 8);
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
              const uint32_t off = toff(dt) + (32 * qb + 16 * st) * D * 2;
              const bf16x4 o0 = ld_tr4_at(ot + off), o1 = ld_tr4_at(ot + off + 16 * D);
              const bf16x4 q0v = ld_tr4_at(qt + off), q1v = ld_tr4_at(qt + off + 16 * D);
              bf16x8 fo, fq;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                fo[e] = o0[e];
                fo[4 + e] = o1[e];
                fq[e] = q0v[e];
                fq[4 + e] = q1v[e];
              }
              accV[dt] = mma32x32(accV[dt], fo, st ? pf1 : pf0);
              accK[dt] = mma32x32(accK[dt], fq, st ? lf1 : lf0);
            }
        }
      }
      if (n + 1 < total) commit(n + 1, cb ^ 1);
      wait_vmem();
      __syncthreads();
    }
  }
  // dk = s Q^T dl rotated back by R_key^T, dv = dO^T P; plus the slot parts of
  // the key row (absorbed at step key + sh).  Each wave puts its 32 x D tile
  // of one output into LDS (the Q / dO buffers are free after the last
  // barrier; pitch D + 4: conflict-free 8-byte writes) and writes it out in
  // whole rows, 16 bytes per lane, adding the slot part read the same way --
  // written straight from the accumulators, each lane would put 8-byte
  // pieces into 32 rows per instruction.
  {
    constexpr int HT = D / 64 > 0 ? D / 64 : 1;
    float ok[D / 32][16];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) ok[dt][e] = accK[dt][e] * scale;
    if (rcs && kvalid) {
      const float2* cs = rcs + (size_t)key * (D / 2);
      if constexpr (D >= 64) {
#pragma unroll
        for (int dt = 0; dt < HT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float2 t = cs[32 * dt + 8 * (e >> 2) + 4 * hf + (e & 3)];
            const float x1 = ok[dt][e], x2 = ok[dt + HT][e];
            ok[dt][e] = x1 * t.x + x2 * t.y;
            ok[dt + HT][e] = x2 * t.x - x1 * t.y;
          }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 t = cs[8 * (e >> 2) + 4 * hf + (e & 3)];
          const float x1 = ok[0][e], x2 = ok[0][e + 8];
          ok[0][e] = x1 * t.x + x2 * t.y;
          ok[0][e + 8] = x2 * t.x - x1 * t.y;
        }
      }
    }
    static_assert(NWV * 32 * (D + 4) * 2 <= 4 * 64 * D * 2, "staging fits the tile buffers");
    // (total == 0: no tile was staged and no barrier passed; the buffers were
    // never used)
    bf16* stg = &qobuf[0][0] + W * 32 * (D + 4);
    auto roff = [&](int row) { return (((size_t)b * Tn + (kl + row)) * Hkv + hg) * D; };
    // this key row is also absorbed (at step key + sh); null: no slots
    auto absorbed = [&](int row) { return kl + row + sh < Tn; };
    const int nrows = min(32, Tn - kl);
    store_tile_rows<D>([&](int dt, int e) { return ok[dt][e]; }, stg, dk, dkap, roff, absorbed, nrows);
    store_tile_rows<D>([&](int dt, int e) { return accV[dt][e]; }, stg, dv, dnu, roff, absorbed, nrows);
  }
}

// ---------------------------------------------------------------- host launcher
template <typename T, int D, int MP, int C>
static hipError_t bwd_impl(const Shape& s, const RopeTheta& th, const BwdPtrs& p, hipStream_t st) {
  if constexpr (sizeof(SlotBwdASmem<T, D, MP, C>) > kMaxLds || sizeof(SlotBwdBSmem<T, D, MP, C>) > kMaxLds ||
                sizeof(WinBwdKvSmem<T, D>) > kMaxLds) {
    return hipErrorInvalidConfiguration;
  } else {
    BwdWs L = bwd_ws_layout(s);
    char* ws = p.ws;
    const T* q = (const T*)p.q;
    const T* k = (const T*)p.k;
    const T* v = (const T*)p.v;
    const T* alpha = (const T*)p.alpha;
    const T* dO = (const T*)p.dO;
    const int units = s.B * s.Hkv;
    Marks mk;
    mk.ev = p.events;
    const Fork fk = side_fork(p.events == nullptr);
    ProloguePtrs pp{ws + L.sst, ws + L.wt, (float*)(ws + L.aend), nullptr, nullptr, nullptr, nullptr, nullptr};
    pp.seg = (float*)(ws + L.seg);
    pp.s0k = p.s0k;
    pp.s0v = p.s0v;
    if (s.rope && s.win) {
      pp.qrot = ws + L.qrot;
      pp.krot = ws + L.krot;
      pp.rcs = (float2*)(ws + L.rcs);
    }
    if (!p.after_fwd) {
      hipError_t e = launch_prologue(s, th, q, k, v, alpha, pp, mk, st, fk);
      if (e != hipSuccess) return e;
    }
    const T* qr = pp.qrot ? (const T*)pp.qrot : q;
    const T* kr = pp.krot ? (const T*)pp.krot : k;
    float* Dt = (float*)(ws + L.dt);
    // the window kernels' dO, lse and D_t: the unified softmax's, or (weighted
    // fusion) the window branch's own
    const T* dOw = p.win_dO ? (const T*)p.win_dO : dO;
    const float* lsew = p.win_lse ? p.win_lse : p.lse;
    const float* Dw = p.win_D ? p.win_D : Dt;
    T* dqs = (T*)(ws + L.dqs);
    T* wpb = (T*)(ws + L.wp);
    float* sdl = (float*)(ws + L.sdl);
    float* ppb = (float*)(ws + L.pp);
    f16* sdlh = s.esz == 2 ? (f16*)(ws + L.sdlh) : nullptr;
    f16* pph = s.esz == 2 ? (f16*)(ws + L.pph) : nullptr;
    float* acon = (float*)(ws + L.acon);
    T* lin = (T*)(ws + L.lin);
    T* dkap = (T*)(ws + L.dkap);
    T* dnu = (T*)(ws + L.dnu);
    float* csum = (float*)(ws + L.csum);
    const long nrows = (long)s.B * s.T * s.H;
    if (s.m == 0) {
      // no slots: D_t, then the window dq and dk/dv with no slot parts
      mk.mark(st);
      hipLaunchKernelGGL((k_bwd_prep<T, D>), dim3((unsigned)((nrows * (D / 8) + 255) / 256)), dim3(256), 0, st,
                         (const T*)p.o, dO, Dt, s.T, s.H, nrows);
      mk.mark(st);
      if constexpr (sizeof(T) == 2) {
        constexpr int NWV = 4;
        const unsigned nt = (unsigned)((s.T + 32 * NWV - 1) / (32 * NWV));
        hipLaunchKernelGGL((k_win_bwd_dq_b16<D, NWV>), dim3(nt, s.B * s.H), dim3(NWV * 64), 0, st, qr, kr, v, dO,
                           p.lse, Dt, (const T*)nullptr, (const float2*)pp.rcs, (T*)p.dq, s.T, s.H, s.Hkv, s.w,
                           s.scale);
        mk.mark(st);
        hipLaunchKernelGGL((k_win_bwd_dkdv_b16<D, NWV>), dim3(nt, units), dim3(NWV * 64), 0, st, qr, kr, v, dO,
                           p.lse, Dt, (const T*)nullptr, (const T*)nullptr, (const float2*)pp.rcs, (T*)p.dk,
                           (T*)p.dv, s.T, s.H, s.Hkv, s.w, s.sh, s.scale);
      } else {
        hipLaunchKernelGGL((k_win_bwd_dq<T, D>), dim3(s.NQ, s.B * s.H), dim3(256), 0, st, qr, kr, v, dO, p.lse, Dt,
                           (const T*)nullptr, (T*)p.dq, s.T, s.H, s.Hkv, s.w, s.scale, th, s.rope ? 1 : 0);
        mk.mark(st);
        hipLaunchKernelGGL((k_win_bwd_dkdv<T, D>), dim3(s.NQ, units), dim3(256), 0, st, qr, kr, v, dO, p.lse, Dt,
                           (const T*)nullptr, (const T*)nullptr, (T*)p.dk, (T*)p.dv, s.T, s.H, s.Hkv, s.w, s.sh, s.scale,
                           th, s.rope ? 1 : 0);
      }
      mk.mark(st);
      return hipGetLastError();
    }
    if constexpr (sizeof(T) == 2) {
      // bf16: pass A also computes D_t
      mk.mark(st);
      hipLaunchKernelGGL((k_bwd_slot_a_b16<D, MP, C>), dim3(s.NC, s.B * s.H), dim3(C / 16 * 64), 0, st, q, k, v,
                         alpha, dO, (const T*)p.o, (const T*)pp.sst, p.lse, Dt, dqs, wpb, sdl, ppb, acon, sdlh, pph,
                         s.T, s.H, s.Hkv, s.m, s.sh, s.NC, s.scale);
    } else {
      mk.mark(st);
      hipLaunchKernelGGL((k_bwd_prep<T, D>), dim3((unsigned)((nrows * (D / 8) + 255) / 256)), dim3(256), 0, st,
                         (const T*)p.o, dO, Dt, s.T, s.H, nrows);
      mk.mark(st);
      const int nitems = s.NC * s.B * s.H;
      const int nwg = nitems < device_cu_count() ? nitems : device_cu_count();
      hipLaunchKernelGGL((k_bwd_slot_a<T, D, MP, C>), dim3(nwg), dim3(C / 16 * 64), 0, st, q, k, v, alpha, dO,
                         (const T*)pp.sst, p.lse, Dt, dqs, wpb, sdl, ppb, acon, s.T, s.H, s.Hkv, s.m, s.sh, s.NC,
                         nitems, s.scale);
    }
    // the adjoint scan and pass B, and beside them on the side stream the
    // window dq (needs D_t and the slot part of dq; nothing after it reads
    // dq), enqueued after the scan so that the scan's workgroups are placed
    // first (the bf16 scan holds no LDS: a dq workgroup fits beside it).
    fk.record(st);
    mk.mark(st);
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL((k_adj_scan_m<MP>), dim3((2 * MP * D + 2047) / 2048, units), dim3(256), 0, st,
                         (const bf16*)wpb, (const float*)pp.aend, (bf16*)lin, p.ds0k, p.ds0v, s.H, s.Hkv, D, s.m,
                         s.NC);
    else
      hipLaunchKernelGGL((k_adj_scan<T, C, MP>), dim3(D / 16, units), dim3(64), 0, st, q, dO, (const T*)wpb,
                         (const float*)pp.aend, lin, p.ds0k, p.ds0v, s.T, s.H, s.Hkv, D, s.m, s.NC);
    fk.mark_mid(st);  // the adjoints are scanned
    const hipStream_t sq = fk.follow(st);
    mk.mark(sq);
    if constexpr (sizeof(T) == 2) {
      constexpr int NWV = 4;
      const unsigned nt = (unsigned)((s.T + 32 * NWV - 1) / (32 * NWV));
      hipLaunchKernelGGL((k_win_bwd_dq_b16<D, NWV>), dim3(nt, s.B * s.H), dim3(NWV * 64), 0, sq, qr, kr, v, dOw,
                         lsew, Dw, dqs, (const float2*)pp.rcs, (T*)p.dq, s.T, s.H, s.Hkv, s.w, s.scale);
    } else {
      hipLaunchKernelGGL((k_win_bwd_dq<T, D>), dim3(s.NQ, s.B * s.H), dim3(256), 0, sq, qr, kr, v, dOw, lsew, Dw,
                         dqs, (T*)p.dq, s.T, s.H, s.Hkv, s.w, s.scale, th, s.rope ? 1 : 0);
    }
    // (bf16) the exact dalpha carries at the checkpoint chunks, from the
    // scanned adjoints, after the window dq on the side stream (beside pass B)
    const float* xckp = nullptr;
    if constexpr (sizeof(T) == 2) {
      const int nq = carry_ckpts(s);
      if (nq > 0) {
        float* xck = (float*)(ws + L.xck);
        fk.wait_mid();
        mk.mark(sq);
        hipLaunchKernelGGL((k_carry_ckpt<D, MP>), dim3(nq, units), dim3(256), 0, sq, (const bf16*)lin,
                           (const bf16*)pp.sst, xck, s.NC);
        xckp = xck;
      }
    }
    mk.mark(st);
    hipLaunchKernelGGL((k_bwd_slot_b<T, D, MP, C>), dim3(s.NC, units), dim3(C / 16 * 64), 0, st, q, k, v, alpha, dO,
                       (const T*)lin, sdl, ppb, acon, sdlh, pph, dkap, dnu, p.dalpha, csum, s.T, s.H, s.Hkv, s.m,
                       s.sh, s.NC);
    // the dalpha carry on the side stream (after dq and pass B), beside the
    // window dk/dv
    const hipStream_t sa = fk.begin(st);
    mk.mark(sa);
    hipLaunchKernelGGL((k_dalpha_tail<T, MP, C>), dim3(s.NC, units), dim3(256), 0, sa, alpha, csum, xckp, p.dalpha,
                       s.T, s.Hkv, s.m, s.sh, s.NC);
    mk.mark(st);
    if constexpr (sizeof(T) == 2) {
      constexpr int NWV = 4;
      const unsigned nt = (unsigned)((s.T + 32 * NWV - 1) / (32 * NWV));
      hipLaunchKernelGGL((k_win_bwd_dkdv_b16<D, NWV>), dim3(nt, units), dim3(NWV * 64), 0, st, qr, kr, v, dOw, lsew,
                         Dw, dkap, dnu, (const float2*)pp.rcs, (T*)p.dk, (T*)p.dv, s.T, s.H, s.Hkv, s.w, s.sh,
                         s.scale);
    } else {
      hipLaunchKernelGGL((k_win_bwd_dkdv<T, D>), dim3(s.NQ, units), dim3(256), 0, st, qr, kr, v, dOw, lsew, Dw, dkap,
                         dnu, (T*)p.dk, (T*)p.dv, s.T, s.H, s.Hkv, s.w, s.sh, s.scale, th, s.rope ? 1 : 0);
    }
    fk.join(st);
    mk.mark(st);
    return hipGetLastError();
  }
}

template <typename T, int MP, int C>
static hipError_t bwd_d(const Shape& s, const RopeTheta& th, const BwdPtrs& p, hipStream_t st) {
  switch (s.d) {
    case 32: return bwd_impl<T, 32, MP, C>(s, th, p, st);
    case 64: return bwd_impl<T, 64, MP, C>(s, th, p, st);
    case 128: return bwd_impl<T, 128, MP, C>(s, th, p, st);
  }
  return hipErrorInvalidValue;
}
template <typename T, int MP>
static hipError_t bwd_c(const Shape& s, const RopeTheta& th, const BwdPtrs& p, hipStream_t st) {
  switch (s.C) {
    case 16: return bwd_d<T, MP, 16>(s, th, p, st);
    case 32: return bwd_d<T, MP, 32>(s, th, p, st);
    case 64: return bwd_d<T, MP, 64>(s, th, p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const Shape& s, const RopeTheta& th, const BwdPtrs& p, hipStream_t st) {
  if (s.dtype == NHA_DTYPE_BF16) return s.mp == 32 ? bwd_c<bf16, 32>(s, th, p, st) : bwd_c<bf16, 64>(s, th, p, st);
  return s.mp == 32 ? bwd_c<float, 32>(s, th, p, st) : bwd_c<float, 64>(s, th, p, st);
}

int bwd_stages(const Shape& s, bool after_fwd, const char** names, int max) {
  const char* all[16];
  int n = 0;
  if (!after_fwd) {
    if (s.m > 0) {
      all[n++] = "chunk_gates";
      if (scan_segments(s).n > 1) {
        all[n++] = "state_scan_seg";
        all[n++] = "scan_combine";
      }
      all[n++] = "state_scan";
    }
    if (s.rope && s.win) {
      all[n++] = "rope_cs";
      all[n++] = "rope";
    }
  }
  if (s.m == 0) {  // no slots
    all[n++] = "bwd_prep";
    all[n++] = "win_bwd_dq";
    all[n++] = "win_bwd_dkdv";
    for (int i = 0; i < n && i < max && names; ++i) names[i] = all[i];
    return n;
  }
  if (s.dtype != NHA_DTYPE_BF16) all[n++] = "bwd_prep";  // bf16: inside slot pass A
  all[n++] = "slot_bwd_a";
  all[n++] = "adj_scan";
  all[n++] = "win_bwd_dq";
  if (carry_ckpts(s) > 0) all[n++] = "carry_ckpt";
  all[n++] = "slot_bwd_b";
  all[n++] = "dalpha_tail";
  all[n++] = "win_bwd_dkdv";
  for (int i = 0; i < n && i < max && names; ++i) names[i] = all[i];
  return n;
}

size_t slot_bwd_lds_bytes(const Shape& s) {
  size_t e = s.esz;
  size_t PD = pitch_of(s.d), PM = pitch_of(s.mp), PC = pitch_of(s.C);
  size_t a = e * (2 * s.mp * PD + s.d * PM + 2 * s.C * PD + s.d * PC + 2 * s.C * PM + s.mp * PC) +
             4 * (size_t)s.C * s.mp;
  size_t b = (e == 2 ? e * (s.mp * PD + s.C * PD + s.C * PM + 16)
                     : e * (s.mp * PD + s.d * PM + s.C * PD + s.d * PC + s.C * PM)) +
             8 * (size_t)s.C * (s.mp + 1);
  size_t kv = e * 2 * (64 * PD + s.d * 68) + 512;
  size_t mx = a > b ? a : b;
  return mx > kv ? mx : kv;
}

}  // namespace nha
