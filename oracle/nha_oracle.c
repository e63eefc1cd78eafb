/*
 * nha_oracle.c -- plain fp64 CPU oracle for the Native Hybrid Attention (NHA)
 * layer operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * What it computes, per (batch b, KV head g), token by token (t = 0 .. T-1):
 *
 *   1. absorb   if t >= w:  SK <- Diag(alpha_t) SK + (1 - alpha_t) (x) k_{t-w}
 *                           SV <- Diag(alpha_t) SV + (1 - alpha_t) (x) v_{t-w}
 *      The gated linear-RNN long-term memory (m slots x d) is the recurrence
 *      for K^long_t printed on the Paper-Notes page "Native Hybrid Attention
 *      for Efficient Sequence Modeling", section 关键设计 > 层内混合; "likewise
 *      for V" follows the same page's 整体框架 section (both K^long and V^long
 *      are gated-RNN memories).  The token shift (only tokens that have left
 *      the window enter the memory; no position encoding on the slots) is the
 *      design-motivation paragraph of that same section.  Reading adopted for
 *      the gate index: the printed recurrence keeps its time index t and only
 *      the token entering changes to k_{t-w} (so w = 0 is the printed
 *      recurrence exactly).  The token-shift ablation of the ai.info page's
 *      findings (every token absorbed at its own step while the window still
 *      holds it) is the shift sh = 0 in place of w: absorb k_{t-sh} for
 *      t >= sh (sh < 0 selects sh = w, the method itself).  Slots start at the given initial states S0
 *      (s0k, s0v; zero when NULL): the ai.info page ("Future Directions",
 *      item 1) names learnable initial slot states as the next step, and the
 *      operator takes them as inputs and returns their gradients.  As for
 *      the zero start, a state is only decayed by the step that absorbs a
 *      token, so S0 is kept unchanged until t = w.
 *   2. window   keys j in [max(0, t-w+1), t]  (the current token and the w-1
 *      before it; w = 0 gives an empty window -> a pure linear RNN, per the
 *      整体框架 / 层间混合 sections).
 *   3. logits   slot i:    s * <SK[i], q_t>            (no RoPE on slots)
 *               window j:  s * <R_t q_t, R_j k_j>     (RoPE on window only)
 *      with s = 1/sqrt(d) as in the o_t formula of 关键设计 > 层内混合 (the
 *      omega_L expression on the same line drops the sqrt(d); we follow o_t).
 *      RoPE: rotate-half pairing (i, i + d/2), theta_i = base^(-2i/d), absolute
 *      positions 0..T-1 (the pages do not name a variant; base 0 disables it).
 *   4. one softmax over all m + n_w logits (the unified softmax of the same
 *      section, and "Fusão Nativa via Softmax Único" on the gist.science page),
 *      o_t = sum_i p_i SV[i] + sum_j p_j v_j,  lse_t = mu + ln Z.
 *
 * Weighted-fusion ablation (lam non-NULL, [B][T][H] in [0, 1]): the slot
 * logits and the window logits each get their own softmax and the two reads
 * are mixed, o_t = lam_t o^L_t + (1 - lam_t) o^W_t.  This is the variant the
 * ai.info page's findings ("Unified softmax beats weighted fusion") compare
 * the unified softmax with -- a fixed coefficient (lam constant) or a learned
 * sequence-dependent one (lam per token, its gradient returned) -- and the
 * separate-then-summed intra-layer hybrids of the Paper-Notes page's 现有痛点
 * paragraph.  lse then holds the slot softmax's lse and lse_w the window's;
 * it needs m >= 1 and w >= 1 (both softmaxes non-empty).
 *
 * Backward: the adjoint of the same per-token recurrence, written from the
 * chain rule (not from the chunkwise form):
 *   dl = p (dp - D_t),  D_t = <dO_t, o_t>
 *   dS^K_t[i] += s dl^L_i q_t,  dS^V_t[i] += p^L_i dO_t      (direct sources)
 *   Lam_t = dS_t + a_{t+1} Lam_{t+1}, a_u = alpha_u if u >= sh else 1
 *   for t >= sh: dk_{t-sh} += sum_i (1-alpha_t[i]) LamK_t[i]   (same for v)
 *               dalpha_t[i] = <LamK_t[i], SK_{t-1}[i] - k_{t-sh}>
 *                           + <LamV_t[i], SV_{t-1}[i] - v_{t-sh}>
 *   window: dq_t += R_t^T s sum_j dl^W_j R_j k_j,
 *           dk_j += R_j^T s dl^W_j R_t q_t, dv_j += p^W_j dO_t.
 *   initial states: dS0 = a_0 Lam_0 (the adjoint carried to before t = 0).
 *   weighted fusion: with cL = lam_t, cW = 1 - lam_t and each branch's own
 *   probabilities, dl^L = cL p^L (dp^L - <dO, o^L>), dl^W = cW p^W (dp^W -
 *   <dO, o^W>), the value sources carry cL p^L and cW p^W, and
 *   dlam_t = <dO_t, o^L_t - o^W_t>.
 * The reverse sweep recomputes states segment by segment from checkpoints
 * spaced every SEG tokens.
 *
 * Layouts (row-major, C order):
 *   q, o, dq, dO : [B][T][H][d]      k, v, dk, dv : [B][T][Hkv][d]
 *   alpha, dalpha: [B][T][Hkv][m]    lse          : [B][H][T]
 *   s0k, s0v (initial slot states, nullable = zero), sk_out, sv_out (final
 *   slot states, nullable), ds0k, ds0v (gradients of s0k, s0v, nullable):
 *   [B][Hkv][m][d]
 * Query head h reads KV head h / (H / Hkv).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC nha_oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SEG 64 /* state checkpoint spacing of the backward reverse sweep */

typedef struct {
  int B, T, H, Hkv, d, m, w;
  double base, scale;
  int sh; /* absorption shift: token t - sh enters the slots at step t >= sh */
} dims_t;

static int check_dims(const dims_t* D) {
  if (D->B < 0 || D->T < 0 || D->H <= 0 || D->Hkv <= 0 || D->d <= 0 ||
      D->m < 0 || D->w < 0)
    return 1;
  if (D->H % D->Hkv) return 1;
  if (D->base != 0.0 && (D->d % 2)) return 1;
  return 0;
}

/* cos/sin tables [T][d/2] for rotate-half RoPE; NULL tables when disabled. */
static void rope_tables(const dims_t* D, double** cs, double** sn) {
  *cs = *sn = NULL;
  if (D->base == 0.0 || D->T == 0) return;
  int h = D->d / 2;
  *cs = (double*)malloc(sizeof(double) * (size_t)D->T * h);
  *sn = (double*)malloc(sizeof(double) * (size_t)D->T * h);
  for (int i = 0; i < h; ++i) {
    double theta = pow(D->base, -2.0 * i / D->d);
    for (int t = 0; t < D->T; ++t) {
      (*cs)[(size_t)t * h + i] = cos(t * theta);
      (*sn)[(size_t)t * h + i] = sin(t * theta);
    }
  }
}

/* y = R_pos x (rotate-half). */
static void rope_apply(const dims_t* D, const double* cs, const double* sn,
                       int pos, const double* x, double* y) {
  int d = D->d;
  if (!cs) {
    memcpy(y, x, sizeof(double) * d);
    return;
  }
  int h = d / 2;
  const double* c = cs + (size_t)pos * h;
  const double* s = sn + (size_t)pos * h;
  for (int i = 0; i < h; ++i) {
    y[i] = x[i] * c[i] - x[i + h] * s[i];
    y[i + h] = x[i + h] * c[i] + x[i] * s[i];
  }
}

/* y = R_pos^T x (inverse rotation). */
static void rope_apply_T(const dims_t* D, const double* cs, const double* sn,
                         int pos, const double* x, double* y) {
  int d = D->d;
  if (!cs) {
    memcpy(y, x, sizeof(double) * d);
    return;
  }
  int h = d / 2;
  const double* c = cs + (size_t)pos * h;
  const double* s = sn + (size_t)pos * h;
  for (int i = 0; i < h; ++i) {
    y[i] = x[i] * c[i] + x[i + h] * s[i];
    y[i + h] = x[i + h] * c[i] - x[i] * s[i];
  }
}

static double dot(const double* a, const double* b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

#define QIDX(b, t, h) ((((size_t)(b) * D->T + (t)) * D->H + (h)) * D->d)
#define KIDX(b, t, g) ((((size_t)(b) * D->T + (t)) * D->Hkv + (g)) * D->d)
#define AIDX(b, t, g) ((((size_t)(b) * D->T + (t)) * D->Hkv + (g)) * D->m)

/* One absorption step (token shift): state <- Diag(a) state + (1-a) (x) x. */
static void absorb(int m, int d, const double* a, const double* x, double* S) {
  for (int i = 0; i < m; ++i) {
    double ai = a[i], bi = 1.0 - a[i];
    double* row = S + (size_t)i * d;
    for (int j = 0; j < d; ++j) row[j] = ai * row[j] + bi * x[j];
  }
}

/* Logits and probabilities for one query at time t of head h (group g).
 * SK/SV: state after the absorption at t.  kr: rotated keys of this (b,g).
 * Writes p (length m + nw), returns lse; o_out (nullable) gets the output. */
/* softmax over p[0..n) in place; returns its lse (-inf when n = 0) */
static double softmax_inplace(double* p, int n) {
  double mu = -INFINITY, Z = 0.0;
  for (int e = 0; e < n; ++e)
    if (p[e] > mu) mu = p[e];
  for (int e = 0; e < n; ++e) {
    p[e] = exp(p[e] - mu);
    Z += p[e];
  }
  for (int e = 0; e < n; ++e) p[e] /= Z;
  return mu + log(Z);
}

/* Logits and probabilities for one query at time t of head h (group g).
 * SK/SV: state after the absorption at t.  kr: rotated keys of this (b,g).
 * Unified softmax (mix = NULL): p (length m + nw) is one softmax over all
 * logits, o_out (nullable) the output; returns the lse.
 * Weighted fusion (mix = {lam}): p[0..m) is the softmax of the slot logits,
 * p[m..m+nw) that of the window logits; oL, oW (nullable) get the two reads
 * and o_out lam oL + (1 - lam) oW; returns the slot lse, *lse_w the window's. */
typedef struct {
  double lam;
  double* oL;
  double* oW;
  double lse_w;
} mix_t;

static double read_step(const dims_t* D, const double* cs, const double* sn,
                        int t, const double* qv, const double* SK,
                        const double* SV, const double* kr, const double* vg,
                        size_t vstride, double* qr, double* p, double* o_out,
                        int* nw_out, mix_t* mix) {
  int d = D->d, m = D->m, w = D->w;
  double s = D->scale;
  int j0 = t - w + 1;
  if (j0 < 0) j0 = 0;
  int nw = (w > 0) ? (t - j0 + 1) : 0;
  rope_apply(D, cs, sn, t, qv, qr);
  for (int i = 0; i < m; ++i) p[i] = s * dot(SK + (size_t)i * d, qv, d);
  for (int j = 0; j < nw; ++j) p[m + j] = s * dot(qr, kr + (size_t)(j0 + j) * d, d);
  double lse;
  if (!mix) {
    lse = softmax_inplace(p, m + nw);
  } else {
    lse = softmax_inplace(p, m);
    mix->lse_w = softmax_inplace(p + m, nw);
  }
  double cL = mix ? mix->lam : 1.0, cW = mix ? 1.0 - mix->lam : 1.0;
  if (o_out) {
    for (int c = 0; c < d; ++c) o_out[c] = 0.0;
    if (mix && mix->oL)
      for (int c = 0; c < d; ++c) mix->oL[c] = mix->oW[c] = 0.0;
    for (int i = 0; i < m; ++i) {
      const double* r = SV + (size_t)i * d;
      for (int c = 0; c < d; ++c) o_out[c] += cL * p[i] * r[c];
      if (mix && mix->oL)
        for (int c = 0; c < d; ++c) mix->oL[c] += p[i] * r[c];
    }
    for (int j = 0; j < nw; ++j) {
      const double* r = vg + (size_t)(j0 + j) * vstride;
      for (int c = 0; c < d; ++c) o_out[c] += cW * p[m + j] * r[c];
      if (mix && mix->oW)
        for (int c = 0; c < d; ++c) mix->oW[c] += p[m + j] * r[c];
    }
  }
  *nw_out = nw;
  return lse;
}

/* rotated keys of one (b, g): kr[t][d] */
static void rotate_keys(const dims_t* D, const double* cs, const double* sn,
                        const double* k, int b, int g, double* kr) {
  for (int t = 0; t < D->T; ++t)
    rope_apply(D, cs, sn, t, k + KIDX(b, t, g), kr + (size_t)t * D->d);
}

int nha_oracle_fwd(int B, int T, int H, int Hkv, int d, int m, int w, int shift,
                   double rope_base, double scale, const double* q,
                   const double* k, const double* v, const double* alpha,
                   const double* s0k, const double* s0v, const double* lam,
                   double* o, double* lse, double* lse_w, double* sk_out,
                   double* sv_out, int nthreads) {
  dims_t Dm = {B, T, H, Hkv, d, m, w, rope_base, scale, shift < 0 ? w : shift};
  const dims_t* D = &Dm;
  if (check_dims(D)) return 1;
  if (lam && (m < 1 || w < 1)) return 1;
  if (Dm.scale == 0.0) Dm.scale = 1.0 / sqrt((double)d);
  double *cs, *sn;
  rope_tables(D, &cs, &sn);
  int G = H / Hkv, units = B * Hkv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    int b = u / Hkv, g = u % Hkv;
    double* SK = (double*)calloc((size_t)m * d + 1, sizeof(double));
    double* SV = (double*)calloc((size_t)m * d + 1, sizeof(double));
    if (s0k) memcpy(SK, s0k + (size_t)u * m * d, sizeof(double) * m * d);
    if (s0v) memcpy(SV, s0v + (size_t)u * m * d, sizeof(double) * m * d);
    double* kr = (double*)malloc(sizeof(double) * ((size_t)T * d + 1));
    double* qr = (double*)malloc(sizeof(double) * d);
    double* p = (double*)malloc(sizeof(double) * (m + (size_t)(w < T ? w : T) + 1));
    rotate_keys(D, cs, sn, k, b, g, kr);
    const double* vg = v + KIDX(b, 0, g);
    size_t vstride = (size_t)Hkv * d;
    for (int t = 0; t < T; ++t) {
      if (t >= Dm.sh) {
        absorb(m, d, alpha + AIDX(b, t, g), k + KIDX(b, t - Dm.sh, g), SK);
        absorb(m, d, alpha + AIDX(b, t, g), v + KIDX(b, t - Dm.sh, g), SV);
      }
      for (int hh = 0; hh < G; ++hh) {
        int h = g * G + hh, nw;
        mix_t mx = {lam ? lam[((size_t)b * T + t) * H + h] : 0.0, NULL, NULL, 0.0};
        double l = read_step(D, cs, sn, t, q + QIDX(b, t, h), SK, SV, kr, vg,
                             vstride, qr, p, o + QIDX(b, t, h), &nw, lam ? &mx : NULL);
        if (lse) lse[((size_t)b * H + h) * T + t] = l;
        if (lam && lse_w) lse_w[((size_t)b * H + h) * T + t] = mx.lse_w;
      }
    }
    if (sk_out) memcpy(sk_out + (size_t)u * m * d, SK, sizeof(double) * m * d);
    if (sv_out) memcpy(sv_out + (size_t)u * m * d, SV, sizeof(double) * m * d);
    free(SK);
    free(SV);
    free(kr);
    free(qr);
    free(p);
  }
  free(cs);
  free(sn);
  return 0;
}

int nha_oracle_bwd(int B, int T, int H, int Hkv, int d, int m, int w, int shift,
                   double rope_base, double scale, const double* q,
                   const double* k, const double* v, const double* alpha,
                   const double* s0k, const double* s0v, const double* lam,
                   const double* dO, double* dq, double* dk, double* dv,
                   double* dalpha, double* ds0k, double* ds0v, double* dlam,
                   int nthreads) {
  dims_t Dm = {B, T, H, Hkv, d, m, w, rope_base, scale, shift < 0 ? w : shift};
  const dims_t* D = &Dm;
  if (check_dims(D)) return 1;
  if (lam && (m < 1 || w < 1)) return 1;
  if (Dm.scale == 0.0) Dm.scale = 1.0 / sqrt((double)d);
  double s = Dm.scale;
  double *cs, *sn;
  rope_tables(D, &cs, &sn);
  int G = H / Hkv, units = B * Hkv;
  size_t md = (size_t)m * d;
  int nseg = (T + SEG - 1) / SEG;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    int b = u / Hkv, g = u % Hkv;
    size_t vstride = (size_t)Hkv * d;
    const double* vg = v + KIDX(b, 0, g);
    /* checkpoints: state BEFORE the absorption at each segment start */
    double* ckK = (double*)calloc((size_t)nseg * md + 1, sizeof(double));
    double* ckV = (double*)calloc((size_t)nseg * md + 1, sizeof(double));
    /* per-segment states after the absorption at t (SEG + 1 entries: index 0
       holds the state before the segment) */
    double* stK = (double*)malloc(sizeof(double) * ((SEG + 1) * md + 1));
    double* stV = (double*)malloc(sizeof(double) * ((SEG + 1) * md + 1));
    double* kr = (double*)malloc(sizeof(double) * ((size_t)T * d + 1));
    double* dkr = (double*)calloc((size_t)T * d + 1, sizeof(double));
    double* LK = (double*)calloc(md + 1, sizeof(double));
    double* LV = (double*)calloc(md + 1, sizeof(double));
    int wmax = w < T ? w : T;
    double* p = (double*)malloc(sizeof(double) * (m + (size_t)wmax + 1));
    double* dl = (double*)malloc(sizeof(double) * (m + (size_t)wmax + 1));
    double* qr = (double*)malloc(sizeof(double) * d);
    double* ov = (double*)malloc(sizeof(double) * d);
    double* oL = (double*)malloc(sizeof(double) * d);
    double* oW = (double*)malloc(sizeof(double) * d);
    double* dqr = (double*)malloc(sizeof(double) * d);
    double* tmp = (double*)malloc(sizeof(double) * d);
    rotate_keys(D, cs, sn, k, b, g, kr);
    /* forward sweep: checkpoints */
    {
      double* SK = (double*)calloc(md + 1, sizeof(double));
      double* SV = (double*)calloc(md + 1, sizeof(double));
      if (s0k) memcpy(SK, s0k + (size_t)u * md, sizeof(double) * md);
      if (s0v) memcpy(SV, s0v + (size_t)u * md, sizeof(double) * md);
      for (int t = 0; t < T; ++t) {
        if (t % SEG == 0) {
          memcpy(ckK + (size_t)(t / SEG) * md, SK, sizeof(double) * md);
          memcpy(ckV + (size_t)(t / SEG) * md, SV, sizeof(double) * md);
        }
        if (t >= Dm.sh) {
          absorb(m, d, alpha + AIDX(b, t, g), k + KIDX(b, t - Dm.sh, g), SK);
          absorb(m, d, alpha + AIDX(b, t, g), v + KIDX(b, t - Dm.sh, g), SV);
        }
      }
      free(SK);
      free(SV);
    }
    /* zero this unit's dk, dv rows (window and slot paths both add) */
    for (int t = 0; t < T; ++t) {
      memset(dk + KIDX(b, t, g), 0, sizeof(double) * d);
      memset(dv + KIDX(b, t, g), 0, sizeof(double) * d);
    }
    /* reverse sweep; LK/LV hold a_{t+1} Lam_{t+1} on entry to step t */
    for (int sg = nseg - 1; sg >= 0; --sg) {
      int t0 = sg * SEG, t1 = t0 + SEG < T ? t0 + SEG : T;
      memcpy(stK, ckK + (size_t)sg * md, sizeof(double) * md);
      memcpy(stV, ckV + (size_t)sg * md, sizeof(double) * md);
      for (int t = t0; t < t1; ++t) {
        double* nK = stK + (size_t)(t - t0 + 1) * md;
        double* nV = stV + (size_t)(t - t0 + 1) * md;
        memcpy(nK, nK - md, sizeof(double) * md);
        memcpy(nV, nV - md, sizeof(double) * md);
        if (t >= Dm.sh) {
          absorb(m, d, alpha + AIDX(b, t, g), k + KIDX(b, t - Dm.sh, g), nK);
          absorb(m, d, alpha + AIDX(b, t, g), v + KIDX(b, t - Dm.sh, g), nV);
        }
      }
      for (int t = t1 - 1; t >= t0; --t) {
        const double* SK = stK + (size_t)(t - t0 + 1) * md; /* S_t */
        const double* SV = stV + (size_t)(t - t0 + 1) * md;
        const double* SKp = SK - md; /* S_{t-1} */
        const double* SVp = SV - md;
        /* Lam_t = direct sources + carried */
        for (int hh = 0; hh < G; ++hh) {
          int h = g * G + hh, nw;
          const double* qv = q + QIDX(b, t, h);
          const double* dov = dO + QIDX(b, t, h);
          mix_t mx = {lam ? lam[((size_t)b * T + t) * H + h] : 0.0, oL, oW, 0.0};
          read_step(D, cs, sn, t, qv, SK, SV, kr, vg, vstride, qr, p, ov, &nw, lam ? &mx : NULL);
          int j0 = t - w + 1;
          if (j0 < 0) j0 = 0;
          /* unified: one softmax, cL = cW = 1 and D_L = D_W = <dO, o>;
             weighted: each branch's own softmax, scaled by its coefficient */
          double cL = 1.0, cW = 1.0, DL, DW;
          if (lam) {
            cL = mx.lam;
            cW = 1.0 - mx.lam;
            DL = dot(dov, oL, d);
            DW = dot(dov, oW, d);
            if (dlam) dlam[((size_t)b * T + t) * H + h] = DL - DW;
          } else {
            DL = DW = dot(dov, ov, d);
          }
          for (int i = 0; i < m; ++i) {
            double dp = dot(dov, SV + (size_t)i * d, d);
            dl[i] = cL * p[i] * (dp - DL);
          }
          for (int j = 0; j < nw; ++j) {
            double dp = dot(dov, vg + (size_t)(j0 + j) * vstride, d);
            dl[m + j] = cW * p[m + j] * (dp - DW);
          }
          /* dq: slots (unrotated) + window (rotated frame, then R_t^T) */
          double* dqv = dq + QIDX(b, t, h);
          for (int c = 0; c < d; ++c) dqv[c] = 0.0;
          for (int i = 0; i < m; ++i) {
            const double* r = SK + (size_t)i * d;
            for (int c = 0; c < d; ++c) dqv[c] += s * dl[i] * r[c];
          }
          for (int c = 0; c < d; ++c) dqr[c] = 0.0;
          for (int j = 0; j < nw; ++j) {
            const double* r = kr + (size_t)(j0 + j) * d;
            double* dr = dkr + (size_t)(j0 + j) * d;
            double* dvr = dv + KIDX(b, j0 + j, g);
            for (int c = 0; c < d; ++c) {
              dqr[c] += s * dl[m + j] * r[c];
              dr[c] += s * dl[m + j] * qr[c];
              dvr[c] += cW * p[m + j] * dov[c];
            }
          }
          rope_apply_T(D, cs, sn, t, dqr, tmp);
          for (int c = 0; c < d; ++c) dqv[c] += tmp[c];
          /* direct sources into the adjoint */
          for (int i = 0; i < m; ++i) {
            double* rk = LK + (size_t)i * d;
            double* rv = LV + (size_t)i * d;
            for (int c = 0; c < d; ++c) {
              rk[c] += s * dl[i] * qv[c];
              rv[c] += cL * p[i] * dov[c];
            }
          }
        }
        /* LK/LV now hold Lam_t. */
        if (t >= Dm.sh) {
          const double* a = alpha + AIDX(b, t, g);
          const double* kap = k + KIDX(b, t - Dm.sh, g);
          const double* nu = v + KIDX(b, t - Dm.sh, g);
          double* dkk = dk + KIDX(b, t - Dm.sh, g);
          double* dvv = dv + KIDX(b, t - Dm.sh, g);
          double* da = dalpha + AIDX(b, t, g);
          for (int i = 0; i < m; ++i) {
            const double* lk = LK + (size_t)i * d;
            const double* lv = LV + (size_t)i * d;
            const double* sk = SKp + (size_t)i * d;
            const double* sv = SVp + (size_t)i * d;
            double bi = 1.0 - a[i], acc = 0.0;
            for (int c = 0; c < d; ++c) {
              dkk[c] += bi * lk[c];
              dvv[c] += bi * lv[c];
              acc += lk[c] * (sk[c] - kap[c]) + lv[c] * (sv[c] - nu[c]);
            }
            da[i] = acc;
          }
          for (int i = 0; i < m; ++i) {
            double* lk = LK + (size_t)i * d;
            double* lv = LV + (size_t)i * d;
            for (int c = 0; c < d; ++c) {
              lk[c] *= a[i];
              lv[c] *= a[i];
            }
          }
        } else {
          double* da = dalpha + AIDX(b, t, g);
          for (int i = 0; i < m; ++i) da[i] = 0.0;
        }
      }
    }
    /* LK/LV now hold a_0 Lam_0: the gradient of the initial states */
    if (ds0k) memcpy(ds0k + (size_t)u * md, LK, sizeof(double) * md);
    if (ds0v) memcpy(ds0v + (size_t)u * md, LV, sizeof(double) * md);
    /* window dk: un-rotate and add */
    for (int t = 0; t < T; ++t) {
      rope_apply_T(D, cs, sn, t, dkr + (size_t)t * d, tmp);
      double* dkk = dk + KIDX(b, t, g);
      for (int c = 0; c < d; ++c) dkk[c] += tmp[c];
    }
    free(ckK);
    free(ckV);
    free(stK);
    free(stV);
    free(kr);
    free(dkr);
    free(LK);
    free(LV);
    free(p);
    free(dl);
    free(qr);
    free(ov);
    free(oL);
    free(oW);
    free(dqr);
    free(tmp);
  }
  free(cs);
  free(sn);
  return 0;
}
