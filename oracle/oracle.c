/*
 * oracle.c -- plain fp64 CPU oracle for the hybrid gated-linear + sliding-window
 * attention layer of Lizard.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct definition
 * that the GPU library is checked against.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or helper with the HIP library, and it never calls into it.
 *
 * Sources (the pages, cited by title and section):
 *  - "Lizard" technical summary (gist.science, paper 2507.09025), Methodology
 *    section A.1 "Gated Linear Attention": a learnable data-dependent gate
 *    Gamma_i = sigmoid(W_gamma x_i) controls how fast past tokens decay, and a
 *    hidden state S_i is updated token by token so memory stays constant.
 *  - same page, Methodology section A.2 "Anchor window attention": sliding-window
 *    softmax attention whose denominator is extended by learnable meta-memory
 *    scalars t_j that act as an attention sink.
 *  - same page, Methodology section C "Hardware-aware algorithm": the feature map
 *    is Hedgehog's and is non-negative.
 *  - Lizard abstract (chatpaper.ai): the layer is the combination of gated linear
 *    attention (global compression) and meta-memory sliding-window attention
 *    (local detail).
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *  R1 phi(x) = [softmax(x W), softmax(-x W)], softmax over the f/2 axis.
 *  R2 separate Hedgehog projections for q and k, one per head, [H][d][f/2].
 *  R4 the gate is per feature channel (diagonal over the f rows of S).
 *  R5 S_t = diag(Gamma_t) S_{t-1} + phi(k_t)^T v_t: the token's own outer product
 *     is not decayed; readout o_t = phi(q_t) S_t, no normaliser (R7).
 *  R6 the linear-attention part covers every j <= t (also inside the window).
 *  R8 the two parts are summed with unit weights.
 *  R9 each meta scalar t_m adds exp(t_m) to the softmax denominator and carries a
 *     zero value vector.
 *  R10 the window of token t is j in [t-w+1, t] (w keys including t itself).
 *  R11 SWA score = scale * (q_t . k_j).
 *
 * Everything is double precision; inputs arrive already widened to double.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PART_GLA 1
#define ORACLE_PART_SWA 2

/* Hedgehog feature map of one d-vector x with projection W[d][f2]:
 * u = x W, phi[0..f2) = softmax(u), phi[f2..2 f2) = softmax(-u). */
static void hedgehog(const double *x, const double *W, int d, int f2, double *u,
                     double *phi) {
  for (int j = 0; j < f2; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += x[i] * W[(size_t)i * f2 + j];
    u[j] = acc;
  }
  double mx = -INFINITY, mn = INFINITY;
  for (int j = 0; j < f2; ++j) {
    if (u[j] > mx) mx = u[j];
    if (u[j] < mn) mn = u[j];
  }
  double zp = 0.0, zn = 0.0;
  for (int j = 0; j < f2; ++j) {
    phi[j] = exp(u[j] - mx);
    phi[f2 + j] = exp(-u[j] + mn);
    zp += phi[j];
    zn += phi[f2 + j];
  }
  for (int j = 0; j < f2; ++j) {
    phi[j] /= zp;
    phi[f2 + j] /= zn;
  }
}

/* Gate value Gamma in [0,1] for one channel: sigmoid of a logit, or exp of a
 * log-gate (gate_is_log != 0, values <= 0, -inf allowed). */
static double gate_value(double g, int gate_is_log) {
  if (gate_is_log) return exp(g);
  if (g >= 0.0) return 1.0 / (1.0 + exp(-g));
  double e = exp(g);
  return e / (1.0 + e);
}

/* Sliding-window softmax with meta-memory sinks for one query.
 * keys[j], vals[j] for j in [0, n): the n window keys (already selected).
 * Writes out[dv] = sum_j p_j v_j with p_j = e^{s_j} / (sum_j e^{s_j} + sum_m e^{t_m}). */
static void window_softmax(const double *qt, const double *const *keys,
                           const double *const *vals, int n, int d, int dv,
                           const double *meta, int n_meta, double scale,
                           double *s, double *out) {
  double m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += qt[i] * keys[j][i];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  for (int mm = 0; mm < n_meta; ++mm)
    if (meta[mm] > m) m = meta[mm];
  double den = 0.0;
  for (int c = 0; c < dv; ++c) out[c] = 0.0;
  for (int j = 0; j < n; ++j) {
    double p = exp(s[j] - m);
    den += p;
    for (int c = 0; c < dv; ++c) out[c] += p * vals[j][c];
  }
  for (int mm = 0; mm < n_meta; ++mm) den += exp(meta[mm] - m);
  for (int c = 0; c < dv; ++c) out[c] /= den;
}

/*
 * Full layer, token by token, for every (b, h).
 * Layouts (row-major): q,k [B][H][L][d]; v,o [B][H][L][dv]; g [B][H][L][f];
 * wq,wk [H][d][f/2]; meta [H][n_meta]; state [B][H][f][dv].
 * parts: bit 1 = gated linear attention, bit 2 = window attention (o is the sum
 * of the enabled parts).  state_in may be NULL (zero state); state_out may be
 * NULL.  Returns 0, or -1 on bad arguments.
 */
int oracle_layer_fwd(int B, int H, int L, int d, int dv, int f, int window,
                     int n_meta, double scale, int gate_is_log, int parts,
                     const double *q, const double *k, const double *v,
                     const double *g, const double *wq, const double *wk,
                     const double *meta, const double *state_in,
                     double *state_out, double *o) {
  if (B < 0 || H < 0 || L < 0 || d <= 0 || dv <= 0 || f <= 0 || (f & 1) ||
      window < 1 || n_meta < 0)
    return -1;
  const int f2 = f / 2;
  const int BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < BH; ++bh) {
    const int h = bh % H;
    const double *qh = q + (size_t)bh * L * d;
    const double *kh = k + (size_t)bh * L * d;
    const double *vh = v + (size_t)bh * L * dv;
    const double *gh = g ? g + (size_t)bh * L * f : NULL;
    const double *Wq = wq ? wq + (size_t)h * d * f2 : NULL;
    const double *Wk = wk ? wk + (size_t)h * d * f2 : NULL;
    const double *mh = n_meta ? meta + (size_t)h * n_meta : NULL;
    double *oh = o + (size_t)bh * L * dv;

    double *S = calloc((size_t)f * dv, sizeof(double));
    double *u = malloc(sizeof(double) * f2);
    double *phq = malloc(sizeof(double) * f);
    double *phk = malloc(sizeof(double) * f);
    double *s = malloc(sizeof(double) * window);
    double *sw = malloc(sizeof(double) * dv);
    const double **keys = malloc(sizeof(double *) * window);
    const double **vals = malloc(sizeof(double *) * window);
    if (state_in) memcpy(S, state_in + (size_t)bh * f * dv, sizeof(double) * f * dv);

    for (int t = 0; t < L; ++t) {
      const double *qt = qh + (size_t)t * d;
      const double *kt = kh + (size_t)t * d;
      const double *vt = vh + (size_t)t * dv;
      double *ot = oh + (size_t)t * dv;
      for (int c = 0; c < dv; ++c) ot[c] = 0.0;

      if (parts & ORACLE_PART_GLA) {
        hedgehog(qt, Wq, d, f2, u, phq);
        hedgehog(kt, Wk, d, f2, u, phk);
        for (int r = 0; r < f; ++r) {
          const double gam = gate_value(gh[(size_t)t * f + r], gate_is_log);
          for (int c = 0; c < dv; ++c)
            S[(size_t)r * dv + c] = gam * S[(size_t)r * dv + c] + phk[r] * vt[c];
        }
        for (int c = 0; c < dv; ++c) {
          double acc = 0.0;
          for (int r = 0; r < f; ++r) acc += phq[r] * S[(size_t)r * dv + c];
          ot[c] += acc;
        }
      }
      if (parts & ORACLE_PART_SWA) {
        const int j0 = t - window + 1 > 0 ? t - window + 1 : 0;
        int n = 0;
        for (int j = j0; j <= t; ++j, ++n) {
          keys[n] = kh + (size_t)j * d;
          vals[n] = vh + (size_t)j * dv;
        }
        window_softmax(qt, keys, vals, n, d, dv, mh, n_meta, scale, s, sw);
        for (int c = 0; c < dv; ++c) ot[c] += sw[c];
      }
    }
    if (state_out) memcpy(state_out + (size_t)bh * f * dv, S, sizeof(double) * f * dv);
    free(S); free(u); free(phq); free(phk); free(s); free(sw); free(keys); free(vals);
  }
  return 0;
}

/*
 * One recurrent decode step for every (b, h): the constant-memory inference form.
 * q,k [B][H][d]; v,o [B][H][dv]; g [B][H][f]; state [B][H][f][dv] (in/out);
 * kcache [B][H][w][d], vcache [B][H][w][dv] (in/out ring: token p lives in slot
 * p mod w); pos[b] = number of tokens already consumed by sequence b (the new
 * token's position).  The step appends the token to the ring, then attends over
 * positions [max(0, pos-w+1), pos].
 */
int oracle_decode_step(int B, int H, int d, int dv, int f, int window,
                       int n_meta, double scale, int gate_is_log, int parts,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *wq, const double *wk,
                       const double *meta, double *state, double *kcache,
                       double *vcache, const long long *pos, double *o) {
  if (B < 0 || H < 0 || d <= 0 || dv <= 0 || f <= 0 || (f & 1) || window < 1 ||
      n_meta < 0)
    return -1;
  const int f2 = f / 2;
  const int BH = B * H;
  for (int b = 0; b < B; ++b)
    if (pos[b] < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < BH; ++bh) {
    const int b = bh / H, h = bh % H;
    const long long p = pos[b];
    const double *qt = q + (size_t)bh * d;
    const double *kt = k + (size_t)bh * d;
    const double *vt = v + (size_t)bh * dv;
    double *ot = o + (size_t)bh * dv;
    double *S = state + (size_t)bh * f * dv;
    double *kc = kcache + (size_t)bh * window * d;
    double *vc = vcache + (size_t)bh * window * dv;
    const double *mh = n_meta ? meta + (size_t)h * n_meta : NULL;
    double *u = malloc(sizeof(double) * f2);
    double *phq = malloc(sizeof(double) * f);
    double *phk = malloc(sizeof(double) * f);
    double *s = malloc(sizeof(double) * window);
    double *sw = malloc(sizeof(double) * dv);
    const double **keys = malloc(sizeof(double *) * window);
    const double **vals = malloc(sizeof(double *) * window);
    for (int c = 0; c < dv; ++c) ot[c] = 0.0;

    if (parts & ORACLE_PART_GLA) {
      hedgehog(qt, wq + (size_t)h * d * f2, d, f2, u, phq);
      hedgehog(kt, wk + (size_t)h * d * f2, d, f2, u, phk);
      const double *gt = g + (size_t)bh * f;
      for (int r = 0; r < f; ++r) {
        const double gam = gate_value(gt[r], gate_is_log);
        for (int c = 0; c < dv; ++c)
          S[(size_t)r * dv + c] = gam * S[(size_t)r * dv + c] + phk[r] * vt[c];
      }
      for (int c = 0; c < dv; ++c) {
        double acc = 0.0;
        for (int r = 0; r < f; ++r) acc += phq[r] * S[(size_t)r * dv + c];
        ot[c] += acc;
      }
    }
    /* the ring always receives the new token, so a later step can attend to it */
    const int slot = (int)(p % window);
    memcpy(kc + (size_t)slot * d, kt, sizeof(double) * d);
    memcpy(vc + (size_t)slot * dv, vt, sizeof(double) * dv);
    if (parts & ORACLE_PART_SWA) {
      const long long j0 = p - window + 1 > 0 ? p - window + 1 : 0;
      int n = 0;
      for (long long j = j0; j <= p; ++j, ++n) {
        const int sl = (int)(j % window);
        keys[n] = kc + (size_t)sl * d;
        vals[n] = vc + (size_t)sl * dv;
      }
      window_softmax(qt, keys, vals, n, d, dv, mh, n_meta, scale, s, sw);
      for (int c = 0; c < dv; ++c) ot[c] += sw[c];
    }
    free(u); free(phq); free(phk); free(s); free(sw); free(keys); free(vals);
  }
  return 0;
}

/* Number of OpenMP threads the oracle's parallel loops use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
