/*
 * fp64 CPU oracle for causal linear attention with an optional decay.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library or its kernels calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * What it computes is the plain definition, token by token, in double precision:
 *   textbook chapter 1.6 (long context and efficient attention), section "linear
 *   attention": the state S_t (d_v x d_k) gains the outer product v_t phi(k_t)^T at
 *   every step, the normaliser z_t gains phi(k_t), and the output is
 *   S_t phi(q_t) / (z_t^T phi(q_t)).  The chapter's recurrent code listing is the same
 *   loop without a decay.
 *   The decayed/gated generalisation S_t = G_t (.) S_{t-1} + v_t phi(k_t)^T, with G_t = 1,
 *   a per-head scalar gamma (RetNet retention) or a per-token, per-key gate alpha_t (GLA),
 *   is the one the FLA blog posts name (RetNet, GLA; "chunk" mode) and the same chapter's
 *   Mamba-2 remark (decay-masked linear attention).
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - the decay multiplies the old state first, then the current token is added
 *     undecayed; the initial state is decayed by the first token's gate;
 *   - a per-key gate alpha_t[c] scales key column c of S for every value row;
 *   - z decays with the same gate as S (z is S with v = 1);
 *   - elu is PyTorch's default (alpha = 1): x for x > 0, exp(x) - 1 otherwise;
 *   - no 1/sqrt(d) scale and no epsilon in the denominator.
 *
 * Inputs are widened exactly (bf16 -> fp32 -> fp64, fp32 -> fp64).  The state is
 * kept per (batch, head, block of 16 value rows) so the blocks run in parallel with
 * OpenMP; every value row sees the same operations in the same order whatever the
 * thread count.  Build without -ffast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_DECAY_NONE = 0, OR_DECAY_GAMMA = 1, OR_DECAY_GATE = 2, OR_DECAY_TOKEN = 3 };
enum { OR_PHI_ELU1 = 1, OR_NORMALIZE = 2 };

#define EBLK 16

static double widen(const void *p, int dtype, int64_t i) {
  if (dtype == OR_BF16) {
    uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)p)[i];
}

static double phi(double x, int elu1) {
  if (!elu1) return x;
  return x > 0.0 ? x + 1.0 : exp(x); /* elu(x) + 1 = exp(x) - 1 + 1 for x <= 0 */
}

/* Gate value g_t[c] of token t for head (b, h). */
static double gate_of(const float *decay, int kind, int64_t b, int64_t h, int64_t t,
                      int64_t c, int64_t H, int64_t T, int64_t dk) {
  switch (kind) {
  case OR_DECAY_GAMMA: return (double)decay[h];
  case OR_DECAY_GATE: return (double)decay[((b * H + h) * T + t) * dk + c];
  case OR_DECAY_TOKEN: return (double)decay[(b * H + h) * T + t];
  default: return 1.0;
  }
}

/*
 * oracle_fwd: the token-by-token recurrence.
 *   q, k: [B][H][T][dk]; v: [B][H][T][dv]; dtype OR_F32 or OR_BF16.
 *   decay: gamma [H], gate [B][H][T][dk] or per-token scalar gate [B][H][T] (fp32), or NULL.
 *   init: fp64 [B][H][dk][dv+n] (h = S^T, column dv holds z when normalising) or NULL.
 *   out: fp64 [B][H][nrows][dv] for the token indices listed in rows (ascending), or
 *        all T tokens when rows == NULL (then nrows must equal T).  May be NULL.
 *   final_state: fp64 [B][H][dk][dv+n] or NULL.  May alias init.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_fwd(const void *q, const void *k, const void *v, int dtype, const float *decay,
               int decay_kind, const double *init, double *out, const int64_t *rows,
               int64_t nrows, double *final_state, int64_t B, int64_t H, int64_t T,
               int64_t dk, int64_t dv, int flags, int nthreads) {
  if (!q || !k || !v || B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return -1;
  if (decay_kind != OR_DECAY_NONE && !decay) return -1;
  if (out && !rows && nrows != T) return -1;
  const int elu1 = (flags & OR_PHI_ELU1) != 0;
  const int norm = (flags & OR_NORMALIZE) != 0;
  const int64_t ncol = dv + (norm ? 1 : 0);
  const int64_t nblk = (dv + EBLK - 1) / EBLK;
  const int64_t ntask = B * H * nblk;

  double *init_copy = NULL;
  if (init && init == final_state) { /* in-place resume: read the old state first */
    size_t n = (size_t)(B * H * dk * ncol);
    init_copy = (double *)malloc(n * sizeof(double));
    if (!init_copy) return -1;
    memcpy(init_copy, init, n * sizeof(double));
    init = init_copy;
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < ntask; ++task) {
    const int64_t bh = task / nblk, eb = task % nblk;
    const int64_t b = bh / H, h = bh % H;
    const int64_t e0 = eb * EBLK, ne = (dv - e0) < EBLK ? (dv - e0) : EBLK;
    double *S = (double *)malloc(sizeof(double) * (size_t)(EBLK * dk)); /* S[e][c] */
    double *z = (double *)malloc(sizeof(double) * (size_t)dk);
    double *qb = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kb = (double *)malloc(sizeof(double) * (size_t)dk);
    double *g = (double *)malloc(sizeof(double) * (size_t)dk);
    if (!S || !z || !qb || !kb || !g) {
#pragma omp atomic write
      bad = 1;
      free(S); free(z); free(qb); free(kb); free(g);
      continue;
    }
    const double *h0 = init ? init + bh * dk * ncol : NULL;
    for (int64_t e = 0; e < ne; ++e)
      for (int64_t c = 0; c < dk; ++c) S[e * dk + c] = h0 ? h0[c * ncol + e0 + e] : 0.0;
    for (int64_t c = 0; c < dk; ++c) z[c] = (h0 && norm) ? h0[c * ncol + dv] : 0.0;

    int64_t next_row = 0; /* index into rows */
    for (int64_t t = 0; t < T; ++t) {
      const int64_t qk_off = (bh * T + t) * dk, v_off = (bh * T + t) * dv;
      for (int64_t c = 0; c < dk; ++c) {
        qb[c] = phi(widen(q, dtype, qk_off + c), elu1);
        kb[c] = phi(widen(k, dtype, qk_off + c), elu1);
        g[c] = gate_of(decay, decay_kind, b, h, t, c, H, T, dk);
      }
      /* S_t = G_t (.) S_{t-1} + v_t phi(k_t)^T  (decay first, then the new token) */
      for (int64_t e = 0; e < ne; ++e) {
        const double ve = widen(v, dtype, v_off + e0 + e);
        double *Se = S + e * dk;
        for (int64_t c = 0; c < dk; ++c) Se[c] = g[c] * Se[c] + ve * kb[c];
      }
      double den = 1.0;
      if (norm) {
        for (int64_t c = 0; c < dk; ++c) z[c] = g[c] * z[c] + kb[c];
        den = 0.0;
        for (int64_t c = 0; c < dk; ++c) den += z[c] * qb[c];
      }
      int64_t orow = -1;
      if (out) {
        if (!rows) orow = t;
        else if (next_row < nrows && rows[next_row] == t) orow = next_row++;
      }
      if (orow >= 0) {
        double *o = out + (bh * nrows + orow) * dv + e0;
        for (int64_t e = 0; e < ne; ++e) {
          const double *Se = S + e * dk;
          double num = 0.0;
          for (int64_t c = 0; c < dk; ++c) num += Se[c] * qb[c];
          o[e] = norm ? num / den : num;
        }
      }
    }
    if (final_state) {
      double *hf = final_state + bh * dk * ncol;
      for (int64_t e = 0; e < ne; ++e)
        for (int64_t c = 0; c < dk; ++c) hf[c * ncol + e0 + e] = S[e * dk + c];
      if (norm && eb == 0)
        for (int64_t c = 0; c < dk; ++c) hf[c * ncol + dv] = z[c];
    }
    free(S); free(z); free(qb); free(kb); free(g);
  }
  free(init_copy);
  return bad ? -1 : 0;
}

/*
 * oracle_step: one token of recurrent decoding, the T = 1 case of oracle_fwd with the
 * state updated in place.  q, k: [B][H][dk]; v: [B][H][dv]; decay: gamma [H],
 * gate [B][H][dk], per-token scalar [B][H] or NULL; state fp64 [B][H][dk][dv+n];
 * out fp64 [B][H][dv].
 */
int oracle_step(const void *q, const void *k, const void *v, int dtype, const float *decay,
                int decay_kind, double *state, double *out, int64_t B, int64_t H, int64_t dk,
                int64_t dv, int flags, int nthreads) {
  if (!state) return -1;
  return oracle_fwd(q, k, v, dtype, decay, decay_kind, state, out, NULL, 1, state, B, H, 1,
                    dk, dv, flags, nthreads);
}
