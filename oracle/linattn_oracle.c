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
 * Inputs are widened exactly (bf16 -> fp32 -> fp64, fp32 -> fp64; fp64 as is).  The state is
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

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 }; /* fp64: inputs the oracle itself derived */
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
  if (dtype == OR_F64) return ((const double *)p)[i];
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

/*
 * oracle_bwd: reverse-mode derivative of oracle_fwd (without the normaliser), by back-
 * propagation through time over the same recurrence, one head at a time.
 *
 * The loss is L = sum_t dout_t . o_t + sum dfinal (.) h_T with h_t = S_t^T [dk][dv] and
 * o_t = h_t^T phi(q_t).  Chain rule on h_t = diag(g_t) h_{t-1} + phi(k_t) v_t^T:
 *   dh_t   = phi(q_t) dout_t^T + diag(g_{t+1}) dh_{t+1}     (dh_{T-1} starts from dfinal)
 *   dphi(q_t) = h_t dout_t,  dphi(k_t) = dh_t v_t,  dv_t = dh_t^T phi(k_t),
 *   dg_t[c] = sum_e dh_t[c][e] h_{t-1}[c][e]  (h_{-1} = init),  dinit = diag(g_0) dh_0,
 * and dq = dphi(q) phi'(q), dk = dphi(k) phi'(k) with phi'(x) = 1 (identity) or
 * (x > 0 ? 1 : e^x) (elu + 1).  A per-token decay gathers dg over c; gamma over t, c and
 * the batch.
 *
 * The forward states h_t of one head are kept (T * dk * dv doubles), split into blocks
 * of 16 value columns that run in parallel; the sums over value columns (dq, dk, dg) are
 * taken block by block in a fixed order, so results do not depend on the thread count.
 *   dout: like v; dfinal, init: fp64 [B][H][dk][dv] or NULL.
 *   dq, dk: fp64 [B][H][T][dk]; dv: fp64 [B][H][T][dv]; dgate: fp64, shaped like the
 *   decay (gamma [H], gate [B][H][T][dk], token [B][H][T]) or NULL; dinit fp64
 *   [B][H][dk][dv] or NULL.  Returns 0, or -1 on bad arguments or memory.
 */
int oracle_bwd(const void *q, const void *k, const void *v, int dtype, const float *decay,
               int decay_kind, const double *init, const void *dout, const double *dfinal,
               double *dq, double *dk_out, double *dv_out, double *dgate, double *dinit,
               int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int flags,
               int nthreads) {
  if (!q || !k || !v || !dout || !dq || !dk_out || !dv_out) return -1;
  if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return -1;
  if (decay_kind != OR_DECAY_NONE && !decay) return -1;
  if (flags & OR_NORMALIZE) return -1;
  const int elu1 = (flags & OR_PHI_ELU1) != 0;
  const int64_t nblk = (dv + EBLK - 1) / EBLK;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  if (dgate && decay_kind == OR_DECAY_GAMMA)
    for (int64_t h = 0; h < H; ++h) dgate[h] = 0.0;
  /* per-head scratch: states per block [nblk][T][dk][EBLK], block partial sums */
  const size_t hs_n = (size_t)nblk * (size_t)T * (size_t)dk * EBLK;
  const size_t part_n = (size_t)nblk * (size_t)T * (size_t)dk;
  double *hs = (double *)malloc(sizeof(double) * (hs_n ? hs_n : 1));
  double *pq = (double *)malloc(sizeof(double) * (part_n ? part_n : 1));
  double *pk = (double *)malloc(sizeof(double) * (part_n ? part_n : 1));
  double *pg = (double *)malloc(sizeof(double) * (part_n ? part_n : 1));
  double *gall = (double *)malloc(sizeof(double) * (size_t)(T * dk > 0 ? T * dk : 1));
  if (!hs || !pq || !pk || !pg || !gall) {
    free(hs); free(pq); free(pk); free(pg); free(gall);
    return -1;
  }
  int bad = 0;
  for (int64_t bh = 0; bh < B * H && !bad; ++bh) {
    const int64_t b = bh / H, h = bh % H;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t c = 0; c < dk; ++c)
        gall[t * dk + c] = gate_of(decay, decay_kind, b, h, t, c, H, T, dk);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t eb = 0; eb < nblk; ++eb) {
      const int64_t e0 = eb * EBLK, ne = (dv - e0) < EBLK ? (dv - e0) : EBLK;
      double *hb = hs + (size_t)eb * (size_t)T * (size_t)dk * EBLK; /* [T][dk][EBLK] */
      double *S = (double *)malloc(sizeof(double) * (size_t)(dk * EBLK)); /* h[c][e] */
      double *dS = (double *)malloc(sizeof(double) * (size_t)(dk * EBLK));
      double *qb = (double *)malloc(sizeof(double) * (size_t)dk);
      double *kb = (double *)malloc(sizeof(double) * (size_t)dk);
      if (!S || !dS || !qb || !kb) {
#pragma omp atomic write
        bad = 1;
        free(S); free(dS); free(qb); free(kb);
        continue;
      }
      const double *h0 = init ? init + bh * dk * dv : NULL;
      for (int64_t c = 0; c < dk; ++c)
        for (int64_t e = 0; e < EBLK; ++e)
          S[c * EBLK + e] = (h0 && e < ne) ? h0[c * dv + e0 + e] : 0.0;
      /* forward: h_t for every t, and the block's share of dphi(q_t) = h_t dout_t */
      for (int64_t t = 0; t < T; ++t) {
        const int64_t qk_off = (bh * T + t) * dk, v_off = (bh * T + t) * dv;
        for (int64_t c = 0; c < dk; ++c) kb[c] = phi(widen(k, dtype, qk_off + c), elu1);
        for (int64_t c = 0; c < dk; ++c) {
          const double gc = gall[t * dk + c];
          double *Sc = S + c * EBLK;
          for (int64_t e = 0; e < ne; ++e)
            Sc[e] = gc * Sc[e] + kb[c] * widen(v, dtype, v_off + e0 + e);
        }
        memcpy(hb + (size_t)t * dk * EBLK, S, sizeof(double) * (size_t)(dk * EBLK));
        double *pqt = pq + ((size_t)eb * T + t) * dk;
        for (int64_t c = 0; c < dk; ++c) {
          double s = 0.0;
          for (int64_t e = 0; e < ne; ++e) s += S[c * EBLK + e] * widen(dout, dtype, v_off + e0 + e);
          pqt[c] = s;
        }
      }
      /* reverse: dh_t, then dphi(k_t), dv_t, dg_t from it */
      const double *dF = dfinal ? dfinal + bh * dk * dv : NULL;
      for (int64_t c = 0; c < dk; ++c)
        for (int64_t e = 0; e < EBLK; ++e)
          dS[c * EBLK + e] = (dF && e < ne) ? dF[c * dv + e0 + e] : 0.0;
      for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t qk_off = (bh * T + t) * dk, v_off = (bh * T + t) * dv;
        for (int64_t c = 0; c < dk; ++c) {
          qb[c] = phi(widen(q, dtype, qk_off + c), elu1);
          kb[c] = phi(widen(k, dtype, qk_off + c), elu1);
        }
        for (int64_t c = 0; c < dk; ++c)
          for (int64_t e = 0; e < ne; ++e)
            dS[c * EBLK + e] += qb[c] * widen(dout, dtype, v_off + e0 + e);
        double *pkt = pk + ((size_t)eb * T + t) * dk;
        double *pgt = pg + ((size_t)eb * T + t) * dk;
        const double *hprev = t > 0 ? hb + (size_t)(t - 1) * dk * EBLK : NULL;
        for (int64_t c = 0; c < dk; ++c) {
          double sk = 0.0, sg = 0.0;
          for (int64_t e = 0; e < ne; ++e) {
            const double d = dS[c * EBLK + e];
            sk += d * widen(v, dtype, v_off + e0 + e);
            sg += d * (hprev ? hprev[c * EBLK + e] : (h0 ? h0[c * dv + e0 + e] : 0.0));
          }
          pkt[c] = sk;
          pgt[c] = sg;
        }
        for (int64_t e = 0; e < ne; ++e) {
          double s = 0.0;
          for (int64_t c = 0; c < dk; ++c) s += dS[c * EBLK + e] * kb[c];
          dv_out[v_off + e0 + e] = s;
        }
        for (int64_t c = 0; c < dk; ++c) {
          const double gc = gall[t * dk + c];
          for (int64_t e = 0; e < ne; ++e) dS[c * EBLK + e] *= gc;
        }
      }
      if (dinit) {
        double *di = dinit + bh * dk * dv;
        for (int64_t c = 0; c < dk; ++c)
          for (int64_t e = 0; e < ne; ++e) di[c * dv + e0 + e] = dS[c * EBLK + e];
      }
      free(S); free(dS); free(qb); free(kb);
    }
    if (bad) break;
    /* gather the blocks in order; chain rule through phi */
    for (int64_t t = 0; t < T; ++t) {
      const int64_t qk_off = (bh * T + t) * dk;
      double gtok = 0.0;
      for (int64_t c = 0; c < dk; ++c) {
        double sq = 0.0, sk = 0.0, sg = 0.0;
        for (int64_t eb = 0; eb < nblk; ++eb) {
          const size_t i = ((size_t)eb * T + t) * dk + c;
          sq += pq[i];
          sk += pk[i];
          sg += pg[i];
        }
        const double xq = widen(q, dtype, qk_off + c), xk = widen(k, dtype, qk_off + c);
        const double fq = elu1 ? (xq > 0.0 ? 1.0 : exp(xq)) : 1.0;
        const double fk = elu1 ? (xk > 0.0 ? 1.0 : exp(xk)) : 1.0;
        dq[qk_off + c] = sq * fq;
        dk_out[qk_off + c] = sk * fk;
        if (dgate) {
          if (decay_kind == OR_DECAY_GATE) dgate[qk_off + c] = sg;
          else gtok += sg;
        }
      }
      if (dgate && decay_kind == OR_DECAY_TOKEN) dgate[bh * T + t] = gtok;
      if (dgate && decay_kind == OR_DECAY_GAMMA) dgate[h] += gtok;
    }
  }
  free(hs); free(pq); free(pk); free(pg); free(gall);
  return bad ? -1 : 0;
}

/*
 * oracle_gdn_fwd: the gated delta rule, token by token, in fp64 (textbook chapter 1.6,
 * section "gated delta rule"): with the unit-norm key k^_t = k_t / max(|k_t|, 1e-12),
 *     S_t = alpha_t S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T,   o_t = S_t q_t,
 * i.e. decay the memory, remove what it stores under k^_t (a beta_t share of the
 * prediction S k^_t) and write beta_t v_t there.  q is used as given.  The state is kept
 * as h = S^T ([dk][dv]); value rows of S (columns e of h) evolve independently, so blocks
 * of 16 of them run in parallel.
 *   q, k: [B][H][T][dk]; v: [B][H][T][dv] (fp32 or bf16 bits); alpha, beta: fp32 [B][H][T].
 *   init, final_state: fp64 [B][H][dk][dv] or NULL (final may alias init).
 *   out: fp64 [B][H][T][dv] or NULL.  Returns 0, or -1 on bad arguments or memory.
 */
int oracle_gdn_fwd(const void *q, const void *k, const void *v, int dtype, const float *alpha,
                   const float *beta, const double *init, double *out, double *final_state,
                   int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int nthreads) {
  if (!q || !k || !v || !alpha || !beta || B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return -1;
  const int64_t nblk = (dv + EBLK - 1) / EBLK;
  const int64_t ntask = B * H * nblk;
  double *init_copy = NULL;
  if (init && init == final_state) {
    size_t n = (size_t)(B * H * dk * dv);
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
    const int64_t e0 = eb * EBLK, ne = (dv - e0) < EBLK ? (dv - e0) : EBLK;
    double *S = (double *)malloc(sizeof(double) * (size_t)(EBLK * dk)); /* S[e][c] */
    double *kh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *qv = (double *)malloc(sizeof(double) * (size_t)dk);
    if (!S || !kh || !qv) {
#pragma omp atomic write
      bad = 1;
      free(S); free(kh); free(qv);
      continue;
    }
    const double *h0 = init ? init + bh * dk * dv : NULL;
    for (int64_t e = 0; e < ne; ++e)
      for (int64_t c = 0; c < dk; ++c) S[e * dk + c] = h0 ? h0[c * dv + e0 + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const int64_t qk_off = (bh * T + t) * dk, v_off = (bh * T + t) * dv;
      double nrm = 0.0;
      for (int64_t c = 0; c < dk; ++c) {
        kh[c] = widen(k, dtype, qk_off + c);
        qv[c] = widen(q, dtype, qk_off + c);
        nrm += kh[c] * kh[c];
      }
      nrm = sqrt(nrm);
      const double den = nrm > 1e-12 ? nrm : 1e-12;
      for (int64_t c = 0; c < dk; ++c) kh[c] /= den;
      const double al = (double)alpha[bh * T + t], be = (double)beta[bh * T + t];
      for (int64_t e = 0; e < ne; ++e) {
        double *Se = S + e * dk;
        double pred = 0.0; /* (S_{t-1} k^)_e */
        for (int64_t c = 0; c < dk; ++c) pred += Se[c] * kh[c];
        const double ve = widen(v, dtype, v_off + e0 + e);
        for (int64_t c = 0; c < dk; ++c)
          Se[c] = al * (Se[c] - be * pred * kh[c]) + be * ve * kh[c];
      }
      if (out) {
        double *o = out + (bh * T + t) * dv + e0;
        for (int64_t e = 0; e < ne; ++e) {
          const double *Se = S + e * dk;
          double s = 0.0;
          for (int64_t c = 0; c < dk; ++c) s += Se[c] * qv[c];
          o[e] = s;
        }
      }
    }
    if (final_state) {
      double *hf = final_state + bh * dk * dv;
      for (int64_t e = 0; e < ne; ++e)
        for (int64_t c = 0; c < dk; ++c) hf[c * dv + e0 + e] = S[e * dk + c];
    }
    free(S); free(kh); free(qv);
  }
  free(init_copy);
  return bad ? -1 : 0;
}
