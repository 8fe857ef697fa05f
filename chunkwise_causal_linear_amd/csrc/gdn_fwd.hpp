// Gated delta rule, chunkwise forward — gfx950 kernel.
//
// Recurrence (textbook chapter 1.6, section "gated delta rule"), with the unit-norm key
// k^_t = k_t / max(|k_t|, 1e-12) and h = S^T (dk x dv):
//     h_t = alpha_t (I - beta_t k^_t k^_t^T) h_{t-1} + beta_t k^_t v_t^T,   o_t = h_t^T q_t.
// Written as h_t = alpha_t h_{t-1} + k^_t u_t^T with the pseudo-value
// u_t = beta_t (v_t - alpha_t h_{t-1}^T k^_t), one chunk of L rows starting from state H,
// with g the inclusive product of alpha inside the chunk, satisfies
//     (I + A) U = diag(beta) V - diag(beta g) K^ H,   A_tj = beta_t (g_t / g_j) k^_t . k^_j (j < t),
// so with T = (I + A)^-1 (unit lower triangular), W = T diag(beta g) K^ and
// U0 = T diag(beta) V:
//     U = U0 - W H,
//     O = diag(g) Q H + (M (.) Q K^^T) U,        M_tj = g_t / g_j (j <= t),
//     H <- g_L H + K^^T diag(g_L / g) U.
// One workgroup (4 waves) owns one (b, h, 64-wide slice of dv); wave w owns value columns
// 16w..16w+15 of the slice, whose state rows live in MFMA accumulators for the whole
// sequence.  Per chunk: k normalised and the decay scanned while the tiles go to LDS;
// K^ K^^T on MFMA gives A; the 16 x 16 diagonal blocks of T are inverted by forward
// substitution (one wave each), the off-diagonal blocks follow block row by block row with
// fp32 MFMA; then W, U0, the score tiles, U, the outputs and the state on bf16 (or fp32)
// MFMA.  The next chunk's inputs are prefetched into registers meanwhile.
#pragma once

#include "chunk_bwd.hpp" // shared MFMA / LDS fragment helpers

namespace fla {

struct GdnArgs {
  const void *q, *k, *v;
  const float *alpha, *beta; // [B][H][T] each
  const float *init;         // [B][H][dk][dv] or null
  float *fin;                // [B][H][dk][dv] or null
  void *out;                 // [B][H][T][dv]
  int64_t T;
  int H, dv;
  int nvs;                   // 64-wide value slices
  int nunits;                // B * H * nvs
};

template <typename TIn, int DK>
struct GdnCfg {
  static constexpr int C = 64, XW = 64, NT = 256;
  static constexpr int ES = sizeof(TIn);
  static constexpr int VE = 16 / ES;
  static constexpr int KU = ES == 2 ? 32 : 16;
  static constexpr int LDK = DK + VE;  // Q, K^, W rows
  static constexpr int LDV = XW + VE;  // V, U, Us rows
  static constexpr int LDT = C + VE;   // Tb, Tg rows
  static constexpr int NVQ = C * DK / VE / NT;  // 16-byte vectors per thread (q, k)
  static constexpr int NVV = C * XW / VE / NT;  // (v slice)
  static constexpr int VPRQ = DK / VE;          // vectors per q/k row
  static_assert(NVQ >= 1 && NVV >= 1 && VPRQ <= 64, "tile shape");
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + C * LDK * ES;
  static constexpr int OFF_W = OFF_K + C * LDK * ES;
  static constexpr int OFF_V = OFF_W + C * LDK * ES;
  static constexpr int OFF_TB = OFF_V + C * LDV * ES;
  static constexpr int OFF_TG = OFF_TB + C * LDT * ES;
  static constexpr int OFF_R = OFF_TG + C * LDT * ES;  // region: A, T (fp32), later U, Us, P
  static constexpr int R_FP32 = 2 * C * C * 4;
  static constexpr int R_LATE = 2 * C * LDV * ES + 16 * 256 * ES;
  static constexpr int R_BYTES = R_FP32 > R_LATE ? R_FP32 : R_LATE;
  static constexpr int OFF_AF = OFF_R;                   // A, fp32 [C][C]
  static constexpr int OFF_TF = OFF_R + C * C * 4;       // T, fp32 [C][C]
  static constexpr int OFF_U = OFF_R;                    // U [C][LDV]
  static constexpr int OFF_US = OFF_U + C * LDV * ES;    // U (.) g_L / g
  static constexpr int OFF_P = OFF_US + C * LDV * ES;    // masked scores, 16 tile images
  static constexpr int OFF_G = OFF_R + R_BYTES;          // g [C], beta [C]
  static constexpr int OFF_BETA = OFF_G + C * 4;
  static constexpr int LDS = OFF_BETA + C * 4;
  static constexpr bool FITS = LDS <= kMaxLds;
};

template <typename TIn, int DK>
__global__ void __launch_bounds__(256) gdn_fwd_kernel(GdnArgs a) {
  using K = GdnCfg<TIn, DK>;
  constexpr int C = K::C, XW = K::XW, VE = K::VE, KU = K::KU;
  constexpr int LDK = K::LDK, LDV = K::LDV, LDT = K::LDT;
  constexpr int NCB = DK / 16;   // state row blocks
  __shared__ __attribute__((aligned(16))) unsigned char lds[K::LDS];
  TIn *sQ = reinterpret_cast<TIn *>(lds + K::OFF_Q);
  TIn *sK = reinterpret_cast<TIn *>(lds + K::OFF_K);
  TIn *sW = reinterpret_cast<TIn *>(lds + K::OFF_W);
  TIn *sV = reinterpret_cast<TIn *>(lds + K::OFF_V);
  TIn *sTb = reinterpret_cast<TIn *>(lds + K::OFF_TB);
  TIn *sTg = reinterpret_cast<TIn *>(lds + K::OFF_TG);
  float *sAf = reinterpret_cast<float *>(lds + K::OFF_AF);
  float *sTf = reinterpret_cast<float *>(lds + K::OFF_TF);
  TIn *sU = reinterpret_cast<TIn *>(lds + K::OFF_U);
  TIn *sUs = reinterpret_cast<TIn *>(lds + K::OFF_US);
  TIn *sP = reinterpret_cast<TIn *>(lds + K::OFF_P);
  float *sG = reinterpret_cast<float *>(lds + K::OFF_G);
  float *sBeta = reinterpret_cast<float *>(lds + K::OFF_BETA);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, li = lane & 15;

  // unit -> (b h, value slice); sibling slices of one head on the same XCD (ids = mod 8)
  int unit = blockIdx.x;
  if ((a.nunits & 7) == 0) unit = (unit & 7) * (a.nunits >> 3) + (unit >> 3);
  const int vs = unit % a.nvs;
  const int64_t bh = unit / a.nvs;
  const int64_t T = a.T;
  const int dv = a.dv;
  const int e_base = vs * XW;
  const int nchunks = (int)((T + C - 1) / C);
  const TIn *gq = static_cast<const TIn *>(a.q) + bh * T * DK;
  const TIn *gk = static_cast<const TIn *>(a.k) + bh * T * DK;
  const TIn *gv = static_cast<const TIn *>(a.v) + bh * T * dv;
  TIn *gout = static_cast<TIn *>(a.out) + bh * T * dv;
  const float *galpha = a.alpha + bh * T, *gbeta = a.beta + bh * T;

  auto chunk_len = [&](int n) -> int {
    const int64_t l = T - (int64_t)n * C;
    return (int)(l < C ? l : C);
  };

  // ---- register prefetch of one chunk -----------------------------------------------
  uint32_t rq[K::NVQ][4], rk[K::NVQ][4], rv[K::NVV][4];
  float ralpha = 1.f, rbeta = 0.f;
  auto load = [&](int n) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;
#pragma unroll
    for (int j = 0; j < K::NVQ; ++j) {
      const int vi = tid + 256 * j, r = vi / K::VPRQ, c = (vi % K::VPRQ) * VE;
      uint4 x = make_uint4(0, 0, 0, 0), y = x;
      if (r < L) {
        x = *reinterpret_cast<const uint4 *>(gq + (t0 + r) * DK + c);
        y = *reinterpret_cast<const uint4 *>(gk + (t0 + r) * DK + c);
      }
      rq[j][0] = x.x; rq[j][1] = x.y; rq[j][2] = x.z; rq[j][3] = x.w;
      rk[j][0] = y.x; rk[j][1] = y.y; rk[j][2] = y.z; rk[j][3] = y.w;
    }
    constexpr int VPRV = XW / VE;
#pragma unroll
    for (int j = 0; j < K::NVV; ++j) {
      const int vi = tid + 256 * j, r = vi / VPRV, c = (vi % VPRV) * VE;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (r < L && e_base + c < dv) x = *reinterpret_cast<const uint4 *>(gv + (t0 + r) * dv + e_base + c);
      rv[j][0] = x.x; rv[j][1] = x.y; rv[j][2] = x.z; rv[j][3] = x.w;
    }
    ralpha = 1.f;
    rbeta = 0.f;
    if (tid < L) {
      ralpha = galpha[t0 + tid];
      rbeta = gbeta[t0 + tid];
    }
  };

  // ---- state: H[c][e], e = e_base + 16 wave + li; tile cb holds rows 16cb + 4g + q ----
  const int e_lane = e_base + 16 * wave + li;
  f32x4 Hs[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int c = 16 * cb + 4 * g + qq;
      Hs[cb][qq] = (a.init && e_lane < dv) ? a.init[(bh * DK + c) * dv + e_lane] : 0.f;
    }

  if (nchunks > 0) load(0);

  for (int n = 0; n < nchunks; ++n) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;

    // ---- P0: tiles; k normalised per row; decay scan ---------------------------------
#pragma unroll
    for (int j = 0; j < K::NVQ; ++j) {
      const int vi = tid + 256 * j, r = vi / K::VPRQ, c = (vi % K::VPRQ) * VE;
      float fk[VE];
      unpack<TIn, VE>(fk, rk[j]);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) ss += fk[e] * fk[e];
      // the row's VPRQ vectors sit in VPRQ consecutive lanes
#pragma unroll
      for (int d = 1; d < K::VPRQ; d <<= 1) ss += __shfl_xor(ss, d);
      const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
      for (int e = 0; e < VE; ++e) fk[e] *= inv;
      st_lds<TIn, VE>(sK + r * LDK + c, fk);
      st_words_lds<4>(sQ + r * LDK + c, rq[j]);
    }
    {
      constexpr int VPRV = XW / VE;
#pragma unroll
      for (int j = 0; j < K::NVV; ++j) {
        const int vi = tid + 256 * j, r = vi / VPRV, c = (vi % VPRV) * VE;
        st_words_lds<4>(sV + r * LDV + c, rv[j]);
      }
    }
    if (wave == 0) {
      float x = ralpha; // rows past L carry alpha = 1, beta = 0
      for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(x, d);
        if (lane >= d) x *= o;
      }
      sG[lane] = x;
      sBeta[lane] = rbeta;
    }
    __syncthreads();
    const float gL = sG[C - 1]; // = g[L-1]

    // ---- P1: A = strictly lower (beta_t g_t / g_j) k^_t . k^_j, fp32 ------------------
    // tile (tb, jb), jb <= tb: 10 tiles over 4 waves
    static_for<0, 16>([&](auto I) {
      constexpr int tb = I / 4, jb = I % 4;
      if constexpr (jb <= tb) {
        constexpr int pos = tb * (tb + 1) / 2 + jb;
        if (pos % 4 == wave) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const TIn *at = sK + (16 * tb + li) * LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
          const TIn *bj = sK + (16 * jb + li) * LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
#pragma unroll
          for (int u = 0; u < DK / KU; ++u)
            acc = mma(acc, ld_frag_c_at<TIn, true>(bj, u, g), ld_frag_c_at<TIn, true>(at, u, g));
          // acc[qq] = k^_j . k^_t with j = 16 jb + 4g + qq, t = 16 tb + li
          const int t = 16 * tb + li;
          const float bt = sBeta[t] * sG[t];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int j = 16 * jb + 4 * g + qq;
            sAf[t * C + j] = (j < t) ? bt / sG[j] * acc[qq] : 0.f;
          }
        }
      }
    });
    __syncthreads();

    // ---- P2: diagonal blocks of T = (I + A)^-1 by forward substitution ----------------
    if (li == lane) { // lanes 0..15 of every wave: wave w inverts diagonal block w
      const int base = 16 * wave;
      float col[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == li) ? 1.f : 0.f;
#pragma unroll
        for (int kk = 0; kk < i; ++kk) s -= sAf[(base + i) * C + base + kk] * col[kk];
        col[i] = (i < li) ? 0.f : s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sTf[(base + i) * C + base + li] = col[i];
    }
    __syncthreads();

    // ---- P3: off-diagonal blocks, block row by block row:
    //      T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj), wave j computes block (i, j)
    static_for<1, 4>([&](auto IB) {
      constexpr int ib = IB;
      if (wave < ib) {
        const int jb = wave;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        for (int kb = jb; kb < ib; ++kb) {
          // A operand: A[16ib + li][16kb + 4g + r]; B operand: T[16kb + 4g + r][16jb + li]
          const f32x4 fa = *reinterpret_cast<const f32x4 *>(sAf + (16 * ib + li) * C + 16 * kb + 4 * g);
          const float *tb = sTf + (16 * kb + 4 * g) * C + 16 * jb + li;
          const f32x4 fb = {tb[0], tb[C], tb[2 * C], tb[3 * C]};
          x = mma(x, fa, fb);
        }
        // x[qq] = X[16ib-local row 4g + qq][col li]: as a B operand (k = 4g + qq)
        const f32x4 ft = *reinterpret_cast<const f32x4 *>(sTf + (16 * ib + li) * C + 16 * ib + 4 * g);
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        y = mma(y, ft, x);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) sTf[(16 * ib + 4 * g + qq) * C + 16 * jb + li] = -y[qq];
      }
      __syncthreads();
    });

    // ---- P4: Tb = T diag(beta), Tg = T diag(beta g) in the MFMA input type ---------------
#pragma unroll
    for (int i = 0; i < C * C / 256; ++i) {
      const int idx = tid + 256 * i, t = idx / C, j = idx % C;
      const float tv = (j <= t) ? sTf[t * C + j] : 0.f;
      const float bj = sBeta[j];
      sTb[t * LDT + j] = (TIn)(tv * bj);
      sTg[t * LDT + j] = (TIn)(tv * bj * sG[j]);
    }
    // next chunk's inputs go out now; P0 of the next iteration consumes them
    if (n + 1 < nchunks) load(n + 1);
    __syncthreads();

    // ---- P5: W = Tg K^ (all dk columns), U0 = Tb V (this wave's columns), masked scores
    constexpr int NZU = C / KU;
    f32x4 U0[4];
    {
      // W tiles (tb, cb): 4 * NCB tiles over the 4 waves
#pragma unroll
      for (int ti = 0; ti < NCB; ++ti) {
        const int tile = wave * NCB + ti, tb = tile / NCB, cb = tile % NCB;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const TIn *ta = sTg + (16 * tb + li) * LDT + 4 * g;
#pragma unroll
        for (int u = 0; u < NZU; ++u)
          acc = mma(acc, ld_frag_at<TIn, true>(ta, u), ld_frag_t<TIn, true>(sK, LDK, 16 * cb, u, g, li));
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) sW[(16 * tb + 4 * g + qq) * LDK + 16 * cb + li] = (TIn)acc[qq];
      }
      Frag<TIn> vf[NZU];
#pragma unroll
      for (int u = 0; u < NZU; ++u) vf[u] = ld_frag_t<TIn, true>(sV, LDV, 16 * wave, u, g, li);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const TIn *ta = sTb + (16 * tb + li) * LDT + 4 * g;
#pragma unroll
        for (int u = 0; u < NZU; ++u) acc = mma(acc, ld_frag_at<TIn, true>(ta, u), vf[u]);
        U0[tb] = acc;
      }
      // score tiles P[t][j] = (g_t / g_j) q_t . k^_j, j <= t; image of tile (tb, jb) is
      // row-major [t][j]
      static_for<0, 16>([&](auto I) {
        constexpr int tb = I / 4, jb = I % 4;
        if constexpr (jb <= tb) {
          constexpr int pos = tb * (tb + 1) / 2 + jb;
          if (pos % 4 == wave) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const TIn *kj = sK + (16 * jb + li) * LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
            const TIn *qt = sQ + (16 * tb + li) * LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
#pragma unroll
            for (int u = 0; u < DK / KU; ++u)
              acc = mma(acc, ld_frag_c_at<TIn, true>(kj, u, g), ld_frag_c_at<TIn, true>(qt, u, g));
            // acc[qq]: j = 16 jb + 4g + qq, t = 16 tb + li
            const int t = 16 * tb + li;
            const float gt = sG[t];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int j = 16 * jb + 4 * g + qq;
              acc[qq] = (j <= t) ? gt / sG[j] * acc[qq] : 0.f;
            }
            st_ptile<TIn>(sP + I * 256 + li * 16 + 4 * g, acc);
          }
        }
      });
    }
    __syncthreads();

    // ---- P6: U = U0 - W H (this wave's columns); U and U (.) g_L / g to LDS ------------
    {
      Frag<TIn> hf[DK / KU];
#pragma unroll
      for (int u = 0; u < DK / KU; ++u) {
        if constexpr (sizeof(TIn) == 2) hf[u] = acc_frag_bf(Hs[2 * u], Hs[2 * u + 1]);
        else hf[u] = Hs[u];
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        const TIn *wa = sW + (16 * tb + li) * LDK + 4 * g;
#pragma unroll
        for (int u = 0; u < DK / KU; ++u) x = mma(x, ld_frag_at<TIn, true>(wa, u), hf[u]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int t = 16 * tb + 4 * g + qq;
          const float uval = U0[tb][qq] - x[qq];
          sU[t * LDV + 16 * wave + li] = (TIn)uval;
          sUs[t * LDV + 16 * wave + li] = (TIn)(uval * (gL / sG[t]));
        }
      }
    }
    __syncthreads();

    // ---- P7: O = (masked scores) U + diag(g) Q H --------------------------------------
    {
      Frag<TIn> uf[NZU];
#pragma unroll
      for (int u = 0; u < NZU; ++u) uf[u] = ld_frag_t<TIn, true>(sU, LDV, 16 * wave, u, g, li);
      Frag<TIn> hf[DK / KU];
#pragma unroll
      for (int u = 0; u < DK / KU; ++u) {
        if constexpr (sizeof(TIn) == 2) hf[u] = acc_frag_bf(Hs[2 * u], Hs[2 * u + 1]);
        else hf[u] = Hs[u];
      }
      static_for<0, 4>([&](auto TB) {
        constexpr int tb = TB;
        f32x4 oi = {0.f, 0.f, 0.f, 0.f};
        static_for<0, NZU>([&](auto U) {
          constexpr int u = U;
          if constexpr (sizeof(TIn) == 2) {
            constexpr int TA = (2 * u <= tb) ? tb * 4 + 2 * u : -1;
            constexpr int TB2 = (2 * u + 1 <= tb) ? tb * 4 + 2 * u + 1 : -1;
            if constexpr (TA >= 0 || TB2 >= 0)
              oi = mma(oi, ld_ptile2<TIn, TA, TB2>(sP + li * 16 + 4 * g), uf[u]);
          } else {
            constexpr int TA = (u <= tb) ? tb * 4 + u : -1;
            if constexpr (TA >= 0) oi = mma(oi, ld_ptile2<TIn, TA, -1>(sP + li * 16 + 4 * g), uf[u]);
          }
        });
        f32x4 ox = {0.f, 0.f, 0.f, 0.f};
        const TIn *qa = sQ + (16 * tb + li) * LDK + 4 * g;
#pragma unroll
        for (int u = 0; u < DK / KU; ++u) ox = mma(ox, ld_frag_at<TIn, true>(qa, u), hf[u]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int t = 16 * tb + 4 * g + qq;
          const float o = oi[qq] + sG[t] * ox[qq];
          if (t < L && e_lane < dv) gout[(t0 + t) * dv + e_lane] = (TIn)o;
        }
      });
    }

    // ---- P8: H <- g_L H + K^^T (U (.) g_L / g) -----------------------------------------
    {
      Frag<TIn> usf[NZU];
#pragma unroll
      for (int u = 0; u < NZU; ++u) usf[u] = ld_frag_t<TIn, true>(sUs, LDV, 16 * wave, u, g, li);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 hnew = Hs[cb] * gL;
#pragma unroll
        for (int u = 0; u < NZU; ++u)
          hnew = mma(hnew, ld_frag_t<TIn, true>(sK, LDK, 16 * cb, u, g, li), usf[u]);
        Hs[cb] = hnew;
      }
    }
    __syncthreads();
  }

  if (a.fin && e_lane < dv) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) a.fin[(bh * DK + 16 * cb + 4 * g + qq) * dv + e_lane] = Hs[cb][qq];
  }
}

} // namespace fla
