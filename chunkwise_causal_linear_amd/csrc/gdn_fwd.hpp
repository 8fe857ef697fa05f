// Gated delta rule, chunkwise forward — gfx950 kernels.
//
// Recurrence (textbook chapter 1.6, section "gated delta rule"), with the unit-norm key
// k^_t = k_t / max(|k_t|, 1e-12) and h = S^T (dk x dv):
//     h_t = alpha_t (I - beta_t k^_t k^_t^T) h_{t-1} + beta_t k^_t v_t^T,   o_t = h_t^T q_t.
// Written as h_t = alpha_t h_{t-1} + k^_t u_t^T with the pseudo-value
// u_t = beta_t (v_t - alpha_t h_{t-1}^T k^_t), one chunk of L rows starting from state H,
// with g the inclusive product of alpha inside the chunk, satisfies
//     (I + A) U = diag(beta) V - diag(beta g) K^ H,   A_tj = beta_t (g_t / g_j) k^_t . k^_j (j < t),
// so with T = (I + A)^-1 (unit lower triangular) and Tb = T diag(beta):
//     U = Tb (V - diag(g) K^ H),
//     O = diag(g) Q H + (M (.) Q K^^T) U,        M_tj = g_t / g_j (j <= t),
//     H <- g_L H + K^^T diag(g_L / g) U.
// The ratios g_t / g_j (t >= j) are formed from g kept as a mantissa in [0.5, 1) and an
// integer exponent, as ldexp(m_t / m_j, e_t - e_j): exact for any decay in [0, 1] however
// long its product underflows fp32 (a ratio is then only ever rounded or flushed to zero
// where it is negligible), where g_t * (1 / g_j) would overflow (textbook chapter 1.6,
// "gated delta rule": a decay near 0 clears the memory).  Plain g (<= 1) is used as is.
// K^ = diag(rn) K with rn_t = 1 / max(|k_t|, 1e-12) is never formed: the kernels multiply
// the keys as given and apply rn to the products' rows or columns in fp32.
// Tb does not depend on the state, so it is formed for every chunk at once by a
// pre-pass (one workgroup per (b, h, chunk): K K^T on MFMA, scaled, gives A; the 16 x 16 diagonal
// blocks of T are inverted by forward substitution, one wave each, and the off-diagonal
// blocks follow block row by block row with fp32 MFMA), written to a workspace in the input
// type.  The state pass streams the chunks, one workgroup per (b, h, 64-wide slice of dv):
// four consumer waves keep the state columns in MFMA accumulators and compute per chunk
// the masked scores, X = K^ H, W = V - diag(g) X (in registers, fp32, rounded once), U = Tb W,
// the outputs and the state update, while four producer waves stage the next chunk's q, k,
// rn, Tb and value slice.
#pragma once

#include "chunk_bwd.hpp" // shared MFMA / LDS fragment helpers

namespace fla {

struct GdnArgs {
  const void *q, *k, *v;
  const float *alpha, *beta; // [B][H][T] each
  const float *init;         // [B][H][dk][dv] or null
  float *fin;                // [B][H][dk][dv] or null
  void *out;                 // [B][H][T][dv]
  void *tb;                  // workspace [B][H][nch][kGdnTbElems], input type: T diag(beta)
                             // per chunk, its lower-triangle 16 x 16 blocks (see tri_vec)
  int64_t T;
  int H, dv;
  int nvs;                   // 64-wide value slices
  int nch;                   // chunks per (b, h)
  int nunits;                // state pass: B * H * nvs; pre-pass: B * H * nch
};

// Tb per chunk in the workspace: the 10 blocks (bi, bj), bj <= bi, of its 64 x 64 lower
// triangle in 16 x 16 blocks, block b = bi (bi + 1) / 2 + bj at b * 256, row-major inside
// (the blocks above the diagonal are zero and are neither stored nor multiplied).
constexpr int kGdnTbElems = 10 * 256;

template <typename TIn, int DK>
struct GdnCfg {
  static constexpr int C = 64, XW = 64, NT = 256;
  static constexpr int ES = sizeof(TIn);
  static constexpr int VE = 16 / ES;
  static constexpr int KU = ES == 2 ? 32 : 16;
  static constexpr int LDK = DK + VE;  // Q, K^ rows
  static constexpr int LDV = XW + VE;  // V, U, Us rows
  static constexpr int LDT = C + VE;   // Tb rows
  static constexpr int NVQ = C * DK / VE / NT;  // 16-byte vectors per thread (q, k)
  static constexpr int NVV = C * XW / VE / NT;  // (v slice)
  static constexpr int VPRQ = DK / VE;          // vectors per q/k row
  static constexpr int NCB = DK / 16;           // 16-row blocks of the state
  static constexpr int NZU = C / KU;            // K units over the chunk rows
  static_assert(NVQ >= 1 && NVV >= 1 && VPRQ <= 64, "tile shape");
  // pre-pass LDS: A (fp32), replaced block by block by T, over K^
  static constexpr int cmax(int x, int y) { return x > y ? x : y; }
  static constexpr int P_K = 0;
  // A, fp32 [C][C], over K^ (whose last reader is A itself: the tiles wait in registers
  // for a barrier), replaced block by block by T = (I + A)^-1; Tb is formed from T
  // in registers as they are written out
  static constexpr int P_A = P_K;
  static constexpr int P_G = P_K + cmax(C * LDK * ES, C * C * 4);    // g [C], beta [C]
  static constexpr int P_BETA = P_G + C * 4;
  static constexpr int P_GM = P_BETA + C * 4;                         // g = m 2^e: m [C]
  static constexpr int P_GMI = P_GM + C * 4;                          // 1 / m [C]
  static constexpr int P_GE = P_GMI + C * 4;                          // e [C] (int)
  static constexpr int P_RN = P_GE + C * 4;                          // 1 / |k| [C]
  static constexpr int P_LDS = P_RN + C * 4;
  // state-pass LDS: two input stages {q, k, g, m, 1/m, e, rn} (producer waves fill one while the
  // consumer waves read the other); one {Tb, V slice} buffer, which the consumers use
  // before the chunk's first barrier and the producers refill after it; the score tiles
  static constexpr int S_Q = 0;
  static constexpr int S_K = S_Q + C * LDK * ES;
  static constexpr int S_G = S_K + C * LDK * ES;    // g [C]
  static constexpr int S_GM = S_G + C * 4;          // g = m 2^e: m [C], 1 / m [C], e [C]
  static constexpr int S_GMI = S_GM + C * 4;
  static constexpr int S_GE = S_GMI + C * 4;
  static constexpr int S_RN = S_GE + C * 4;         // 1 / |k| [C]
  static constexpr int S_STAGE = S_RN + C * 4;
  static constexpr int S_TB = 2 * S_STAGE;          // Tb [C][LDT]
  static constexpr int S_V = S_TB + C * LDT * ES;   // V slice [C][LDV]
  static constexpr int S_P = S_V + C * LDV * ES;    // masked scores, 16 tile images
  // bf16: the scores' rounding remainders (hi + lo operands of O = P U, see the state pass)
  static constexpr int S_PL = S_P + 16 * 256 * ES;
  static constexpr int NV_TB = kGdnTbElems / VE;    // 16-byte vectors of a chunk's Tb
  static constexpr int NVT = (NV_TB + NT - 1) / NT; // per thread (the last ones partly idle)
  static constexpr int S_LDS = S_PL + (ES == 2 ? 16 * 256 * ES : 0);
  static constexpr bool FITS = P_LDS <= kMaxLds && S_LDS <= kMaxLds;
};

namespace gdn {

// Vector vi of a chunk's stored Tb (kGdnTbElems elements, VE per vector): its row r and
// first column c in the 64 x 64 tile.  vi must be below kGdnTbElems / VE.
template <int VE>
__device__ __forceinline__ void tri_vec(int vi, int &r, int &c) {
  constexpr int VPB = 16 / VE;                  // vectors per block row
  const int b = vi / (16 * VPB), w = vi % (16 * VPB);
  const int bi = b >= 6 ? 3 : b >= 3 ? 2 : b >= 1 ? 1 : 0;
  const int bj = b - bi * (bi + 1) / 2;
  r = 16 * bi + w / VPB;
  c = 16 * bj + (w % VPB) * VE;
}

// k rows of one chunk (registers, 16-byte vectors in row-major order) into LDS as they
// are, and rn[r] = 1 / max(|k_r|, 1e-12) (0 for a zero row): the unit key is
// k^ = rn k, and every product with it takes rn as an fp32 row or column scale after the
// MFMA, so k^ is never rounded to the input type (a bf16 k^ put 9e-3 of error into the
// final state where consecutive keys are nearly parallel).  The VPRQ vectors of a row sit
// in VPRQ consecutive lanes, which reduce its squared norm.
template <typename TIn, int DK>
__device__ __forceinline__ void stage_k(const uint32_t (*rk)[4], TIn *sK, float *rn, int tid) {
  using K = GdnCfg<TIn, DK>;
  constexpr int VE = K::VE;
#pragma unroll
  for (int j = 0; j < K::NVQ; ++j) {
    const int vi = tid + 256 * j, r = vi / K::VPRQ, c = (vi % K::VPRQ) * VE;
    float fk[VE];
    unpack<TIn, VE>(fk, rk[j]);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) ss += fk[e] * fk[e];
#pragma unroll
    for (int d = 1; d < K::VPRQ; d <<= 1) ss += __shfl_xor(ss, d);
    if (c == 0) rn[r] = ss > 0.f ? 1.f / fmaxf(sqrtf(ss), 1e-12f) : 0.f;
    st_words_lds<4>(sK + r * K::LDK + c, rk[j]);
  }
}

// Raw tile rows (registers) into LDS.
template <typename TIn, int NV, int VPR, int LD>
__device__ __forceinline__ void stage_raw(const uint32_t (*rx)[4], TIn *s, int tid) {
  constexpr int VE = 16 / sizeof(TIn);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = tid + 256 * j, r = vi / VPR, c = (vi % VPR) * VE;
    st_words_lds<4>(s + r * LD + c, rx[j]);
  }
}

// The chunk's decays as seen by the kernels: g (inclusive product of alpha down the chunk)
// and the same product as m 2^e (m in [0.5, 1), e an integer that does not underflow).
struct Decays {
  float *g, *m, *mi; // g, m, 1 / m  [C]
  int *e;            // e [C]
  // g_t / g_j for t >= j
  __device__ float ratio(int t, int j) const { return ldexpf(m[t] * mi[j], e[t] - e[j]); }
};

// g = inclusive product of alpha down the chunk (one wave; rows past the end carry 1),
// written to g[], m[], mi[], e[] at the lane's row.  alpha = 0 is taken as 2^-65536 (the
// products that cross it are then zero after ldexp, the others exact).
__device__ __forceinline__ void decay_scan(float alpha, int lane, float *g, float *m, float *mi,
                                           int *e) {
  int ex = 0;
  float mx = frexpf(alpha, &ex);
  if (!(alpha > 0.f)) { mx = 0.5f; ex = -65536; }
  for (int d = 1; d < 64; d <<= 1) {
    const float om = __shfl_up(mx, d);
    const int oe = __shfl_up(ex, d);
    if (lane >= d) {
      int k = 0;
      mx = frexpf(mx * om, &k);
      ex += oe + k;
    }
  }
  m[lane] = mx;
  mi[lane] = 1.f / mx;
  e[lane] = ex;
  g[lane] = ldexpf(mx, ex);
}

// Masked score tiles P[t][j] = (g_t / g_j) q_t . k^_j = (g_t / g_j) rn_j q_t . k_j (j <= t),
// as accumulator images (lane
// l of a tile owns elements 4l .. 4l + 3); 10 tiles over the 4 waves.  bf16: sPl receives
// each element's rounding remainder P - bf16(P), also in bf16.
template <typename TIn, int DK>
__device__ __forceinline__ void scores(const TIn *sQ, const TIn *sK, const float *rn,
                                       const Decays &dec, TIn *sP, TIn *sPl, int wave, int g,
                                       int li) {
  using K = GdnCfg<TIn, DK>;
  static_for<0, 16>([&](auto I) {
    constexpr int tb = I / 4, jb = I % 4;
    if constexpr (jb <= tb) {
      constexpr int pos = tb * (tb + 1) / 2 + jb;
      if (pos % 4 == wave) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const TIn *kj = sK + (16 * jb + li) * K::LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
        const TIn *qt = sQ + (16 * tb + li) * K::LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
#pragma unroll
        for (int u = 0; u < DK / K::KU; ++u)
          acc = mma(acc, ld_frag_c_at<TIn, true>(kj, u, g), ld_frag_c_at<TIn, true>(qt, u, g));
        // acc[qq]: j = 16 jb + 4g + qq, t = 16 tb + li
        const int t = 16 * tb + li;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int j = 16 * jb + 4 * g + qq;
          acc[qq] = (j <= t) ? dec.ratio(t, j) * rn[j] * acc[qq] : 0.f;
        }
        st_ptile<TIn>(sP + I * 256 + (16 * g + li) * 4, acc);
        if constexpr (sizeof(TIn) == 2) {
          f32x4 lo;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) lo[qq] = acc[qq] - (float)(__bf16)acc[qq];
          st_ptile<TIn>(sPl + I * 256 + (16 * g + li) * 4, lo);
        }
      }
    }
  });
}

} // namespace gdn

// ---- pre-pass: Tb of one chunk ---------------------------------------------------
template <typename TIn, int DK>
__global__ void __launch_bounds__(256) gdn_prep_kernel(GdnArgs a) {
  using K = GdnCfg<TIn, DK>;
  constexpr int C = K::C, XW = K::XW, VE = K::VE, KU = K::KU, NCB = K::NCB, NZU = K::NZU;
  constexpr int LDK = K::LDK;
  __shared__ __attribute__((aligned(16))) unsigned char lds[K::P_LDS];
  TIn *sK = reinterpret_cast<TIn *>(lds + K::P_K);
  float *sA = reinterpret_cast<float *>(lds + K::P_A);
  float *sT = sA; // T overwrites A: each block of A is dead once its block of T is known
  float *sG = reinterpret_cast<float *>(lds + K::P_G);
  float *sBeta = reinterpret_cast<float *>(lds + K::P_BETA);
  float *sGm = reinterpret_cast<float *>(lds + K::P_GM);
  float *sGmi = reinterpret_cast<float *>(lds + K::P_GMI);
  int *sGe = reinterpret_cast<int *>(lds + K::P_GE);
  float *sRn = reinterpret_cast<float *>(lds + K::P_RN);
  const gdn::Decays dec{sG, sGm, sGmi, sGe};

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int n = blockIdx.x % a.nch;
  const int64_t bh = blockIdx.x / a.nch;
  const int64_t T = a.T, t0 = (int64_t)n * C;
  const int L = (int)((T - t0) < C ? (T - t0) : C);
  const TIn *gk = static_cast<const TIn *>(a.k) + (bh * T + t0) * DK;

  // Every input of the chunk (k, the decay, beta) is requested before the first wait, from
  // clamped rows without a branch, so one memory round trip covers them; rows past the
  // end are masked where the values are used.
  {
    uint32_t rk[K::NVQ][4];
#pragma unroll
    for (int j = 0; j < K::NVQ; ++j) {
      const int vi = tid + 256 * j, r = vi / K::VPRQ, c = (vi % K::VPRQ) * VE;
      const uint4 y = *reinterpret_cast<const uint4 *>(gk + (r < L ? r : L - 1) * DK + c);
      rk[j][0] = y.x; rk[j][1] = y.y; rk[j][2] = y.z; rk[j][3] = y.w;
    }
    float al = 1.f, be = 0.f;
    if (wave == 0) {
      const int64_t tl = bh * T + t0 + (lane < L ? lane : L - 1);
      al = a.alpha[tl];
      be = a.beta[tl];
    }
#pragma unroll
    for (int j = 0; j < K::NVQ; ++j) {
      const int r = (tid + 256 * j) / K::VPRQ;
      if (r >= L) rk[j][0] = rk[j][1] = rk[j][2] = rk[j][3] = 0u; // past the end: k = 0
    }
    gdn::stage_k<TIn, DK>(rk, sK, sRn, tid);
    if (wave == 0) {
      gdn::decay_scan(lane < L ? al : 1.f, lane, sG, sGm, sGmi, sGe); // past the end: alpha 1, beta 0
      sBeta[lane] = lane < L ? be : 0.f;
    }
  }
  __syncthreads();

  // A = strictly lower (beta_t g_t / g_j) k^_t . k^_j = (beta_t g_t / g_j) rn_t rn_j k_t . k_j,
  // fp32: tile k = tb (tb + 1) / 2 + jb
  // (jb <= tb, 10 tiles) is wave k % 4's slot k / 4; the tiles wait in registers until
  // every wave has read K^, whose LDS they then take
  f32x4 atile[3];
#pragma unroll
  for (int sl = 0; sl < 3; ++sl) {
    const int k = 4 * sl + wave;
    if (k < 10) {
      const int tb = k >= 6 ? 3 : k >= 3 ? 2 : k >= 1 ? 1 : 0, jb = k - tb * (tb + 1) / 2;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const TIn *at = sK + (16 * tb + li) * LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
      const TIn *bj = sK + (16 * jb + li) * LDK + (sizeof(TIn) == 2 ? 8 : 4) * g;
#pragma unroll
      for (int u = 0; u < DK / KU; ++u)
        acc = mma(acc, ld_frag_c_at<TIn, true>(bj, u, g), ld_frag_c_at<TIn, true>(at, u, g));
      atile[sl] = acc;
    }
  }
  __syncthreads();
#pragma unroll
  for (int sl = 0; sl < 3; ++sl) {
    const int k = 4 * sl + wave;
    if (k < 10) {
      const int tb = k >= 6 ? 3 : k >= 3 ? 2 : k >= 1 ? 1 : 0, jb = k - tb * (tb + 1) / 2;
      // atile[sl][qq] = k_j . k_t with j = 16 jb + 4g + qq, t = 16 tb + li
      const int t = 16 * tb + li;
      const float bt = sBeta[t] * sRn[t];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int jj = 16 * jb + 4 * g + qq;
        sA[t * C + jj] = (jj < t) ? bt * dec.ratio(t, jj) * sRn[jj] * atile[sl][qq] : 0.f;
      }
    }
  }
  __syncthreads();

  // diagonal blocks of T = (I + A)^-1 by forward substitution: lanes 0..15 of wave w
  // invert block w, one column each (all of the block's reads precede its writes: one wave)
  if (li == lane) {
    const int base = 16 * wave;
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == li) ? 1.f : 0.f;
#pragma unroll
      for (int kk = 0; kk < i; ++kk) s -= sA[(base + i) * C + base + kk] * col[kk];
      col[i] = (i < li) ? 0.f : s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[(base + i) * C + base + li] = col[i];
  }
  __syncthreads();

  // off-diagonal blocks, block row by block row: T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj),
  // wave j computes block (i, j); block (i, j) of A is read by the waves j' <= j of the
  // same row, so every result waits in registers for the row's barrier before it replaces
  // its block of A
  static_for<1, 4>([&](auto IB) {
    constexpr int ib = IB;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (wave < ib) {
      const int jb = wave;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int kb = jb; kb < ib; ++kb) {
        // A operand: A[16ib + li][16kb + 4g + r]; B operand: T[16kb + 4g + r][16jb + li]
        const f32x4 fa = *reinterpret_cast<const f32x4 *>(sA + (16 * ib + li) * C + 16 * kb + 4 * g);
        const float *tb = sT + (16 * kb + 4 * g) * C + 16 * jb + li;
        const f32x4 fb = {tb[0], tb[C], tb[2 * C], tb[3 * C]};
        x = mma(x, fa, fb);
      }
      // x[qq] = X[row 4g + qq][col li]: a B operand with k = 4g + qq
      const f32x4 ft = *reinterpret_cast<const f32x4 *>(sT + (16 * ib + li) * C + 16 * ib + 4 * g);
      y = mma(y, ft, x);
    }
    __syncthreads();
    if (wave < ib) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) sT[(16 * ib + 4 * g + qq) * C + 16 * wave + li] = -y[qq];
    }
    __syncthreads();
  });

  // Tb = T diag(beta) to the workspace in the input type, formed from T in registers:
  // element (t, j) = T_tj beta_j, rounded once; T's upper triangle (never written) is
  // masked by j <= t.  The lower-triangle blocks of the C x C tile (their columns past the
  // end are zero: beta = 0 there), 16-byte vectors in the stored order (tri_vec).
  auto t_scaled4 = [&](int t, int j0) -> f32x4 {
    const f32x4 tv = *reinterpret_cast<const f32x4 *>(sT + t * C + j0);
    const f32x4 bv = *reinterpret_cast<const f32x4 *>(sBeta + j0);
    f32x4 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = ((j0 + s <= t) ? tv[s] : 0.f) * bv[s];
    return r;
  };
  auto put = [&](TIn *dst, int r, int c) {
    if constexpr (sizeof(TIn) == 2) {
      const f32x4 lo = t_scaled4(r, c), hi = t_scaled4(r, c + 4);
      const bf16x8 v = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                        (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
      *reinterpret_cast<bf16x8 *>(dst) = v;
    } else {
      *reinterpret_cast<f32x4 *>(dst) = t_scaled4(r, c);
    }
  };
  {
    const int64_t off = (bh * a.nch + n) * kGdnTbElems;
    TIn *gtb = static_cast<TIn *>(a.tb) + off;
#pragma unroll
    for (int j = 0; j < K::NVT; ++j) {
      const int vi = tid + 256 * j;
      if (vi < K::NV_TB) {
        int r, c;
        gdn::tri_vec<VE>(vi, r, c);
        put(gtb + vi * VE, r, c);
      }
    }
  }
}

// ---- state pass ---------------------------------------------------------------------------
// 8 waves: waves 4..7 (producers) load q and k of chunk n+1 into registers, take k's reciprocal norms
// and write them, with the chunk's decay, into one LDS stage, and after the mid-chunk
// barrier stage Tb and the value slice of the chunk the consumers take next, while waves
// 0..3 (consumers) compute chunk n (scores, X = K^ H, U = Tb (V - diag(g) X), outputs, state
// update) from the other stage; two barriers per chunk.
template <typename TIn, int DK>
__global__ void __launch_bounds__(512) gdn_state_kernel(GdnArgs a) {
  using K = GdnCfg<TIn, DK>;
  constexpr int C = K::C, XW = K::XW, VE = K::VE, KU = K::KU, NCB = K::NCB, NZU = K::NZU;
  constexpr int LDK = K::LDK, LDV = K::LDV;
  __shared__ __attribute__((aligned(16))) unsigned char lds[K::S_LDS];
  auto stage_q = [&](int s) { return reinterpret_cast<TIn *>(lds + s * K::S_STAGE + K::S_Q); };
  auto stage_k = [&](int s) { return reinterpret_cast<TIn *>(lds + s * K::S_STAGE + K::S_K); };
  auto stage_rn = [&](int s) { return reinterpret_cast<float *>(lds + s * K::S_STAGE + K::S_RN); };
  auto stage_dec = [&](int s) {
    unsigned char *b = lds + s * K::S_STAGE;
    return gdn::Decays{reinterpret_cast<float *>(b + K::S_G), reinterpret_cast<float *>(b + K::S_GM),
                       reinterpret_cast<float *>(b + K::S_GMI), reinterpret_cast<int *>(b + K::S_GE)};
  };
  TIn *sTb = reinterpret_cast<TIn *>(lds + K::S_TB);
  TIn *sV = reinterpret_cast<TIn *>(lds + K::S_V);
  TIn *sP = reinterpret_cast<TIn *>(lds + K::S_P);
  TIn *sPl = reinterpret_cast<TIn *>(lds + K::S_PL); // bf16 only

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
  const int nchunks = a.nch;
  auto chunk_len = [&](int n) -> int {
    const int64_t l = T - (int64_t)n * C;
    return (int)(l < C ? l : C);
  };

  if (wave >= 4) {
    // =========================== producer waves ===========================
    const int ptid = tid - 256, pwave = wave - 4;
    const TIn *gq = static_cast<const TIn *>(a.q) + bh * T * DK;
    const TIn *gk = static_cast<const TIn *>(a.k) + bh * T * DK;
    const float *galpha = a.alpha + bh * T;
    const TIn *gtb = static_cast<const TIn *>(a.tb) + bh * nchunks * kGdnTbElems;
    const TIn *gv = static_cast<const TIn *>(a.v) + bh * T * dv + vs * XW;
    // Two register sets of one chunk each: the loads of chunk n + 3 go out while chunk
    // n + 2's are still in flight and chunk n + 1 is staged.  Every load is unconditional
    // (the chunk index and its rows are clamped into the sequence), so the compiler's wait
    // counts stay exact across the loop; rows past a chunk's end are masked when staged.
    // Staging one chunk past the end writes a buffer no consumer reads again.
    uint32_t rq[2][K::NVQ][4], rk[2][K::NVQ][4];
    uint32_t rtb[2][K::NVT][4], rv[2][K::NVV][4];
    float ralpha[2] = {1.f, 1.f};
    auto clamp_n = [&](int n) { return n < nchunks ? n : nchunks - 1; };
    // Tb and the value slice of chunk n
    auto load_tv = [&](auto S, int n) {
      constexpr int s = decltype(S)::value;
      n = clamp_n(n);
      const int L = chunk_len(n);
      const int64_t t0 = (int64_t)n * C;
      // (idle vector slots load the chunk's last vector again and store it again)
#pragma unroll
      for (int j = 0; j < K::NVT; ++j) {
        int vi = ptid + 256 * j;
        vi = vi < K::NV_TB ? vi : K::NV_TB - 1;
        const uint4 x = *reinterpret_cast<const uint4 *>(gtb + (int64_t)n * kGdnTbElems + vi * VE);
        rtb[s][j][0] = x.x; rtb[s][j][1] = x.y; rtb[s][j][2] = x.z; rtb[s][j][3] = x.w;
      }
#pragma unroll
      for (int j = 0; j < K::NVV; ++j) {
        const int vi = ptid + 256 * j, r = vi / (XW / VE), c = (vi % (XW / VE)) * VE;
        const uint4 x = *reinterpret_cast<const uint4 *>(gv + (t0 + (r < L ? r : L - 1)) * dv + c);
        rv[s][j][0] = x.x; rv[s][j][1] = x.y; rv[s][j][2] = x.z; rv[s][j][3] = x.w;
      }
    };
    auto stage_tv = [&](auto S, int n) {
      constexpr int s = decltype(S)::value;
      const int L = chunk_len(clamp_n(n));
#pragma unroll
      for (int j = 0; j < K::NVT; ++j) {
        int vi = ptid + 256 * j, r, c;
        vi = vi < K::NV_TB ? vi : K::NV_TB - 1;
        gdn::tri_vec<VE>(vi, r, c);
        st_words_lds<4>(sTb + r * K::LDT + c, rtb[s][j]);
      }
#pragma unroll
      for (int j = 0; j < K::NVV; ++j) {
        const int vi = ptid + 256 * j, r = vi / (XW / VE), c = (vi % (XW / VE)) * VE;
        const uint32_t m = r < L ? ~0u : 0u;
        const uint32_t w[4] = {rv[s][j][0] & m, rv[s][j][1] & m, rv[s][j][2] & m, rv[s][j][3] & m};
        st_words_lds<4>(sV + r * LDV + c, w);
      }
    };
    // q, k rows and the decay of chunk n
    auto load = [&](auto S, int n) {
      constexpr int s = decltype(S)::value;
      n = clamp_n(n);
      const int L = chunk_len(n);
      const int64_t t0 = (int64_t)n * C;
#pragma unroll
      for (int j = 0; j < K::NVQ; ++j) {
        const int vi = ptid + 256 * j, r = vi / K::VPRQ, c = (vi % K::VPRQ) * VE;
        const int64_t row = t0 + (r < L ? r : L - 1);
        const uint4 x = *reinterpret_cast<const uint4 *>(gq + row * DK + c);
        const uint4 y = *reinterpret_cast<const uint4 *>(gk + row * DK + c);
        rq[s][j][0] = x.x; rq[s][j][1] = x.y; rq[s][j][2] = x.z; rq[s][j][3] = x.w;
        rk[s][j][0] = y.x; rk[s][j][1] = y.y; rk[s][j][2] = y.z; rk[s][j][3] = y.w;
      }
      ralpha[s] = galpha[t0 + (ptid < L ? ptid : L - 1)];
    };
    // rows past the chunk's end: q = k = 0 and alpha = 1 (no decay)
    auto stage = [&](auto S, int n) {
      constexpr int s = decltype(S)::value;
      const int L = chunk_len(clamp_n(n));
#pragma unroll
      for (int j = 0; j < K::NVQ; ++j) {
        const uint32_t m = (ptid + 256 * j) / K::VPRQ < L ? ~0u : 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rq[s][j][e] &= m;
          rk[s][j][e] &= m;
        }
      }
      const int buf = n & 1;
      gdn::stage_k<TIn, DK>(rk[s], stage_k(buf), stage_rn(buf), ptid);
      gdn::stage_raw<TIn, K::NVQ, K::VPRQ, LDK>(rq[s], stage_q(buf), ptid);
      if (pwave == 0) {
        const gdn::Decays d = stage_dec(buf);
        gdn::decay_scan(ptid < L ? ralpha[s] : 1.f, lane, d.g, d.m, d.mi, d.e);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (nchunks > 0) {
      load(I0{}, 0);
      load_tv(I0{}, 0);
      load(I1{}, 1);
      load_tv(I1{}, 1);
      stage(I0{}, 0);
      stage_tv(I0{}, 0);
      load(I0{}, 2);
      load_tv(I0{}, 2);
    }
    __syncthreads();
    // chunk n + 1 sits in set (n + 1) & 1; its loads went out two chunks earlier
    auto step = [&](auto S, int n) {
      stage(S, n + 1);
      load(S, n + 3);
      __syncthreads(); // consumers: scores and U of chunk n formed (Tb, V read)
      stage_tv(S, n + 1);
      load_tv(S, n + 3);
      __syncthreads(); // consumers: chunk n done; the next stage is complete
    };
    for (int n = 0; n < nchunks; n += 2) {
      step(I1{}, n);
      if (n + 1 < nchunks) step(I0{}, n + 1);
    }
    return;
  }

  // =========================== consumer waves ===========================
  const int e_lane = vs * XW + 16 * wave + li; // this lane's value column
  TIn *gout = static_cast<TIn *>(a.out) + bh * T * dv;

  // the output rows of a chunk: buffer stores over its L rows, so rows past the end are
  // dropped without a branch (with a branch the compiler cannot count the stores in
  // flight and waits for all of them before the next chunk's loads)
  auto out_rsrc = [&](int64_t t0, int L) { return make_rsrc(gout + t0 * dv, L * dv * K::ES); };
  const int e4 = vs * XW + 16 * wave + 4 * g; // this lane's 4 output columns (transposed tiles)

  // state: H[c][e_lane]; tile cb holds rows 16cb + 4g + q
  f32x4 Hs[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int c = 16 * cb + 4 * g + qq;
      Hs[cb][qq] = (a.init && e_lane < dv) ? a.init[(bh * DK + c) * dv + e_lane] : 0.f;
    }
  // the state's loads complete here, not at a wait inside the loop (which, with vmcnt
  // counting in order, would also wait for the previous chunk's stores)
  __builtin_amdgcn_s_waitcnt(0);

  __syncthreads();

  for (int n = 0; n < nchunks; ++n) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;
    const TIn *sQ = stage_q(n & 1);
    const TIn *sK = stage_k(n & 1);
    const float *sRn = stage_rn(n & 1);
    const gdn::Decays dec = stage_dec(n & 1);
    const float *sG = dec.g;
    const float gL = sG[C - 1]; // = g[L-1]: rows past the end carry alpha = 1

    // ---- masked scores (shared by the consumer waves); U = Tb (V - diag(g) K^ H) (this
    // wave's columns)
    gdn::scores<TIn, DK>(sQ, sK, sRn, dec, sP, sPl, wave, g, li);
    Frag<TIn> hf[DK / KU];
#pragma unroll
    for (int u = 0; u < DK / KU; ++u) {
      if constexpr (sizeof(TIn) == 2) hf[u] = acc_frag_bf(Hs[2 * u], Hs[2 * u + 1]);
      else hf[u] = Hs[u];
    }
    // X, U and U (.) g_L / g stay in accumulator tiles: two 16-row tiles are the MFMA
    // operand of a 32-row K unit (rows 32u + 4g + s and +16 of column li), so no LDS round
    // trip
    auto frag_of = [&](const f32x4 *tiles, int u) -> Frag<TIn> {
      if constexpr (sizeof(TIn) == 2) return acc_frag_bf(tiles[2 * u], tiles[2 * u + 1]);
      else return tiles[u];
    };
    f32x4 xacc[4]; // X = K^ H
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      const TIn *ka = sK + (16 * tb + li) * LDK + 4 * g;
#pragma unroll
      for (int u = 0; u < DK / KU; ++u) x = mma(x, ld_frag_at<TIn, true>(ka, u), hf[u]);
      xacc[tb] = x;
    }
    f32x4 uacc[4], usacc[4];
    // W = V - diag(g) X as the B operand of Tb W (K = the chunk's rows): the value slice's
    // fragment and X's accumulator tiles share the row order (rows 32u + 4g + s, + 16), so
    // W is formed element by element in fp32 and rounded once
    Frag<TIn> wf[NZU];
#pragma unroll
    for (int u = 0; u < NZU; ++u) {
      const Frag<TIn> vf = ld_frag_t<TIn, true>(sV, LDV, 16 * wave, u, g, li);
      constexpr int NS = sizeof(TIn) == 2 ? 8 : 4;
      float w[8];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int half = sizeof(TIn) == 2 ? (s >> 2) : 0;
        const int row = (sizeof(TIn) == 2 ? 32 * u + 16 * half : 16 * u) + 4 * g + (s & 3);
        const float x = xacc[sizeof(TIn) == 2 ? 2 * u + half : u][s & 3];
        w[s] = (float)vf[s] - sG[row] * sRn[row] * x; // X = K^ H = diag(rn) K H
      }
      wf[u] = frag_from<TIn>(w);
    }
    // only Tb's lower-triangle blocks are in LDS: row block tb takes column blocks <= tb
    static_for<0, 4>([&](auto TBI) {
      constexpr int tb = decltype(TBI)::value;
      f32x4 u0 = {0.f, 0.f, 0.f, 0.f};
      const TIn *ta = sTb + (16 * tb + li) * K::LDT + 4 * g;
      static_for<0, NZU>([&](auto UI) {
        constexpr int u = decltype(UI)::value;
        if constexpr (sizeof(TIn) == 2) {
          // K unit u = column blocks 2u (low half of the fragment) and 2u + 1 (high half)
          if constexpr (2 * u + 1 <= tb) u0 = mma(u0, ld_frag_at<TIn, true>(ta, u), wf[u]);
          else if constexpr (2 * u <= tb) u0 = mma(u0, ld_frag_at<TIn, false>(ta, u), wf[u]);
        } else {
          if constexpr (u <= tb) u0 = mma(u0, ld_frag_at<TIn, true>(ta, u), wf[u]);
        }
      });
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int t = 16 * tb + 4 * g + qq;
        uacc[tb][qq] = u0[qq];
        usacc[tb][qq] = u0[qq] * dec.ratio(C - 1, t) * sRn[t]; // K^T (.) = K^T diag(rn) (.)
      }
    });
    __syncthreads(); // every consumer wave's score tiles written

    // ---- O = (masked scores) U + diag(g) Q H -------------------------------------------
    // bf16: P and U enter as hi + lo pairs (P U ~ Ph Uh + Ph Ul + Pl Uh).  Where writes
    // nearly cancel (near-parallel keys with beta ~ 1) U is a small difference of large
    // terms and the output a sum of many such U rows with almost equal scores, so single
    // bf16 roundings of P and U cost about 1e-2 of the output's scale; the pairs keep their
    // error near that of the other roundings (k^, Tb, W, the H operand).
    {
      Frag<TIn> uf[NZU], ufl[NZU];
#pragma unroll
      for (int u = 0; u < NZU; ++u) uf[u] = frag_of(uacc, u);
      if constexpr (sizeof(TIn) == 2) {
        f32x4 ulo[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) ulo[tb][qq] = uacc[tb][qq] - (float)(__bf16)uacc[tb][qq];
#pragma unroll
        for (int u = 0; u < NZU; ++u) ufl[u] = frag_of(ulo, u);
      }
      // formed transposed (O^T = U^T P^T + H^T Q^T: the same fragments with the operands
      // swapped), so a lane holds 4 adjacent value columns of one row: one 8-byte store
      const auto rs = out_rsrc(t0, L);
      static_for<0, 4>([&](auto TB) {
        constexpr int tb = TB;
        f32x4 oi = {0.f, 0.f, 0.f, 0.f};
        static_for<0, NZU>([&](auto U) {
          constexpr int u = U;
          if constexpr (sizeof(TIn) == 2) {
            constexpr int TA = (2 * u <= tb) ? tb * 4 + 2 * u : -1;
            constexpr int TB2 = (2 * u + 1 <= tb) ? tb * 4 + 2 * u + 1 : -1;
            if constexpr (TA >= 0 || TB2 >= 0) {
              const Frag<TIn> ph = ld_ptile2<TIn, TA, TB2>(sP + (16 * g + li) * 4);
              oi = mma(oi, uf[u], ph);
              oi = mma(oi, ufl[u], ph);
              oi = mma(oi, uf[u], ld_ptile2<TIn, TA, TB2>(sPl + (16 * g + li) * 4));
            }
          } else {
            constexpr int TA = (u <= tb) ? tb * 4 + u : -1;
            if constexpr (TA >= 0) oi = mma(oi, uf[u], ld_ptile2<TIn, TA, -1>(sP + (16 * g + li) * 4));
          }
        });
        f32x4 ox = {0.f, 0.f, 0.f, 0.f};
        const TIn *qa = sQ + (16 * tb + li) * LDK + 4 * g;
#pragma unroll
        for (int u = 0; u < DK / KU; ++u) ox = mma(ox, hf[u], ld_frag_at<TIn, true>(qa, u));
        // oi[qq], ox[qq]: row t = 16 tb + li, value column e4 + qq
        const int t = 16 * tb + li;
        const float gt = sG[t];
        f32x4 o;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) o[qq] = oi[qq] + gt * ox[qq];
        st_out4_buf<TIn>(rs, (t * dv + e4) * K::ES, 0, o);
      });
    }

    // ---- H <- g_L H + K^^T (U (.) g_L / g) = g_L H + K^T (U (.) rn g_L / g) ----------------
    // bf16: the scaled U enters as a hi + lo pair, for the reason given for P U above (its
    // single rounding alone put 5e-3 of error into the final state there)
    {
      Frag<TIn> usf[NZU], usfl[NZU];
#pragma unroll
      for (int u = 0; u < NZU; ++u) usf[u] = frag_of(usacc, u);
      if constexpr (sizeof(TIn) == 2) {
        f32x4 uslo[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) uslo[tb][qq] = usacc[tb][qq] - (float)(__bf16)usacc[tb][qq];
#pragma unroll
        for (int u = 0; u < NZU; ++u) usfl[u] = frag_of(uslo, u);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 hnew = Hs[cb] * gL;
#pragma unroll
        for (int u = 0; u < NZU; ++u) {
          const Frag<TIn> kf = ld_frag_t<TIn, true>(sK, LDK, 16 * cb, u, g, li);
          hnew = mma(hnew, kf, usf[u]);
          if constexpr (sizeof(TIn) == 2) hnew = mma(hnew, kf, usfl[u]);
        }
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
