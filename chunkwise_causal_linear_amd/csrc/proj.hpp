// Input side of a linear-attention layer: the q / k / v projections of the activations
// with the feature map fused into the same kernel (the FLA Triton post fuses the Q/K/V
// projections with the phi computation; the FLA guide's layers map x [B][T][hidden] to
// per-head q, k, v).  One GEMM per projection,
//     Y[m][n] = phi( sum_c X[m][c] W[c][n] ),   m = b T + t,  n = h d + j,
// so Y is already the token-major [B][T][H][d] layout the chunk kernel reads.  X [M][K]
// and W [K][N] are row-major in the input type; accumulation in fp32 on MFMA
// (v_mfma_f32_16x16x32_bf16, or 16x16x4 for fp32 inputs), phi (identity or elu + 1) and
// the rounding to the input type in the epilogue.
//
// Tiles: 256 x 128 outputs per workgroup of 4 waves (2 x 2, 128 x 64 each: 32 accumulator
// tiles; fp32 128 x 128), K in steps of 32 through two LDS stages; A fragments are row reads of the
// row-major X tile, B fragments transposed reads of the row-major W tile (the split K
// convention of chunk_fwd.hpp for both).  The next K step's tiles are loaded into
// registers while the current one is multiplied.
//
// One launch covers the three projections (they share X).  Tile order: each XCD (blocks
// id, id + 8, ... run on XCD id mod 8) takes a contiguous range of the logical tile order,
// which walks groups of GM row tiles and, inside a group, every column tile of the three
// projections with the row tile fastest: the XCD's resident workgroups then share a few X
// row tiles and W column tiles through its L2, where the plain row-major order made every
// XCD read all of X (X fetched 8 times per projection).
#pragma once

#include "chunk_fwd.hpp"

namespace fla {

struct ProjArgs {
  const void *x;     // [M][K]
  const void *w[3];  // [K][n[p]] per projection
  void *y[3];        // [M][n[p]]
  int64_t M;
  int K;
  int n[3];          // columns per projection
  int nbn[3];        // column tiles per projection (a zero skips the projection)
  int elu_mask;      // bit p: phi = elu + 1 on projection p
};
constexpr int kProjGroup = 8; // row tiles per group of the tile order

template <typename TIn>
struct ProjCfg {
  // bf16: 256 x 128 tiles, each wave 128 x 64 (8 x 4 accumulator tiles), so every 16-byte
  // operand fragment read from LDS feeds 4 or 8 MFMAs; fp32 keeps 128 x 128 (64 x 64 per
  // wave) for its registers
  static constexpr int ES = sizeof(TIn);
  static constexpr int BM = ES == 2 ? 256 : 128, BN = 128, BK = 32, NT = 256;
  static constexpr int MI = BM / 32;       // 16-row fragments per wave (wave rows BM / 2)
  static constexpr int VE = 16 / ES;
  static constexpr int LA = BK + VE;       // X tile row stride (elements)
  static constexpr int LB = BN + VE;       // W tile row stride
  static constexpr int A_VEC = BM * BK / VE / NT;  // 16-byte vectors per thread
  static constexpr int B_VEC = BK * BN / VE / NT;
  static constexpr int A_VPR = BK / VE, B_VPR = BN / VE;
  static constexpr int KU = ES == 2 ? 32 : 16;     // K per fragment
  static constexpr int NKU = BK / KU;
  static constexpr int STAGE = (BM * LA + BK * LB); // elements
  static_assert(A_VEC >= 1 && B_VEC >= 1, "tile shape");
};

template <typename TIn>
__global__ __launch_bounds__(256, 2) void proj_phi_kernel(ProjArgs a) {
  using P = ProjCfg<TIn>;
  using F = Frag<TIn>;
  constexpr int BM = P::BM, BN = P::BN, BK = P::BK, VE = P::VE, LA = P::LA, LB = P::LB;
  constexpr int MI = P::MI;
  constexpr int GM = kProjGroup;
  __shared__ __attribute__((aligned(16))) TIn lds[2 * P::STAGE];

  // logical tile of this block (see the tile order above)
  const int nbn_t = a.nbn[0] + a.nbn[1] + a.nbn[2];
  const int64_t nbm = (a.M + BM - 1) / BM;
  const int64_t total = nbm * nbn_t;
  const int64_t per = (total + 7) / 8;
  const int64_t L = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (L >= total) return;
  const int64_t grp = L / ((int64_t)GM * nbn_t);
  const int64_t mbase = grp * GM;
  const int gm = (int)(nbm - mbase < GM ? nbm - mbase : GM);
  const int64_t lin = L - grp * GM * nbn_t;
  int nt = (int)(lin / gm), p = 0;
  while (p < 2 && nt >= a.nbn[p]) {
    nt -= a.nbn[p];
    ++p;
  }
  const int N = a.n[p];
  const int64_t m0 = (mbase + lin % gm) * BM;
  const int n0 = nt * BN;
  const bool elu = ((a.elu_mask >> p) & 1) != 0;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * 64; // this wave's BM/2 x 64 block
  const TIn *X = static_cast<const TIn *>(a.x);
  const TIn *W = static_cast<const TIn *>(a.w[p]);

  uint32_t ra[P::A_VEC][4], rb[P::B_VEC][4];
  // rows past M and columns past N read a clamped in-range vector (discarded at the end)
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < P::A_VEC; ++j) {
      const int vi = tid + P::NT * j, r = vi / P::A_VPR, c = (vi % P::A_VPR) * VE;
      int64_t m = m0 + r;
      m = m < a.M ? m : a.M - 1;
      const uint4 v = *reinterpret_cast<const uint4 *>(X + m * a.K + k0 + c);
      ra[j][0] = v.x; ra[j][1] = v.y; ra[j][2] = v.z; ra[j][3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < P::B_VEC; ++j) {
      const int vi = tid + P::NT * j, r = vi / P::B_VPR, c = (vi % P::B_VPR) * VE;
      int n = n0 + c;
      n = n < N ? n : N - VE;
      const uint4 v = *reinterpret_cast<const uint4 *>(W + (int64_t)(k0 + r) * N + n);
      rb[j][0] = v.x; rb[j][1] = v.y; rb[j][2] = v.z; rb[j][3] = v.w;
    }
  };
  auto store = [&](int st) {
    TIn *sA = lds + st * P::STAGE, *sB = sA + BM * LA;
#pragma unroll
    for (int j = 0; j < P::A_VEC; ++j) {
      const int vi = tid + P::NT * j, r = vi / P::A_VPR, c = (vi % P::A_VPR) * VE;
      *reinterpret_cast<uint4 *>(sA + r * LA + c) = make_uint4(ra[j][0], ra[j][1], ra[j][2], ra[j][3]);
    }
#pragma unroll
    for (int j = 0; j < P::B_VEC; ++j) {
      const int vi = tid + P::NT * j, r = vi / P::B_VPR, c = (vi % P::B_VPR) * VE;
      *reinterpret_cast<uint4 *>(sB + r * LB + c) = make_uint4(rb[j][0], rb[j][1], rb[j][2], rb[j][3]);
    }
  };

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4;

  const int nk = a.K / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK); // in flight while this step multiplies
    const TIn *sA = lds + st * P::STAGE, *sB = sA + BM * LA;
#pragma unroll
    for (int u = 0; u < P::NKU; ++u) {
      F af[MI], bf[4];
#pragma unroll
      for (int i = 0; i < MI; ++i) af[i] = ld_frag<TIn, true>(sA + (wm + 16 * i + li) * LA, u, g);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = ld_frag_t<TIn, true>(sB, LB, wn + 16 * j, u, g, li);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma(acc[i][j], bf[j], af[i]);
    }
    if (kt + 1 < nk) {
      store(st ^ 1);
      __syncthreads();
    }
  }

  // epilogue: acc[i][j] lane (g, li) holds Y[m = wm + 16 i + li][n = wn + 16 j + 4 g + r]
  TIn *Y = static_cast<TIn *>(a.y[p]);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t m = m0 + wm + 16 * i + li;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + 16 * j + 4 * g;
      if (n >= N) continue;
      f32x4 o = acc[i][j];
      if (elu) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = o[r] > 0.f ? o[r] + 1.f : __expf(o[r]);
      }
      st_out4<TIn>(Y + m * N + n, o);
    }
  }
}

} // namespace fla
