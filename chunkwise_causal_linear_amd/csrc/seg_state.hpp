// End state of every segment from a zero start, for the decays that are constant per head
// (none, or RetNet's gamma): the first pass of the segment schedule.
//
// Unrolling the recurrence h_t = g h_{t-1} + phi(k_t) v_t^T (textbook chapter 1.6, "linear
// attention"; the retention decay of the FLA posts) over a segment of L tokens from zero
// gives E = sum_j g^(L-1-j) phi(k_j) v_j^T (and z likewise with v = 1) and the segment's decay
// D = g^L: a reduction over the segment's tokens, memory-bound (it reads k and v once and
// needs no q, no outputs and no score tiles).  Per block of 64 tokens:
//     E <- g^Lb E + K'^T V,   K' = diag(g^(Lb-1-j)) phi(K)
// with bf16 (or fp32) MFMAs whose K^T and V operands come from row-major LDS tiles through
// the transposed LDS load.  One workgroup of 4 waves per (b, h, segment, value slice of
// 64 NV columns), each wave owning 16 NV value columns of the dk x 64 NV fp32 end state in
// MFMA accumulators; the next block's k and v are loaded into registers while the current
// one is multiplied, and the small footprint (26 KB of LDS at NV = 1, 36 KB at NV = 2)
// lets three or four workgroups share a CU to hide the memory latency.  NV = 2
// (bf16, dk <= 128, dv > 64) reads each k row once for 128 value columns: with 64-wide
// slices the sibling slice's copy of k came from HBM again whenever the two workgroups
// drifted apart by more than the XCD's L2 holds.
#pragma once

#include "chunk_fwd.hpp"

namespace fla {

template <typename TIn, int DK, int NV>
struct SegStateCfg {
  static constexpr int R = 64;                    // tokens per block
  static constexpr int NT = 256;
  static constexpr int SW = kSlice * NV;          // value columns per workgroup
  static constexpr int ES = sizeof(TIn);
  static constexpr int VE = 16 / ES;              // elements per 16-byte vector
  static constexpr int LK = DK + VE;              // k tile row stride (elements)
  static constexpr int LV = SW + (ES == 2 ? 16 : 4); // v tile row stride (conflict-free transposed reads)
  static constexpr int NVK = R * DK / VE / NT;    // 16-byte vectors per thread (k block)
  static constexpr int NVV = R * SW / VE / NT;    // (v block)
  static constexpr int VPRK = DK / VE;            // vectors per k row
  static constexpr int VPRV = SW / VE;            // vectors per v row
  static constexpr int NCB = DK / 16;             // 16-key blocks of the state
  static constexpr int KU = ES == 2 ? 32 : 16;    // tokens per MFMA K unit
  static constexpr int NU = R / KU;
  static constexpr int LDS_BYTES = (R * LK + R * LV) * ES;
  static_assert(NVK >= 1 && NVV >= 1, "block too small for the thread count");
};

// Z: the state carries the normaliser column (computed once per unit, by wave 0 of value
// slice 0).  Four workgroups per CU (at most 128 registers per lane) up to dk = 128 with
// 64-column slices, so the usual 1024 units of the segment schedule run in one round on
// 256 CUs; three with 128-column slices (their 512 units, likewise).  a.nvs counts value
// slices of SW columns.
template <typename TIn, int DK, bool Z, int NV>
__global__ __launch_bounds__(256, (DK > 128 ? 2 : NV == 2 ? 3 : 4)) void seg_state_kernel(ChunkArgs a) {
  using K = SegStateCfg<TIn, DK, NV>;
  using F = Frag<TIn>;
  constexpr int R = K::R, VE = K::VE, LK = K::LK, LV = K::LV, NCB = K::NCB;
  static_assert(NV == 1 || (NV == 2 && !Z), "the normaliser column is summed by 64-wide slices");
  __shared__ __attribute__((aligned(16))) TIn lds[K::LDS_BYTES / sizeof(TIn)];
  TIn *sK = lds;
  TIn *sV = lds + R * LK;

  // same unit numbering as the fused kernel: sibling value slices on one XCD
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vs = rest % a.nvs;
  const int unit = (rest / a.nvs) * 8 + xcd;
  if (unit >= a.nunits) return;
  const int seg = unit % a.nseg;
  const int bh = unit / a.nseg;
  const int h = bh % a.H;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;

  int64_t Tu = a.T, s0 = 0;
  if (a.bthd) s0 = (int64_t)(bh / a.H) * a.T;
  const int64_t rs_k = a.bthd ? (int64_t)a.H * DK : DK;
  const int64_t rs_v = a.bthd ? (int64_t)a.H * a.dv : a.dv;
  const int64_t base_k = a.bthd ? (s0 * a.H + h) * DK : (int64_t)bh * a.T * DK;
  const int64_t base_v = a.bthd ? (s0 * a.H + h) * a.dv : (int64_t)bh * a.T * a.dv;
  const int64_t t_begin = (int64_t)seg * a.seg_len;
  int64_t t_end = t_begin + a.seg_len;
  if (t_end > Tu) t_end = Tu;
  const int64_t len = t_end > t_begin ? t_end - t_begin : 0;
  const int nblk = (int)((len + R - 1) / R);
  const float l2g = a.decay ? log2f(a.decay[h]) : 0.f; // gamma (or none: g = 1)
  const int col0 = vs * K::SW;

  // register prefetch of one block (clamped rows, masked when staged)
  uint32_t rk[K::NVK][4], rv[K::NVV][4];
  auto load = [&](int blk) {
    const int64_t t0 = t_begin + (int64_t)blk * R;
    const int L = (int)((t_end - t0) < R ? (t_end - t0) : R);
    const TIn *gk = static_cast<const TIn *>(a.k) + base_k + t0 * rs_k;
    const TIn *gv = static_cast<const TIn *>(a.v) + base_v + t0 * rs_v + col0;
#pragma unroll
    for (int j = 0; j < K::NVK; ++j) {
      const int vi = tid + K::NT * j, r = vi / K::VPRK, c = (vi % K::VPRK) * VE;
      const uint4 x = *reinterpret_cast<const uint4 *>(gk + (int64_t)(r < L ? r : L - 1) * rs_k + c);
      rk[j][0] = x.x; rk[j][1] = x.y; rk[j][2] = x.z; rk[j][3] = x.w;
    }
#pragma unroll
    for (int j = 0; j < K::NVV; ++j) {
      const int vi = tid + K::NT * j, r = vi / K::VPRV, c = (vi % K::VPRV) * VE;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (col0 + c < a.dv) x = *reinterpret_cast<const uint4 *>(gv + (int64_t)(r < L ? r : L - 1) * rs_v + c);
      rv[j][0] = x.x; rv[j][1] = x.y; rv[j][2] = x.z; rv[j][3] = x.w;
    }
  };
  // phi, the in-block decay weight g^(L-1-j), rows past the end zeroed; into LDS
  auto stage = [&](int blk) {
    const int64_t t0 = t_begin + (int64_t)blk * R;
    const int L = (int)((t_end - t0) < R ? (t_end - t0) : R);
#pragma unroll
    for (int j = 0; j < K::NVK; ++j) {
      const int vi = tid + K::NT * j, r = vi / K::VPRK, c = (vi % K::VPRK) * VE;
      float f[VE];
      unpack<TIn, VE>(f, rk[j]);
      const float w = r < L ? (a.decay ? exp2f(l2g * (float)(L - 1 - r)) : 1.f) : 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float x = f[e];
        if (a.phi_elu1) x = x > 0.f ? x + 1.f : __expf(x);
        f[e] = x * w;
      }
      uint32_t wds[4];
      pack_words<TIn, VE>(wds, f);
      *reinterpret_cast<uint4 *>(sK + r * LK + c) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    }
#pragma unroll
    for (int j = 0; j < K::NVV; ++j) {
      const int vi = tid + K::NT * j, r = vi / K::VPRV, c = (vi % K::VPRV) * VE;
      const uint32_t m = r < L ? ~0u : 0u;
      *reinterpret_cast<uint4 *>(sV + r * LV + c) =
          make_uint4(rv[j][0] & m, rv[j][1] & m, rv[j][2] & m, rv[j][3] & m);
    }
    return L;
  };

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[NCB][NV];
  f32x4 zacc[Z ? NCB : 1];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[cb][j] = zero4;
#pragma unroll
  for (int cb = 0; cb < (Z ? NCB : 1); ++cb) zacc[cb] = zero4;
  const bool do_z = Z && vs == 0 && wave == 0; // normaliser column: once per unit
  F ones;
  {
    float o[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    ones = frag_from<TIn>(o);
  }

  if (nblk > 0) load(0);
  for (int blk = 0; blk < nblk; ++blk) {
    __syncthreads(); // the previous block's operands have been read
    const int L = stage(blk);
    __syncthreads();
    if (blk + 1 < nblk) load(blk + 1);
    const float gl = a.decay ? exp2f(l2g * (float)L) : 1.f;
    F vf[K::NU][NV];
#pragma unroll
    for (int u = 0; u < K::NU; ++u)
#pragma unroll
      for (int j = 0; j < NV; ++j) vf[u][j] = ld_frag_t<TIn, true>(sV, LV, 16 * (NV * wave + j), u, g, li);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      f32x4 x[NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) x[j] = acc[cb][j] * gl;
      f32x4 z = zacc[Z ? cb : 0] * gl;
#pragma unroll
      for (int u = 0; u < K::NU; ++u) {
        const F kf = ld_frag_t<TIn, true>(sK, LK, 16 * cb, u, g, li);
#pragma unroll
        for (int j = 0; j < NV; ++j) x[j] = mma(x[j], kf, vf[u][j]);
        if constexpr (Z) {
          if (do_z) z = mma(z, kf, ones);
        }
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) acc[cb][j] = x[j];
      if constexpr (Z) zacc[cb] = z;
    }
  }

  // end state (rows c = 16 cb + 4 g + r, column e) and the segment's decay product
  float *fo = a.fin + (int64_t)bh * a.fin_bh_stride + (int64_t)seg * a.fin_seg_stride;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 16 * cb + 4 * g + r;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int e = col0 + 16 * (NV * wave + j) + li;
        if (e < a.dv) fo[(int64_t)c * a.ncol + e] = acc[cb][j][r];
      }
      if constexpr (Z) {
        if (do_z && li == 0) fo[(int64_t)c * a.ncol + a.dv] = zacc[cb][r];
      }
    }
  if (a.seg_decay && vs == 0) {
    const float d = a.decay ? exp2f(l2g * (float)len) : 1.f;
    for (int c = tid; c < DK; c += K::NT) a.seg_decay[((int64_t)bh * a.nseg + seg) * DK + c] = d;
  }
}

} // namespace fla
