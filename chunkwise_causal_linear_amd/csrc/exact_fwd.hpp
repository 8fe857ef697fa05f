// Exact 16-token chunk path of the gated forward pass (per-key gate or per-token decay),
// for the (b, h) units where a chunk's decay product fell below kSafeDecay.
//
// The fused kernel factors the in-chunk decay as Qt = phi(q) b, Kt = phi(k) / b, which
// overflows once b (the product of the decays from the chunk start) becomes tiny; any
// decay in [0, 1] is valid input (textbook chapter 1.6, "gated delta rule": a decay near 0
// forgets the memory at once; "state-space models and Mamba": the decay mask of linear
// attention).  This kernel recomputes a flagged unit from its start state with products
// that only ever shrink, so they can underflow to zero only where the exact value is
// negligible, never overflow.  Per chunk of 16 tokens, with P_c(j+1..i) the product of
// the decays of key c over tokens j+1..i:
//   A_ij  = sum_c phi(q_ic) phi(k_jc) P_c(j+1..i)          (j <= i; running products)
//   o_i   = sum_j A_ij v_j + sum_c phi(q_ic) P_c(0..i) H_c   (/ the same with v = 1)
//   H_c  <- P_c(0..15) H_c + sum_j phi(k_jc) P_c(j+1..15) v_j
// in fp32 on the vector ALUs (no MFMA: this path only runs for inputs outside the fused
// kernel's range).  One workgroup of 256 threads per (b, h, 64-wide value slice); the
// state slice lives in LDS.  Units that were not flagged exit at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "chunk_fwd.hpp"

namespace fla {

struct ExactArgs {
  const void *q, *k, *v;
  const float *decay;         // gate (laid out like q) or per-token decay (one per token)
  const float *init;          // [B][H][dk][ncol] or null
  float *fin;                 // [B][H][dk][ncol] or null
  void *out;
  const int *unsafe;          // [B*H][nseg][4] flags from the fused kernel
  const int64_t *cu_seqlens;  // packed sequences (bthd), or null
  int64_t T;
  int H, dv, ncol, nseg, nvs;
  int per_key;                // 1: gate [.., dk]; 0: per-token decay
  int phi_elu1, norm, bthd;
};

template <typename TIn, int DK>
struct ExactCfg {
  static constexpr int R = 16;          // tokens per chunk
  static constexpr int NT = 256;
  static constexpr int XW = 64;         // value columns per workgroup
  static constexpr int KPT = DK / 16;   // keys per thread in the score step
  // LDS (floats): phi(q) / Qt, phi(k) / Khat, decays [R][DK]; V [R][XW]; H [DK][XW]; z [DK];
  // chunk products [DK]; scores [R][R]
  static constexpr int O_Q = 0, O_K = O_Q + R * DK, O_A = O_K + R * DK, O_V = O_A + R * DK;
  static constexpr int O_H = O_V + R * XW, O_Z = O_H + DK * XW, O_D = O_Z + DK;
  static constexpr int O_S = O_D + DK, FLOATS = O_S + R * R;
};

template <typename TIn>
__device__ __forceinline__ float ld_elem(const TIn *p, int64_t i) {
  if constexpr (sizeof(TIn) == 2) return (float)p[i];
  else return p[i];
}

template <typename TIn, int DK>
__global__ __launch_bounds__(256) void exact_fwd_kernel(ExactArgs a) {
  using K = ExactCfg<TIn, DK>;
  constexpr int R = K::R, XW = K::XW;
  __shared__ float lds[K::FLOATS];
  float *sQ = lds + K::O_Q, *sK = lds + K::O_K, *sA = lds + K::O_A, *sV = lds + K::O_V;
  float *sH = lds + K::O_H, *sZ = lds + K::O_Z, *sD = lds + K::O_D, *sS = lds + K::O_S;

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / a.nvs;
  const int vs = blockIdx.x % a.nvs;
  // only units the fused kernel flagged
  int flagged = 0;
  for (int i = tid; i < a.nseg * 4; i += K::NT) flagged |= a.unsafe[bh * a.nseg * 4 + i];
  if (!__syncthreads_or(flagged)) return;

  const int h = (int)(bh % a.H);
  int64_t Tu = a.T, s0 = 0;
  if (a.bthd) {
    const int64_t b = bh / a.H;
    if (a.cu_seqlens) {
      s0 = a.cu_seqlens[b];
      int64_t e = a.cu_seqlens[b + 1];
      s0 = s0 < 0 ? 0 : (s0 > a.T ? a.T : s0);
      e = e < s0 ? s0 : (e > a.T ? a.T : e);
      Tu = e - s0;
    } else {
      s0 = b * a.T;
    }
  }
  const int64_t rs_qk = a.bthd ? (int64_t)a.H * DK : DK;
  const int64_t rs_v = a.bthd ? (int64_t)a.H * a.dv : a.dv;
  const int64_t rs_t = a.bthd ? a.H : 1;
  const int64_t base_qk = a.bthd ? (s0 * a.H + h) * DK : bh * a.T * DK;
  const int64_t base_v = a.bthd ? (s0 * a.H + h) * a.dv : bh * a.T * a.dv;
  const int64_t base_t = a.bthd ? s0 * a.H + h : bh * a.T;
  const TIn *gq = static_cast<const TIn *>(a.q) + base_qk;
  const TIn *gk = static_cast<const TIn *>(a.k) + base_qk;
  const TIn *gv = static_cast<const TIn *>(a.v) + base_v;
  TIn *go = static_cast<TIn *>(a.out) + base_v;
  const int col0 = vs * XW;
  auto phi = [&](float x) { return a.phi_elu1 ? (x > 0.f ? x + 1.f : __expf(x)) : x; };

  // start state
  const float *ini = a.init ? a.init + bh * DK * a.ncol : nullptr;
  for (int i = tid; i < DK * XW; i += K::NT) {
    const int c = i / XW, e = i % XW;
    sH[i] = (ini && col0 + e < a.dv) ? ini[(int64_t)c * a.ncol + col0 + e] : 0.f;
  }
  for (int c = tid; c < DK; c += K::NT) sZ[c] = (ini && a.norm) ? ini[(int64_t)c * a.ncol + a.dv] : 0.f;

  const int64_t nch = (Tu + R - 1) / R;
  for (int64_t n = 0; n < nch; ++n) {
    const int64_t t0 = n * R;
    const int L = (int)((Tu - t0) < R ? (Tu - t0) : R);
    __syncthreads(); // the previous chunk's state update has read the tiles
    // ---- raw tiles: phi(q), phi(k), decays (rows past the end: 0, 0, 1); value slice
    for (int i = tid; i < R * DK; i += K::NT) {
      const int r = i / DK, c = i % DK;
      float qv = 0.f, kv = 0.f, av = 1.f;
      if (r < L) {
        const int64_t t = t0 + r;
        qv = phi(ld_elem(gq, t * rs_qk + c));
        kv = phi(ld_elem(gk, t * rs_qk + c));
        av = a.per_key ? a.decay[base_qk + t * rs_qk + c] : a.decay[base_t + t * rs_t];
      }
      sQ[i] = qv;
      sK[i] = kv;
      sA[i] = av;
    }
    for (int i = tid; i < R * XW; i += K::NT) {
      const int r = i / XW, e = i % XW;
      sV[i] = (r < L && col0 + e < a.dv) ? ld_elem(gv, (t0 + r) * rs_v + col0 + e) : 0.f;
    }
    __syncthreads();
    // ---- A_ij: thread (i, key group kg) walks j = i, i-1, .., 0 with one running product
    // per key (P(j+1..i), times the decay of row j after row j is used)
    {
      const int i = tid / 16, kg = tid % 16;
      float run[K::KPT];
#pragma unroll
      for (int u = 0; u < K::KPT; ++u) run[u] = 1.f;
      float acc[R];
#pragma unroll
      for (int j = R - 1; j >= 0; --j) {
        float s = 0.f;
        if (j <= i) {
#pragma unroll
          for (int u = 0; u < K::KPT; ++u) {
            const int c = kg + 16 * u;
            s += sQ[i * DK + c] * sK[j * DK + c] * run[u];
            run[u] *= sA[j * DK + c];
          }
        }
        acc[j] = s;
      }
#pragma unroll
      for (int j = 0; j < R; ++j) {
        float s = acc[j];
        s += __shfl_xor(s, 8, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 1, 16);
        acc[j] = s;
      }
      if (kg == 0) {
#pragma unroll
        for (int j = 0; j < R; ++j) sS[i * R + j] = j <= i ? acc[j] : 0.f;
      }
    }
    __syncthreads();
    // ---- per key: Qt = phi(q) P(0..i), Khat = phi(k) P(j+1..15), chunk product D
    for (int c = tid; c < DK; c += K::NT) {
      float run = 1.f;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        run *= sA[i * DK + c];
        sQ[i * DK + c] *= run;
      }
      sD[c] = run;
      float suf = 1.f;
#pragma unroll
      for (int j = R - 1; j >= 0; --j) {
        sK[j * DK + c] *= suf;
        suf *= sA[j * DK + c];
      }
    }
    __syncthreads();
    // ---- outputs: thread (row i, 4 adjacent value columns)
    {
      const int i = tid / 16, e4 = 4 * (tid % 16);
      float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float p = sS[i * R + j];
        const float4 vv = *reinterpret_cast<const float4 *>(sV + j * XW + e4);
        num[0] += p * vv.x; num[1] += p * vv.y; num[2] += p * vv.z; num[3] += p * vv.w;
        den += p;
      }
      for (int c = 0; c < DK; ++c) {
        const float qv = sQ[i * DK + c];
        const float4 hv = *reinterpret_cast<const float4 *>(sH + c * XW + e4);
        num[0] += qv * hv.x; num[1] += qv * hv.y; num[2] += qv * hv.z; num[3] += qv * hv.w;
        den += qv * sZ[c];
      }
      if (i < L) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int e = col0 + e4 + x;
          if (e < a.dv) {
            const float o = a.norm ? num[x] / den : num[x];
            go[(t0 + i) * rs_v + e] = (TIn)o;
          }
        }
      }
    }
    __syncthreads(); // every output read the state before it changes
    // ---- state: H_c <- D_c H_c + sum_j Khat_jc v_j; z likewise with v = 1
    {
      const int e = tid % XW;
      for (int c = tid / XW; c < DK; c += K::NT / XW) {
        float hv = sD[c] * sH[c * XW + e];
#pragma unroll
        for (int j = 0; j < R; ++j) hv += sK[j * DK + c] * sV[j * XW + e];
        sH[c * XW + e] = hv;
      }
      if (a.norm) {
        for (int c = tid; c < DK; c += K::NT) {
          float zv = sD[c] * sZ[c];
#pragma unroll
          for (int j = 0; j < R; ++j) zv += sK[j * DK + c];
          sZ[c] = zv;
        }
      }
    }
  }
  __syncthreads();
  if (a.fin) {
    float *fo = a.fin + bh * DK * a.ncol;
    for (int i = tid; i < DK * XW; i += K::NT) {
      const int c = i / XW, e = i % XW;
      if (col0 + e < a.dv) fo[(int64_t)c * a.ncol + col0 + e] = sH[i];
    }
    if (a.norm && vs == 0)
      for (int c = tid; c < DK; c += K::NT) fo[(int64_t)c * a.ncol + a.dv] = sZ[c];
  }
}

} // namespace fla
