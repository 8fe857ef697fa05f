// Measurement probes: the HBM streaming rate and the bf16 MFMA rate this GPU reaches with
// plain hand-written kernels, reported beside the published peaks by the benchmark.
//
// Streams: every lane moves 16-byte vectors with non-temporal loads and stores, UNROLL
// vectors in flight per lane, over a grid of several workgroups per CU that strides
// through the buffers.  Three patterns:
//   read   reads `bytes` and writes one word per workgroup (the XOR of what it read, so
//          the loads cannot be dropped);
//   copy   reads and writes `bytes`;
//   mix5   reads 5 x and writes 1 x `bytes` / 6 of its own (the read:write ratio of the
//          gated forward pass: q, k, v and a four-byte gate in, one output out).
// MFMA: every wave runs four independent v_mfma_f32_32x32x16_bf16 chains on register
// operands (no memory traffic), 32 x 32 x 16 x 2 FLOPs per instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fla_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ u32x4 ld_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4 *p, u32x4 x) { __builtin_nontemporal_store(x, p); }

// n16: 16-byte vectors in the buffer (a multiple of kThreads * kUnroll per workgroup step is
// not required: the tail is handled element by element).
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *src, int64_t n16,
                                                        unsigned *sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n16; i += stride) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = ld_nt(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  for (; i < n16; i += kThreads) acc ^= ld_nt(src + i);
  const unsigned r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __shared__ unsigned red[kThreads];
  red[threadIdx.x] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned s = 0;
    for (int t = 0; t < kThreads; ++t) s ^= red[t];
    sink[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4 *src, u32x4 *dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n16; i += stride) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = ld_nt(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) st_nt(dst + i + u * kThreads, x[u]);
  }
  for (; i < n16; i += kThreads) st_nt(dst + i, ld_nt(src + i));
}

// Five reads per write: output vector j is the XOR of input vectors j, j + m, ..., j + 4m
// (m = n16out), so the input is read once and the output written once.
__global__ __launch_bounds__(kThreads) void mix5_kernel(const u32x4 *src, u32x4 *dst, int64_t m) {
  constexpr int U = kUnroll / 2;
  const int64_t stride = (int64_t)gridDim.x * kThreads * U;
  int64_t j = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
  for (; j + (U - 1) * kThreads < m; j += stride) {
    u32x4 x[U][5];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 5; ++r) x[u][r] = ld_nt(src + j + u * kThreads + r * m);
#pragma unroll
    for (int u = 0; u < U; ++u)
      st_nt(dst + j + u * kThreads, x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3] ^ x[u][4]);
  }
  for (; j < m; j += kThreads)
    st_nt(dst + j, ld_nt(src + j) ^ ld_nt(src + j + m) ^ ld_nt(src + j + 2 * m) ^
                       ld_nt(src + j + 3 * m) ^ ld_nt(src + j + 4 * m));
}

__global__ __launch_bounds__(kThreads) void mfma_kernel(float *out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(lane + i));
    b[i] = (__bf16)(seed * (float)(lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  // one word per wave, so the chains stay live
  if (lane == 0) out[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = s;
}

// The gated forward pass's access pattern with none of its arithmetic: one workgroup of
// four waves per (b, h, 64-wide value slice), the sibling slices of a head on one XCD (block
// id mod 8, as the chunk kernel maps them), walking the 64-token chunks of its head in
// order.  Per chunk it reads the chunk's q and k rows (bf16, dk = 128), its gate rows (fp32)
// and its value slice, and writes its output slice; the next chunk's loads are in flight
// while the current chunk's stores go out.  Lane t takes vectors t + 256 i of each chunk
// region (value and output slice: vector j is row j / 8, bytes 16 (j % 8) of the row's
// 128-byte slice).  Output vector i of lane t = value vector i XOR the XOR of the lane's q, k
// and gate vectors, so no load can be dropped.  Rows past T read zeros and are not
// written (buffer ranges), so any T works.
constexpr int kPatC = 64, kPatDK = 128, kPatSlice = 64;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t pat_rsrc(const void *base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void *b = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, __builtin_amdgcn_readfirstlane((int)bytes),
                                           0x00020000);
}

__global__ __launch_bounds__(kThreads) void chunk_pattern_kernel(const __bf16 *q, const __bf16 *k,
                                                                 const float *g, const __bf16 *v,
                                                                 __bf16 *out, int64_t T,
                                                                 int nunits, int nvs, int dv) {
  constexpr int NQ = kPatC * kPatDK * 2 / 16 / kThreads;    // q or k vectors per lane (4)
  constexpr int NG = kPatC * kPatDK * 4 / 16 / kThreads;    // gate vectors per lane (8)
  constexpr int NV = kPatC * kPatSlice * 2 / 16 / kThreads; // value / output vectors (2)
  struct Buf {
    u32x4 q[NQ], k[NQ], g[NG], v[NV];
  };
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vs = rest % nvs;
  const int unit = (rest / nvs) * 8 + xcd;
  if (unit >= nunits) return;
  const int t = threadIdx.x;
  const int64_t qk_base = (int64_t)unit * T * kPatDK;
  const int64_t v_base = (int64_t)unit * T * dv;
  const int nch = (int)((T + kPatC - 1) / kPatC);
  auto rows = [&](int n) {
    const int64_t l = T - (int64_t)n * kPatC;
    return l < 0 ? 0 : (l < kPatC ? l : kPatC);
  };
  auto voff = [&](int i) {
    const int j = t + kThreads * i;
    return ((j >> 3) * dv + vs * kPatSlice) * 2 + (j & 7) * 16;
  };
  auto load = [&](Buf &b, int n) {
    const int64_t t0 = (int64_t)n * kPatC, L = rows(n);
    const auto rv = pat_rsrc(v + v_base + t0 * dv, L * dv * 2);
    const auto rg = pat_rsrc(g + qk_base + t0 * kPatDK, L * kPatDK * 4);
    const auto rq = pat_rsrc(q + qk_base + t0 * kPatDK, L * kPatDK * 2);
    const auto rk = pat_rsrc(k + qk_base + t0 * kPatDK, L * kPatDK * 2);
#pragma unroll
    for (int i = 0; i < NV; ++i) b.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff(i), 0, 0);
#pragma unroll
    for (int i = 0; i < NG; ++i)
      b.g[i] = __builtin_amdgcn_raw_buffer_load_b128(rg, (t + kThreads * i) * 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      b.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, (t + kThreads * i) * 16, 0, 0);
      b.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (t + kThreads * i) * 16, 0, 0);
    }
  };
  auto store = [&](const Buf &b, int n) {
    const int64_t t0 = (int64_t)n * kPatC;
    const auto ro = pat_rsrc(out + v_base + t0 * dv, rows(n) * dv * 2);
    u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NQ; ++i) x ^= b.q[i] ^ b.k[i];
#pragma unroll
    for (int i = 0; i < NG; ++i) x ^= b.g[i];
#pragma unroll
    for (int i = 0; i < NV; ++i) __builtin_amdgcn_raw_buffer_store_b128(b.v[i] ^ x, ro, voff(i), 0, 0);
  };
  // two register sets: chunk n + 1 loads while chunk n's stores go out (past the last
  // chunk the ranges are empty: nothing is read or written)
  Buf a, b;
  load(a, 0);
  for (int n = 0; n < nch; n += 2) {
    load(b, n + 1);
    store(a, n);
    load(a, n + 2);
    store(b, n + 1);
  }
}

int grid_for(int64_t units_per_block, int64_t n) {
  // enough workgroups to cover the buffer once, capped at 16 per CU of a 256-CU part
  int64_t g = (n + units_per_block - 1) / units_per_block;
  if (g > 4096) g = 4096;
  return (int)(g < 1 ? 1 : g);
}

} // namespace

extern "C" {

int fla_probe_stream(const void *src, void *dst, int64_t bytes, int pattern, void *stream) {
  if (!src || bytes < 16 || (bytes & 15) != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n16 = bytes / 16;
  switch (pattern) {
  case FLA_PROBE_READ: {
    if (!dst) return -1; // receives one word per workgroup (up to 4096 words)
    const int grid = grid_for((int64_t)kThreads * kUnroll, n16);
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const u32x4 *>(src), n16, static_cast<unsigned *>(dst));
    break;
  }
  case FLA_PROBE_COPY: {
    if (!dst) return -1;
    const int grid = grid_for((int64_t)kThreads * kUnroll, n16);
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n16);
    break;
  }
  case FLA_PROBE_MIX5: {
    if (!dst || n16 % 6 != 0) return -1;
    const int64_t m = n16 / 6; // output vectors; the input holds 5 m of them
    const int grid = grid_for((int64_t)kThreads * (kUnroll / 2), m);
    hipLaunchKernelGGL(mix5_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), m);
    break;
  }
  default:
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int fla_probe_mfma(float *out, int64_t workgroups, int64_t iters, void *stream) {
  if (!out || workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 30)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out,
                     (int)iters, 1.0f / 1024.0f);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int fla_probe_chunk_pattern(const void *q, const void *k, const float *gate, const void *v,
                            void *out, int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                            void *stream) {
  if (!q || !k || !gate || !v || !out) return -1;
  for (const void *p : {q, k, static_cast<const void *>(gate), v, static_cast<const void *>(out)})
    if (reinterpret_cast<uintptr_t>(p) & 15) return -1;
  if (dk != kPatDK || dv < kPatSlice || dv > 256 || dv % kPatSlice != 0) return -1;
  // the kernel counts chunks in 32 bits: T below 2^36 keeps that count under 2^30
  if (B < 1 || H < 1 || T < 1 || T > ((int64_t)1 << 36) || B * H > (1 << 24) ||
      T > ((int64_t)1 << 40) / (B * H))
    return -1;
  const int64_t nunits = B * H, nvs = dv / kPatSlice;
  const int64_t grid = ((nunits + 7) / 8) * 8 * nvs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(chunk_pattern_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k), gate,
                     static_cast<const __bf16 *>(v), static_cast<__bf16 *>(out), T, (int)nunits,
                     (int)nvs, (int)dv);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

double fla_probe_mfma_flops(int64_t workgroups, int64_t iters) {
  // 4 waves per workgroup, 4 MFMAs per iteration, 32 x 32 x 16 multiply-adds each
  return (double)workgroups * 4.0 * (double)iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
}

} // extern "C"
