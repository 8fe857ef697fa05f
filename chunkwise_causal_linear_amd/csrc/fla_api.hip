// C ABI of the chunkwise causal linear attention library: validation, schedule choice,
// launches, plus the small kernels around the fused chunk kernel (segment scan, state
// fill/copy, one-token decode step).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fla_linattn.h"
#include "bwd_dispatch.hpp"
#include "dispatch.hpp"
#include "exact_fwd.hpp"
#include "gdn_fwd.hpp"
#include "proj.hpp"
#include "seg_state.hpp"

namespace fla {

using GdnLauncher = hipError_t (*)(const GdnArgs &, unsigned grid, hipStream_t);
struct GdnLaunchers {
  GdnLauncher prep, state;
};
GdnLaunchers gdn_launchers(bool bf16, int dk); // gdn_inst.hip

// Scratch memory of the no-allocation entry point: the segment schedule's workspace (and
// the private start-state copy of an in-place resume) are carved out of this array instead
// of stream-ordered allocations.  Every GPU the library runs on holds its own copy until
// the process ends.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kStepThreads = 256;
constexpr int kScanThreads = 256;
constexpr int kOrderThreads = 256;
constexpr int64_t kOrderMax = 8192; // packed sequences ranked longest-first up to this many
constexpr int64_t kMaxGrid = (int64_t)1 << 31;

bool is_pow2_dim(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }
bool is_chunk(int64_t c) { return c == 16 || c == 32 || c == 64 || c == 128; }
// Chunk sizes a call accepts: the tile sizes above, and larger powers of two up to 1024
// (the FLA posts advise chunk_size = 512 for long-sequence training), which are evaluated
// as consecutive 64-token sub-chunks (see tile_for).  Splitting a chunk into sub-chunks is
// exact in real arithmetic (the state after a sub-chunk is the state before the next), so
// only the rounding differs.
bool is_chunk_arg(int64_t c) { return is_chunk(c) || c == 256 || c == 512 || c == 1024; }
// The tile a requested chunk size runs with.  128-token tiles of the per-key gate and of
// dk = 256 fall to the split schedule with its registers spilling inside the chunk loop
// (measured 4.1 ms against 0.79 ms for the GLA workload, 1.65 against 0.22 ms for the
// d256 retention workload), and fp32 128-token tiles at dk >= 128 do not fit the LDS:
// those run as two 64-token sub-chunks, like any larger chunk.  So does the constant decay
// at dk = 128 in bf16: its 128-token tile takes the split schedule with the narrow row
// padding, its 64-token tile the shared-score one with the wide padding (2.85 against
// 2.95 ms for the T = 2^20 retention workload; 1.7% slower than the 128-token tile where
// all units run in one round, T = 8192).
int64_t tile_for(int64_t chunk, int64_t dk, int kind, bool bf16) {
  if (chunk > 128) return 64;
  if (chunk == 128 && (kind == DECAY_GATE || dk > 128 || (!bf16 && dk >= 128) ||
                       (bf16 && dk == 128 && kind == DECAY_GAMMA)))
    return 64;
  return chunk;
}
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

ChunkLauncher find_launcher(bool bf16, int64_t dk, int64_t chunk, int decay, bool norm) {
  const int c = (int)chunk;
  if (bf16) {
    switch (dk) {
    case 16: return chunk_launcher_bf16_16(c, decay, norm);
    case 32: return chunk_launcher_bf16_32(c, decay, norm);
    case 64: return chunk_launcher_bf16_64(c, decay, norm);
    case 128: return chunk_launcher_bf16_128(c, decay, norm);
    case 256: return chunk_launcher_bf16_256(c, decay, norm);
    }
  } else {
    switch (dk) {
    case 16: return chunk_launcher_f32_16(c, decay, norm);
    case 32: return chunk_launcher_f32_32(c, decay, norm);
    case 64: return chunk_launcher_f32_64(c, decay, norm);
    case 128: return chunk_launcher_f32_128(c, decay, norm);
    case 256: return chunk_launcher_f32_256(c, decay, norm);
    }
  }
  return nullptr;
}

using ExactKernel = void (*)(ExactArgs);
ExactKernel find_exact(bool bf16, int64_t dk) {
  switch (dk) {
  case 16: return bf16 ? &exact_fwd_kernel<__bf16, 16> : &exact_fwd_kernel<float, 16>;
  case 32: return bf16 ? &exact_fwd_kernel<__bf16, 32> : &exact_fwd_kernel<float, 32>;
  case 64: return bf16 ? &exact_fwd_kernel<__bf16, 64> : &exact_fwd_kernel<float, 64>;
  case 128: return bf16 ? &exact_fwd_kernel<__bf16, 128> : &exact_fwd_kernel<float, 128>;
  case 256: return bf16 ? &exact_fwd_kernel<__bf16, 256> : &exact_fwd_kernel<float, 256>;
  }
  return nullptr;
}

using SegStateKernel = void (*)(ChunkArgs);
template <bool Z>
SegStateKernel find_seg_state_z(bool bf16, int64_t dk) {
  switch (dk) {
  case 16: return bf16 ? nullptr : &seg_state_kernel<float, 16, Z, 1>; // (bf16: fused kernel's pass)
  case 32: return bf16 ? &seg_state_kernel<__bf16, 32, Z, 1> : &seg_state_kernel<float, 32, Z, 1>;
  case 64: return bf16 ? &seg_state_kernel<__bf16, 64, Z, 1> : &seg_state_kernel<float, 64, Z, 1>;
  case 128: return bf16 ? &seg_state_kernel<__bf16, 128, Z, 1> : &seg_state_kernel<float, 128, Z, 1>;
  case 256: return bf16 ? &seg_state_kernel<__bf16, 256, Z, 1> : &seg_state_kernel<float, 256, Z, 1>;
  }
  return nullptr;
}
// 128-column slices (one read of k for both halves of a 128-wide state): bf16, no
// normaliser, 32 <= dk <= 128, dv > 64
SegStateKernel find_seg_state_wide(int64_t dk) {
  switch (dk) {
  case 32: return &seg_state_kernel<__bf16, 32, false, 2>;
  case 64: return &seg_state_kernel<__bf16, 64, false, 2>;
  case 128: return &seg_state_kernel<__bf16, 128, false, 2>;
  }
  return nullptr;
}
SegStateKernel find_seg_state(bool bf16, int64_t dk, bool norm) {
  return norm ? find_seg_state_z<true>(bf16, dk) : find_seg_state_z<false>(bf16, dk);
}

int decay_kind(uint32_t flags) {
  if (flags & FLA_DECAY_GAMMA) return DECAY_GAMMA;
  if (flags & FLA_DECAY_GATE) return DECAY_GATE;
  if (flags & FLA_DECAY_TOKEN) return DECAY_TOKEN;
  return DECAY_NONE;
}

constexpr uint32_t kDecayBits = FLA_DECAY_GAMMA | FLA_DECAY_GATE | FLA_DECAY_TOKEN;

// Shape and flag checks shared by the forward and step calls.
int check_common(int64_t B, int64_t H, int64_t dk, int64_t dv, uint32_t flags,
                 const float *gate_or_gamma) {
  if (flags & ~FLA_ALL_FLAGS) return FLA_ERR_INVALID_ARG;
  const uint32_t dbits = flags & kDecayBits;
  if (dbits & (dbits - 1)) return FLA_ERR_INVALID_ARG; // at most one decay kind
  const bool has_decay = dbits != 0;
  if (has_decay != (gate_or_gamma != nullptr)) return FLA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || B > (1 << 24) || H > (1 << 24)) return FLA_ERR_INVALID_ARG;
  if (dk < 1 || dv < 1) return FLA_ERR_INVALID_ARG;
  if (!aligned(gate_or_gamma, (flags & FLA_DECAY_GATE) ? 16 : 4)) return FLA_ERR_INVALID_ARG;
  if (!is_pow2_dim(dk) || !is_pow2_dim(dv)) return FLA_ERR_UNSUPPORTED;
  return FLA_OK;
}

// Segment count: one streaming workgroup per (b, h, value slice) when that already gives
// at least one workgroup per CU; otherwise cut the sequence so ~1024 workgroups exist,
// keeping at least 8 chunks per segment.
int64_t auto_segments(int64_t B, int64_t H, int64_t T, int64_t dv, int64_t chunk) {
  const int64_t nvs = (dv + kSlice - 1) / kSlice;
  const int64_t units = B * H * nvs;
  if (units >= 256) return 1;
  const int64_t nch = (T + chunk - 1) / chunk;
  int64_t p = 1024 / units;
  if (p > nch / 8) p = nch / 8;
  return p < 1 ? 1 : p;
}

BwdLauncher find_bwd(bool bf16, int64_t dy, int role, int decay) {
  if (bf16) {
    switch (dy) {
    case 64: return bwd_launcher_bf16_64(role, decay);
    case 128: return bwd_launcher_bf16_128(role, decay);
    case 256: return bwd_launcher_bf16_256(role, decay);
    }
  } else {
    switch (dy) {
    case 64: return bwd_launcher_f32_64(role, decay);
    case 128: return bwd_launcher_f32_128(role, decay);
    case 256: return bwd_launcher_f32_256(role, decay);
    }
  }
  return nullptr;
}

// ---------------------------------------------------------------------------------
// small kernels

// Per-token decay gradient: d alpha = (sum of the nparts partial sums of d log a) / alpha,
// per (head h, token tok of all sequences); partials tpart[h][p][tok].  The decay and its
// gradient are [B][H][T] (tok = b T + t) or token-major [tokens][H] (bthd).
__global__ void token_dgate_kernel(const float *tpart, const float *decay, float *dgate,
                                   int64_t H, int64_t ntok, int64_t T, int nparts, int bthd) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H * ntok) return;
  const int64_t h = i / ntok, tok = i % ntok;
  float s = 0.f;
  for (int p = 0; p < nparts; ++p) s += tpart[(h * nparts + p) * ntok + tok];
  const int64_t at = bthd ? tok * H + h : ((tok / T) * H + h) * T + tok % T;
  dgate[at] = s / decay[at];
}

// Longest-first order of packed sequences: order[r] is the sequence with the r-th most
// chunks (ties by index), so a grid dispatched in unit order starts the longest sequences
// first and the short ones fill in behind them.  One thread per sequence counts the
// sequences ranked before it; lengths are clamped as the chunk kernel clamps them.
__global__ void seq_order_kernel(const int64_t *cu, int n, int64_t T, int64_t chunk, int *order) {
  __shared__ int64_t tile[kOrderThreads];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  auto nch = [&](int b) -> int64_t {
    int64_t s = cu[b], e = cu[b + 1];
    s = s < 0 ? 0 : (s > T ? T : s);
    e = e < s ? s : (e > T ? T : e);
    return (e - s + chunk - 1) / chunk;
  };
  const int64_t mine = i < n ? nch(i) : 0;
  int r = 0;
  for (int j0 = 0; j0 < n; j0 += kOrderThreads) {
    __syncthreads();
    if (j0 + (int)threadIdx.x < n) tile[threadIdx.x] = nch(j0 + (int)threadIdx.x);
    __syncthreads();
    const int m = n - j0 < kOrderThreads ? n - j0 : kOrderThreads;
    for (int j = 0; j < m; ++j) {
      const int64_t l = tile[j];
      r += (l > mine || (l == mine && j0 + j < i)) ? 1 : 0;
    }
  }
  if (i < n) order[r] = i;
}

// dst[i] = src ? src[i] : 0 (state copy / zero fill).
__global__ void state_fill_kernel(float *dst, const float *src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

// Scan over segments (elementwise per state entry): on entry ws[bh][s] holds segment s's
// end state from a zero start and dec[bh][s][c] the product of its decays; on exit ws[bh][s]
// holds segment s's true start state, and fin (if any) the state after the last segment.
// unsafe: the fused kernel's flags [nbh][nseg][4] (gated kinds) or null; a flagged unit's
// end state is left to the exact kernel (its start state may be the same memory).
__global__ void segment_scan_kernel(float *ws, const float *dec, const float *init, float *fin,
                                    int64_t nbh, int nseg, int dk, int ncol, const int *unsafe) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)dk * ncol;
  if (i >= nbh * per) return;
  const int64_t bh = i / per, ce = i % per;
  if (unsafe) {
    for (int s = 0; s < 4 * nseg; ++s)
      if (unsafe[bh * 4 * nseg + s]) fin = nullptr;
  }
  const int c = (int)(ce / ncol);
  float run = init ? init[i] : 0.f;
  float *w = ws + bh * nseg * per + ce;
  const float *d = dec + bh * nseg * dk + c;
  for (int s = 0; s < nseg; ++s) {
    const float e = w[(int64_t)s * per];
    w[(int64_t)s * per] = run;
    run = d[(int64_t)s * dk] * run + e;
  }
  if (fin) fin[i] = run;
}

template <typename TIn> __device__ __forceinline__ float ld_in(const TIn *p, int64_t i);
template <> __device__ __forceinline__ float ld_in<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_in<__bf16>(const __bf16 *p, int64_t i) {
  return (float)p[i];
}

// One decoding token per (b, h): h <- diag(g) h + phi(k) v^T, z <- g z + phi(k),
// o = h^T phi(q) (/ z^T phi(q)).  Threads own value columns, so state rows are read
// and written coalesced.
template <typename TIn>
__global__ __launch_bounds__(kStepThreads) void step_kernel(const TIn *q, const TIn *k,
                                                            const TIn *v, const float *decay,
                                                            int kind, float *state, TIn *out,
                                                            int H, int dk, int dv, int phi_elu1,
                                                            int norm) {
  __shared__ float sq[256], sk[256], sg[256], sz[256];
  __shared__ float sden;
  const int bh = blockIdx.x, h = bh % H, tid = threadIdx.x;
  const int ncol = dv + (norm ? 1 : 0);
  float *st = state + (int64_t)bh * dk * ncol;
  for (int c = tid; c < dk; c += blockDim.x) {
    float qv = ld_in(q, (int64_t)bh * dk + c), kv = ld_in(k, (int64_t)bh * dk + c);
    if (phi_elu1) {
      qv = qv > 0.f ? qv + 1.f : __expf(qv);
      kv = kv > 0.f ? kv + 1.f : __expf(kv);
    }
    sq[c] = qv;
    sk[c] = kv;
    sg[c] = kind == DECAY_GAMMA   ? decay[h]
            : kind == DECAY_GATE  ? decay[(int64_t)bh * dk + c]
            : kind == DECAY_TOKEN ? decay[bh]
                                  : 1.f;
  }
  __syncthreads();
  if (norm) {
    for (int c = tid; c < dk; c += blockDim.x) {
      const float z = sg[c] * st[(int64_t)c * ncol + dv] + sk[c];
      sz[c] = z;
      st[(int64_t)c * ncol + dv] = z;
    }
    __syncthreads();
    if (tid == 0) {
      float d = 0.f;
      for (int c = 0; c < dk; ++c) d += sz[c] * sq[c];
      sden = d;
    }
    __syncthreads();
  }
  for (int e = tid; e < dv; e += blockDim.x) {
    const float ve = ld_in(v, (int64_t)bh * dv + e);
    float acc = 0.f;
    for (int c = 0; c < dk; ++c) {
      float *p = st + (int64_t)c * ncol + e;
      const float hn = sg[c] * *p + sk[c] * ve;
      *p = hn;
      acc += hn * sq[c];
    }
    if (norm) acc = acc / sden;
    out[(int64_t)bh * dv + e] = (TIn)acc;
  }
}

unsigned blocks_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

int launch_fill(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return FLA_OK;
  void *args[] = {&dst, &src, &n};
  if (hipLaunchKernel(reinterpret_cast<const void *>(&state_fill_kernel), dim3(blocks_for(n, 256)),
                      dim3(256), args, 0, s) != hipSuccess)
    return FLA_ERR_DEVICE;
  return FLA_OK;
}

// An empty sequence has an empty per-token decay, which callers may pass as NULL.
const float *nonnull_decay_if_empty(const float *decay, int64_t T, uint32_t flags) {
  static const float kUnused[4] = {1.f, 1.f, 1.f, 1.f}; // never read: nothing is launched on it
  if (T == 0 && !decay && (flags & (FLA_DECAY_GATE | FLA_DECAY_TOKEN))) return kUnused;
  return decay;
}

// Device memory the forward pass needs beyond its inputs and outputs.  Either
// stream-ordered allocations (hipMallocAsync / hipFreeAsync on the call's stream), or
// carved out of a caller-provided region (the no-allocation entry point's scratch array),
// in which case a request that does not fit fails with FLA_ERR_SCRATCH and nothing is
// allocated.
struct Workspace {
  char *base = nullptr; // scratch region, or null for stream-ordered allocations
  int64_t cap = 0, used = 0;
  hipStream_t s = nullptr;
  void *owned[8] = {};
  int nowned = 0;

  bool from_scratch() const { return base != nullptr; }
  int64_t left() const { return cap - ((used + 255) & ~(int64_t)255); }
  int get(int64_t bytes, void **p) {
    if (base) {
      const int64_t off = (used + 255) & ~(int64_t)255;
      if (bytes > cap - off) return FLA_ERR_SCRATCH;
      *p = base + off;
      used = off + bytes;
      return FLA_OK;
    }
    if (nowned == 8 || hipMallocAsync(p, (size_t)bytes, s) != hipSuccess) return FLA_ERR_DEVICE;
    owned[nowned++] = *p;
    return FLA_OK;
  }
  // frees the stream-ordered allocations (after the launches that use them are enqueued)
  int release() {
    int rc = FLA_OK;
    for (int i = 0; i < nowned; ++i)
      if (hipFreeAsync(owned[i], s) != hipSuccess) rc = FLA_ERR_DEVICE;
    nowned = 0;
    return rc;
  }
};

// cu_seqlens: packed sequences (token-major layout, B = number of sequences, T = total
// tokens); null for B sequences of T tokens each.  ws: where workspaces come from.
int fwd_impl(const void *q, const void *k, const void *v, const float *gate_or_gamma,
             const float *init_state, void *out, float *final_state, int64_t B, int64_t H,
             int64_t T, int64_t dk, int64_t dv, int64_t chunk, uint32_t flags,
             int64_t n_segments, const int64_t *cu_seqlens, Workspace &ws) {
  gate_or_gamma = nonnull_decay_if_empty(gate_or_gamma, T, flags);
  int rc = check_common(B, H, dk, dv, flags, gate_or_gamma);
  if (rc != FLA_OK) return rc;
  const bool bthd = cu_seqlens != nullptr || (flags & FLA_LAYOUT_BTHD) != 0;
  if (bthd && H * (dk > dv ? dk : dv) > ((int64_t)1 << 20)) return FLA_ERR_UNSUPPORTED;
  if (T < 0 || n_segments < 0) return FLA_ERR_INVALID_ARG;
  if (T > 0 && (!q || !k || !v || !out)) return FLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(init_state, 16) || !aligned(final_state, 16))
    return FLA_ERR_INVALID_ARG;
  if (!is_chunk_arg(chunk)) return FLA_ERR_UNSUPPORTED;
  if (B * H > ((int64_t)1 << 26) || T > ((int64_t)1 << 40) / (B * H)) return FLA_ERR_INVALID_ARG;
  const bool bf16 = (flags & FLA_BF16) != 0;
  const bool norm = (flags & FLA_NORMALIZE) != 0;
  const int kind = decay_kind(flags);
  chunk = tile_for(chunk, dk, kind, bf16); // sub-chunks of a faster tile (see is_chunk_arg)
  ChunkLauncher launch = find_launcher(bf16, dk, chunk, kind, norm);
  if (!launch) return FLA_ERR_UNSUPPORTED;
  hipStream_t s = ws.s;
  const int64_t ncol = dv + (norm ? 1 : 0);
  const int64_t nbh = B * H;
  const int64_t state_elems = nbh * dk * ncol;

  if (T == 0) {
    if (final_state && final_state != init_state) return launch_fill(final_state, init_state, state_elems, s);
    return FLA_OK;
  }

  const int64_t nch = (T + chunk - 1) / chunk;
  int64_t nseg = n_segments == 0 ? auto_segments(B, H, T, dv, chunk) : n_segments;
  if (cu_seqlens) nseg = 1; // packed sequences: one streaming workgroup per (sequence, head, slice)
  if (nseg > nch) nseg = nch;
  // Gated kinds: the fused kernel flags the units whose decay products leave its range
  // (one word per producer wave), and the exact kernel recomputes those after it.
  const bool gated = kind == DECAY_GATE || kind == DECAY_TOKEN;
  auto flag_bytes = [&](int64_t p) { return gated ? nbh * p * 4 * (int64_t)sizeof(int) : 0; };
  // segment workspace: every segment's end state and decay product
  auto seg_ws_bytes = [&](int64_t p) { return nbh * p * dk * (ncol + 1) * (int64_t)sizeof(float); };
  if (ws.from_scratch() && n_segments == 0) {
    // the automatic count is cut down until its workspace fits the scratch region
    while (nseg > 1 && flag_bytes(nseg) + 256 + seg_ws_bytes(nseg) > ws.left()) nseg = nseg / 2;
  }
  const int64_t seg_chunks = (nch + nseg - 1) / nseg;
  const int64_t seg_len = seg_chunks * chunk;
  nseg = (T + seg_len - 1) / seg_len;
  const int64_t nvs = (dv + kSlice - 1) / kSlice;
  const int64_t nunits = nbh * nseg;
  const int64_t grid = ((nunits + 7) / 8) * 8 * nvs;
  if (grid >= kMaxGrid) return FLA_ERR_UNSUPPORTED;

  const ExactKernel exact = gated ? find_exact(bf16, dk) : nullptr;
  if (gated && !exact) return FLA_ERR_UNSUPPORTED;
  int *unsafe = nullptr;
  if (gated) {
    void *f = nullptr;
    if ((rc = ws.get(flag_bytes(nseg), &f)) != FLA_OK) return rc;
    unsafe = static_cast<int *>(f);
  }
  // The exact kernel's start states: with an in-place resume, the normaliser and several
  // value slices, a private copy (value slice 0 writes the z column of the final state,
  // which the other slices read as their start).
  const float *exact_init = init_state;
  auto private_start = [&](const float **dst) -> int {
    void *tmp = nullptr;
    int r = ws.get(state_elems * (int64_t)sizeof(float), &tmp);
    if (r == FLA_OK) r = launch_fill(static_cast<float *>(tmp), init_state, state_elems, s);
    if (r != FLA_OK) {
      ws.release();
      return r;
    }
    *dst = static_cast<const float *>(tmp);
    return FLA_OK;
  };
  const bool shared_z = init_state && init_state == final_state && norm && nvs > 1;
  auto run_exact = [&]() -> int {
    if (!gated) return FLA_OK;
    ExactArgs e{};
    e.q = q; e.k = k; e.v = v;
    e.decay = gate_or_gamma;
    e.init = exact_init;
    e.fin = final_state;
    e.out = out;
    e.unsafe = unsafe;
    e.cu_seqlens = cu_seqlens;
    e.T = T;
    e.H = (int)H; e.dv = (int)dv; e.ncol = (int)ncol; e.nseg = (int)nseg; e.nvs = (int)nvs;
    e.per_key = kind == DECAY_GATE ? 1 : 0;
    e.phi_elu1 = (flags & FLA_PHI_ELU1) ? 1 : 0;
    e.norm = norm ? 1 : 0;
    e.bthd = bthd ? 1 : 0;
    void *args[] = {&e};
    return hipLaunchKernel(reinterpret_cast<const void *>(exact), dim3((unsigned)(nbh * nvs)),
                           dim3(256), args, 0, s) == hipSuccess ? FLA_OK : FLA_ERR_DEVICE;
  };

  ChunkArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.decay = gate_or_gamma;
  a.out = out;
  a.unsafe = unsafe;
  a.T = T;
  a.seg_len = seg_len;
  a.H = (int)H; a.dv = (int)dv; a.ncol = (int)ncol;
  a.nseg = (int)nseg; a.nvs = (int)nvs; a.nunits = (int)nunits;
  a.phi_elu1 = (flags & FLA_PHI_ELU1) ? 1 : 0;
  a.bthd = bthd ? 1 : 0;
  a.cu_seqlens = cu_seqlens;

  if (nseg == 1) {
    // The z column is read by every value slice and written by slice 0 only: an in-place
    // resume with several slices reads a private copy of the start state.
    const float *ini = init_state;
    if (shared_z) {
      if ((rc = private_start(&ini)) != FLA_OK) return rc;
      exact_init = ini;
    }
    // packed sequences: dispatch the longest first (the short ones fill in behind them)
    int *order = nullptr;
    if (cu_seqlens && B >= 2 && B <= kOrderMax) {
      void *o = nullptr;
      if ((rc = ws.get(B * (int64_t)sizeof(int), &o)) != FLA_OK) {
        ws.release();
        return rc;
      }
      order = static_cast<int *>(o);
      int n_i = (int)B;
      int64_t T_v = T, chunk_v = chunk;
      void *oargs[] = {&cu_seqlens, &n_i, &T_v, &chunk_v, &order};
      if (hipLaunchKernel(reinterpret_cast<const void *>(&seq_order_kernel),
                          dim3(blocks_for(B, kOrderThreads)), dim3(kOrderThreads), oargs, 0, s) !=
          hipSuccess) {
        ws.release();
        return FLA_ERR_DEVICE;
      }
    }
    a.seq_order = order;
    a.init = ini;
    a.init_bh_stride = dk * ncol;
    a.init_seg_stride = 0;
    a.fin = final_state;
    a.fin_bh_stride = dk * ncol;
    a.fin_seg_stride = 0;
    a.seg_decay = nullptr;
    a.state_only = 0;
    rc = launch(a, (unsigned)grid, s) == hipSuccess ? FLA_OK : FLA_ERR_DEVICE;
    if (rc == FLA_OK) rc = run_exact();
    const int rr = ws.release();
    return rc != FLA_OK ? rc : rr;
  }

  // Segment schedule: (A) end state of every segment from a zero start, (B) scan over
  // segments, (C) outputs of every segment from its start state.
  const int64_t ws_states = nbh * nseg * dk * ncol;
  if (gated && shared_z && (rc = private_start(&exact_init)) != FLA_OK) return rc;
  void *wsp = nullptr;
  if ((rc = ws.get(seg_ws_bytes(nseg), &wsp)) != FLA_OK) {
    ws.release();
    return rc;
  }
  float *wst = static_cast<float *>(wsp);
  float *wdec = wst + ws_states;

  a.init = nullptr;
  a.init_bh_stride = 0;
  a.init_seg_stride = 0;
  a.fin = wst;
  a.fin_bh_stride = nseg * dk * ncol;
  a.fin_seg_stride = dk * ncol;
  a.seg_decay = wdec;
  a.state_only = 1;
  const bool wide = !gated && bf16 && !norm && dv > kSlice && dk >= 32 && dk <= 128;
  if (const SegStateKernel st = gated ? nullptr
                                : wide ? find_seg_state_wide(dk)
                                       : find_seg_state(bf16, dk, norm)) {
    // constant decays: the end states are a plain reduction over each segment (seg_state.hpp),
    // in value slices of 128 columns where that kernel takes them
    ChunkArgs sa = a;
    const int64_t svs = wide ? (dv + 2 * kSlice - 1) / (2 * kSlice) : nvs;
    sa.nvs = (int)svs;
    const int64_t sgrid = ((nunits + 7) / 8) * 8 * svs;
    void *sargs[] = {&sa};
    rc = hipLaunchKernel(reinterpret_cast<const void *>(st), dim3((unsigned)sgrid), dim3(256), sargs,
                         0, s) == hipSuccess ? FLA_OK : FLA_ERR_DEVICE;
  } else {
    rc = launch(a, (unsigned)grid, s) == hipSuccess ? FLA_OK : FLA_ERR_DEVICE;
  }

  if (rc == FLA_OK) {
    const int64_t n = nbh * dk * ncol;
    int nseg_i = (int)nseg, dk_i = (int)dk, ncol_i = (int)ncol;
    const float *ini = init_state;
    float *fin = final_state;
    int64_t nbh_v = nbh;
    void *args[] = {&wst, &wdec, &ini, &fin, &nbh_v, &nseg_i, &dk_i, &ncol_i, &unsafe};
    if (hipLaunchKernel(reinterpret_cast<const void *>(&segment_scan_kernel),
                        dim3(blocks_for(n, kScanThreads)), dim3(kScanThreads), args, 0, s) != hipSuccess)
      rc = FLA_ERR_DEVICE;
  }
  if (rc == FLA_OK) {
    a.init = wst;
    a.init_bh_stride = nseg * dk * ncol;
    a.init_seg_stride = dk * ncol;
    a.fin = nullptr;
    a.seg_decay = nullptr;
    a.state_only = 0;
    rc = launch(a, (unsigned)grid, s) == hipSuccess ? FLA_OK : FLA_ERR_DEVICE;
  }
  if (rc == FLA_OK) rc = run_exact();
  const int rr = ws.release();
  return rc != FLA_OK ? rc : rr;
}

// The layer's input side: q, k, v = phi(x W_q), phi(x W_k), x W_v into token-major
// workspaces (proj.hpp), then the forward pass on them.
int proj_impl(const void *x, const void *w_q, const void *w_k, const void *w_v,
              const float *gate_or_gamma, const float *init_state, void *out, float *final_state,
              int64_t B, int64_t T, int64_t hidden, int64_t H, int64_t dk, int64_t dv,
              int64_t chunk, uint32_t flags, Workspace &ws) {
  if (flags & ~(FLA_ALL_FLAGS)) return FLA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || T < 0 || hidden < 1) return FLA_ERR_INVALID_ARG;
  if (T > 0 && (!x || !w_q || !w_k || !w_v || !out)) return FLA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(w_k, 16) || !aligned(w_v, 16))
    return FLA_ERR_INVALID_ARG;
  if (hidden % 32 != 0 || hidden > (1 << 20)) return FLA_ERR_UNSUPPORTED;
  if (!is_pow2_dim(dk) || !is_pow2_dim(dv) || H > (1 << 16) || (H * dk) % 16 || (H * dv) % 16)
    return FLA_ERR_UNSUPPORTED;
  if (B * T > ((int64_t)1 << 40) / (H * (dk > dv ? dk : dv))) return FLA_ERR_INVALID_ARG;
  const bool bf16 = (flags & FLA_BF16) != 0;
  const int64_t M = B * T;
  const int es = bf16 ? 2 : 4;
  if (T == 0) // nothing to project: the forward pass's own empty-sequence rule
    return fwd_impl(nullptr, nullptr, nullptr, gate_or_gamma, init_state, out, final_state, B, H,
                    0, dk, dv, chunk, (flags & ~FLA_PHI_ELU1) | FLA_LAYOUT_BTHD, 0, nullptr, ws);
  // everything the forward call checks, checked before the projections are enqueued
  {
    const int rc = check_common(B, H, dk, dv, (flags & ~FLA_PHI_ELU1) | FLA_LAYOUT_BTHD,
                                gate_or_gamma);
    if (rc != FLA_OK) return rc;
    if (!aligned(out, 16) || !aligned(init_state, 16) || !aligned(final_state, 16))
      return FLA_ERR_INVALID_ARG;
    if (H * (dk > dv ? dk : dv) > ((int64_t)1 << 20) || B * H > ((int64_t)1 << 26))
      return FLA_ERR_UNSUPPORTED;
    if (!is_chunk_arg(chunk)) return FLA_ERR_UNSUPPORTED;
    if (!find_launcher(bf16, dk, tile_for(chunk, dk, decay_kind(flags), bf16), decay_kind(flags),
                       (flags & FLA_NORMALIZE) != 0))
      return FLA_ERR_UNSUPPORTED;
  }
  void *pq = nullptr, *pk = nullptr, *pv = nullptr;
  int rc = ws.get(M * H * dk * es, &pq);
  if (rc == FLA_OK) rc = ws.get(M * H * dk * es, &pk);
  if (rc == FLA_OK) rc = ws.get(M * H * dv * es, &pv);
  if (rc != FLA_OK) {
    ws.release();
    return rc;
  }
  // the three projections in one launch (proj.hpp: they share x)
  ProjArgs pa{};
  pa.x = x;
  pa.w[0] = w_q; pa.w[1] = w_k; pa.w[2] = w_v;
  pa.y[0] = pq; pa.y[1] = pk; pa.y[2] = pv;
  pa.M = M;
  pa.K = (int)hidden;
  pa.n[0] = pa.n[1] = (int)(H * dk);
  pa.n[2] = (int)(H * dv);
  const int bn = bf16 ? ProjCfg<__bf16>::BN : ProjCfg<float>::BN;
  const int64_t bm = bf16 ? ProjCfg<__bf16>::BM : ProjCfg<float>::BM;
  for (int p = 0; p < 3; ++p) pa.nbn[p] = (pa.n[p] + bn - 1) / bn;
  pa.elu_mask = (flags & FLA_PHI_ELU1) ? 3 : 0;
  const int64_t tiles = ((M + bm - 1) / bm) * (pa.nbn[0] + pa.nbn[1] + pa.nbn[2]);
  const int64_t blocks = ((tiles + 7) / 8) * 8;
  if (blocks >= kMaxGrid) {
    ws.release();
    return FLA_ERR_UNSUPPORTED;
  }
  const void *fn = bf16 ? reinterpret_cast<const void *>(&proj_phi_kernel<__bf16>)
                        : reinterpret_cast<const void *>(&proj_phi_kernel<float>);
  void *args[] = {&pa};
  if (hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, ws.s) != hipSuccess) {
    ws.release();
    return FLA_ERR_DEVICE;
  }
  // phi is already applied: the forward pass takes the projected q, k as they are
  return fwd_impl(pq, pk, pv, gate_or_gamma, init_state, out, final_state, B, H, T, dk, dv, chunk,
                  (flags & ~FLA_PHI_ELU1) | FLA_LAYOUT_BTHD, 0, nullptr, ws);
}

int bwd_impl(const void *q, const void *k, const void *v, const float *gate_or_gamma,
             const float *init_state, const void *dout, const float *dfinal_state, void *dq,
             void *dk_out, void *dv_out, float *dgate, float *dinit_state, int64_t B, int64_t H,
             int64_t T, int64_t dk, int64_t dv, int64_t chunk, uint32_t flags,
             const int64_t *cu_seqlens, void *stream) {
  gate_or_gamma = nonnull_decay_if_empty(gate_or_gamma, T, flags);
  int rc = check_common(B, H, dk, dv, flags, gate_or_gamma);
  if (rc != FLA_OK) return rc;
  if (T < 0) return FLA_ERR_INVALID_ARG;
  const int kind = decay_kind(flags);
  const bool per_token_grad = kind == DECAY_GATE || kind == DECAY_TOKEN;
  if (dgate && !per_token_grad) return FLA_ERR_INVALID_ARG; // no gradient for gamma / none
  if (T > 0 && (!q || !k || !v || !dout || !dq || !dk_out || !dv_out)) return FLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk_out, 16) || !aligned(dv_out, 16) ||
      !aligned(init_state, 16) || !aligned(dfinal_state, 16) || !aligned(dinit_state, 16) ||
      !aligned(dgate, 16))
    return FLA_ERR_INVALID_ARG;
  if (flags & FLA_NORMALIZE) return FLA_ERR_UNSUPPORTED;
  const bool bthd = cu_seqlens != nullptr || (flags & FLA_LAYOUT_BTHD) != 0;
  if (bthd && H * (dk > dv ? dk : dv) > ((int64_t)1 << 20)) return FLA_ERR_UNSUPPORTED;
  // the backward tiles by 64 tokens whatever chunk the forward pass used (same function)
  if (!is_chunk_arg(chunk)) return FLA_ERR_UNSUPPORTED;
  chunk = 64;
  if (dk < 64 || dv < 64) return FLA_ERR_UNSUPPORTED;
  if (B * H > ((int64_t)1 << 26) || T > ((int64_t)1 << 40) / (B * H)) return FLA_ERR_INVALID_ARG;
  const bool bf16 = (flags & FLA_BF16) != 0;
  const BwdLauncher lq = find_bwd(bf16, dv, BWD_DQ, kind);
  const BwdLauncher lk = find_bwd(bf16, dv, BWD_DK, kind);
  const BwdLauncher lv = find_bwd(bf16, dk, BWD_DV, kind);
  if (!lq || !lk || !lv) return FLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nbh = B * H;
  if (T == 0) {
    if (dinit_state) return launch_fill(dinit_state, dfinal_state, nbh * dk * dv, s);
    return FLA_OK;
  }
  const int64_t nslk = dk / kSlice, nslv = dv / kSlice;
  if (nbh * (nslk > nslv ? nslk : nslv) >= kMaxGrid) return FLA_ERR_UNSUPPORTED;

  // workspace for the decay gradient: phi(q) dphi(q) per token and key, the final state's
  // term per key, and (per-token decay) one partial sum per 16 keys and token
  const bool want_dg = dgate != nullptr;
  const int64_t ntok = cu_seqlens ? T : B * T; // tokens over all sequences
  const int64_t n_rq = want_dg ? ntok * H * dk : 0;
  const int64_t n_ft = (want_dg && dfinal_state) ? nbh * dk : 0;
  const int64_t n_tp = (want_dg && kind == DECAY_TOKEN) ? H * nslk * 4 * ntok : 0;
  float *ws = nullptr;
  if (n_rq + n_ft + n_tp > 0 &&
      hipMallocAsync(reinterpret_cast<void **>(&ws), (n_rq + n_ft + n_tp) * sizeof(float), s) != hipSuccess)
    return FLA_ERR_DEVICE;

  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.decay = gate_or_gamma;
  a.init = init_state;
  a.dfinal = dfinal_state;
  a.grad_q = dq; a.grad_k = dk_out; a.grad_v = dv_out;
  a.dgate = dgate;
  a.dinit = dinit_state;
  a.rq = want_dg ? ws : nullptr;
  a.fterm = n_ft ? ws + n_rq : nullptr;
  a.tpart = n_tp ? ws + n_rq + n_ft : nullptr;
  a.T = T;
  a.ntok = ntok;
  a.bthd = bthd ? 1 : 0;
  a.cu_seqlens = cu_seqlens;
  a.H = (int)H; a.dk = (int)dk; a.dv = (int)dv;
  a.phi_elu1 = (flags & FLA_PHI_ELU1) ? 1 : 0;
  a.want_dg = want_dg ? 1 : 0;

  rc = FLA_OK;
  // dphi(q) (forward in time; writes dq and the workspace terms)
  a.nsl = (int)nslk; a.nunits = (int)(nbh * nslk);
  if (lq(a, (unsigned)a.nunits, s) != hipSuccess) rc = FLA_ERR_DEVICE;
  // dv and the initial state's gradient (reverse)
  if (rc == FLA_OK) {
    a.nsl = (int)nslv; a.nunits = (int)(nbh * nslv);
    if (lv(a, (unsigned)a.nunits, s) != hipSuccess) rc = FLA_ERR_DEVICE;
  }
  // dphi(k) and the decay gradient (reverse)
  if (rc == FLA_OK) {
    a.nsl = (int)nslk; a.nunits = (int)(nbh * nslk);
    if (lk(a, (unsigned)a.nunits, s) != hipSuccess) rc = FLA_ERR_DEVICE;
  }
  if (rc == FLA_OK && n_tp) {
    const float *tp = a.tpart;
    const float *dec = gate_or_gamma;
    int64_t H_v = H, ntok_v = ntok, T_v = T;
    int nparts = (int)nslk * 4; // partial sums per token: 4 waves per key slice
    int bthd_i = bthd ? 1 : 0;
    void *args[] = {&tp, &dec, &dgate, &H_v, &ntok_v, &T_v, &nparts, &bthd_i};
    if (hipLaunchKernel(reinterpret_cast<const void *>(&token_dgate_kernel),
                        dim3(blocks_for(H * ntok, 256)), dim3(256), args, 0, s) != hipSuccess)
      rc = FLA_ERR_DEVICE;
  }
  if (ws && hipFreeAsync(ws, s) != hipSuccess) rc = FLA_ERR_DEVICE;
  return rc;
}

int gdn_impl(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
             const float *init_state, void *out, float *final_state, int64_t B, int64_t H,
             int64_t T, int64_t dk, int64_t dv, int64_t chunk, uint32_t flags, void *stream) {
  if (flags & ~FLA_BF16) return FLA_ERR_INVALID_ARG; // no decay / feature-map / layout options
  if (B < 1 || H < 1 || B > (1 << 24) || H > (1 << 24) || T < 0) return FLA_ERR_INVALID_ARG;
  if (dk < 1 || dv < 1) return FLA_ERR_INVALID_ARG;
  if (T > 0 && (!q || !k || !v || !out || !alpha || !beta)) return FLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(init_state, 16) || !aligned(final_state, 16) || !aligned(alpha, 4) ||
      !aligned(beta, 4))
    return FLA_ERR_INVALID_ARG;
  // 64-token tiles for any accepted chunk size (the chunking does not change the function)
  if (!is_chunk_arg(chunk)) return FLA_ERR_UNSUPPORTED;
  if (dv % kSlice != 0 || dv > 256) return FLA_ERR_UNSUPPORTED;
  if (B * H > ((int64_t)1 << 26) || T > ((int64_t)1 << 40) / (B * H)) return FLA_ERR_INVALID_ARG;
  const bool bf16 = (flags & FLA_BF16) != 0;
  const GdnLaunchers launch = gdn_launchers(bf16, (int)dk);
  if (!launch.prep || !launch.state) return FLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nbh = B * H;
  if (T == 0) {
    if (final_state && final_state != init_state) return launch_fill(final_state, init_state, nbh * dk * dv, s);
    return FLA_OK;
  }
  const int64_t nvs = dv / kSlice;
  const int64_t nch = (T + 63) / 64;
  if (nbh * nvs >= kMaxGrid || nbh * nch >= kMaxGrid) return FLA_ERR_UNSUPPORTED;
  // workspace: Tb = T diag(beta) per chunk (its lower-triangle blocks), in the input type
  const int64_t tb_bytes = nbh * nch * kGdnTbElems * (bf16 ? 2 : 4);
  char *ws = nullptr;
  if (hipMallocAsync(reinterpret_cast<void **>(&ws), tb_bytes, s) != hipSuccess)
    return FLA_ERR_DEVICE;
  GdnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.alpha = alpha; a.beta = beta;
  a.init = init_state;
  a.fin = final_state;
  a.out = out;
  a.T = T;
  a.H = (int)H; a.dv = (int)dv;
  a.nvs = (int)nvs;
  a.nch = (int)nch;
  a.tb = ws;
  int rc = FLA_OK;
  a.nunits = (int)(nbh * nch);
  if (launch.prep(a, (unsigned)a.nunits, s) != hipSuccess) rc = FLA_ERR_DEVICE;
  a.nunits = (int)(nbh * nvs);
  if (rc == FLA_OK && launch.state(a, (unsigned)a.nunits, s) != hipSuccess) rc = FLA_ERR_DEVICE;
  if (hipFreeAsync(ws, s) != hipSuccess) rc = FLA_ERR_DEVICE;
  return rc;
}

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up once per device with
// that device current (the array's name in host code is only a host-side stand-in).
int scratch_address(void **p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLA_ERR_DEVICE;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return FLA_ERR_DEVICE;
    addr[dev] = a;
  }
  *p = addr[dev];
  return FLA_OK;
}

} // namespace
} // namespace fla

extern "C" {

int fla_gdn_fwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                const float *init_state, void *out, float *final_state, int64_t B, int64_t H,
                int64_t T, int64_t dk, int64_t dv, int64_t chunk, uint32_t flags, void *stream) {
  return fla::gdn_impl(q, k, v, alpha, beta, init_state, out, final_state, B, H, T, dk, dv,
                       chunk, flags, stream);
}

int fla_linattn_bwd(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                    const float *init_state, const void *dout, const float *dfinal_state,
                    void *dq, void *dk, void *dv, float *dgate, float *dinit_state, int64_t B,
                    int64_t H, int64_t T, int64_t dk_dim, int64_t dv_dim, int64_t chunk,
                    uint32_t flags, void *stream) {
  return fla::bwd_impl(q, k, v, gate_or_gamma, init_state, dout, dfinal_state, dq, dk, dv, dgate,
                       dinit_state, B, H, T, dk_dim, dv_dim, chunk, flags, nullptr, stream);
}

int fla_linattn_bwd_varlen(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                           const float *init_state, const void *dout, const float *dfinal_state,
                           void *dq, void *dk, void *dv, float *dgate, float *dinit_state,
                           const int64_t *cu_seqlens, int64_t n_seqs, int64_t total_T, int64_t H,
                           int64_t dk_dim, int64_t dv_dim, int64_t chunk, uint32_t flags,
                           void *stream) {
  if (!cu_seqlens || !fla::aligned(cu_seqlens, 8)) return FLA_ERR_INVALID_ARG;
  return fla::bwd_impl(q, k, v, gate_or_gamma, init_state, dout, dfinal_state, dq, dk, dv, dgate,
                       dinit_state, n_seqs, H, total_T, dk_dim, dv_dim, chunk,
                       flags | FLA_LAYOUT_BTHD, cu_seqlens, stream);
}

const char *fla_status_string(int status) {
  switch (status) {
  case FLA_OK: return "ok";
  case FLA_ERR_INVALID_ARG: return "invalid argument";
  case FLA_ERR_UNSUPPORTED: return "unsupported shape or option";
  case FLA_ERR_DEVICE: return "device launch or allocation failed";
  case FLA_ERR_SCRATCH: return "request needs more than the no-allocation entry point's scratch";
  default: return "unknown status";
  }
}

int fla_linattn_fwd(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                    const float *init_state, void *out, float *final_state, int64_t B,
                    int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk,
                    uint32_t flags, void *stream) {
  fla::Workspace ws;
  ws.s = static_cast<hipStream_t>(stream);
  return fla::fwd_impl(q, k, v, gate_or_gamma, init_state, out, final_state, B, H, T, dk, dv,
                       chunk, flags, 0, nullptr, ws);
}

int fla_linattn_fwd_noalloc(const void *q, const void *k, const void *v,
                            const float *gate_or_gamma, const float *init_state, void *out,
                            float *final_state, int64_t B, int64_t H, int64_t T, int64_t dk,
                            int64_t dv, int64_t chunk, uint32_t flags, void *stream) {
  fla::Workspace ws;
  ws.s = static_cast<hipStream_t>(stream);
  void *base = nullptr;
  const int rc = fla::scratch_address(&base);
  if (rc != FLA_OK) return rc;
  ws.base = static_cast<char *>(base);
  ws.cap = fla::kScratchBytes;
  return fla::fwd_impl(q, k, v, gate_or_gamma, init_state, out, final_state, B, H, T, dk, dv,
                       chunk, flags, 0, nullptr, ws);
}

int fla_linattn_fwd_proj(const void *x, const void *w_q, const void *w_k, const void *w_v,
                         const float *gate_or_gamma, const float *init_state, void *out,
                         float *final_state, int64_t B, int64_t T, int64_t hidden, int64_t H,
                         int64_t dk, int64_t dv, int64_t chunk, uint32_t flags, void *stream) {
  fla::Workspace ws;
  ws.s = static_cast<hipStream_t>(stream);
  return fla::proj_impl(x, w_q, w_k, w_v, gate_or_gamma, init_state, out, final_state, B, T,
                        hidden, H, dk, dv, chunk, flags, ws);
}

int fla_linattn_fwd_varlen(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                           const float *init_state, void *out, float *final_state,
                           const int64_t *cu_seqlens, int64_t n_seqs, int64_t total_T, int64_t H,
                           int64_t dk, int64_t dv, int64_t chunk, uint32_t flags, void *stream) {
  if (!cu_seqlens || !fla::aligned(cu_seqlens, 8)) return FLA_ERR_INVALID_ARG;
  fla::Workspace ws;
  ws.s = static_cast<hipStream_t>(stream);
  return fla::fwd_impl(q, k, v, gate_or_gamma, init_state, out, final_state, n_seqs, H, total_T,
                       dk, dv, chunk, flags | FLA_LAYOUT_BTHD, 0, cu_seqlens, ws);
}

int fla_linattn_fwd_segments(const void *q, const void *k, const void *v,
                             const float *gate_or_gamma, const float *init_state, void *out,
                             float *final_state, int64_t B, int64_t H, int64_t T, int64_t dk,
                             int64_t dv, int64_t chunk, uint32_t flags, int64_t n_segments,
                             void *stream) {
  fla::Workspace ws;
  ws.s = static_cast<hipStream_t>(stream);
  return fla::fwd_impl(q, k, v, gate_or_gamma, init_state, out, final_state, B, H, T, dk, dv,
                       chunk, flags, n_segments, nullptr, ws);
}

int fla_linattn_segments_for(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                             int64_t chunk, uint32_t flags, int64_t *n_segments) {
  if (!n_segments || T < 0) return FLA_ERR_INVALID_ARG;
  const bool has_decay = (flags & fla::kDecayBits) != 0;
  static const float dummy[4] = {0.f, 0.f, 0.f, 0.f};
  int rc = fla::check_common(B, H, dk, dv, flags, has_decay ? dummy : nullptr);
  if (rc != FLA_OK) return rc;
  if (!fla::is_chunk_arg(chunk)) return FLA_ERR_UNSUPPORTED;
  chunk = fla::tile_for(chunk, dk, fla::decay_kind(flags), (flags & FLA_BF16) != 0);
  const int64_t nch = (T + chunk - 1) / chunk;
  int64_t p = T == 0 ? 1 : fla::auto_segments(B, H, T, dv, chunk);
  if (p > nch && nch > 0) p = nch;
  *n_segments = p;
  return FLA_OK;
}

int fla_linattn_step(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                     float *state, void *out, int64_t B, int64_t H, int64_t dk, int64_t dv,
                     uint32_t flags, void *stream) {
  int rc = fla::check_common(B, H, dk, dv, flags, gate_or_gamma);
  if (rc != FLA_OK) return rc;
  if (!q || !k || !v || !out || !state) return FLA_ERR_INVALID_ARG;
  if (!fla::aligned(q, 16) || !fla::aligned(k, 16) || !fla::aligned(v, 16) ||
      !fla::aligned(out, 16) || !fla::aligned(state, 16))
    return FLA_ERR_INVALID_ARG;
  const int64_t nbh = B * H;
  if (nbh >= fla::kMaxGrid) return FLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float *dec = gate_or_gamma;
  int kind = fla::decay_kind(flags);
  int Hi = (int)H, dki = (int)dk, dvi = (int)dv;
  int phi = (flags & FLA_PHI_ELU1) ? 1 : 0, norm = (flags & FLA_NORMALIZE) ? 1 : 0;
  void *args[] = {const_cast<void **>(&q), const_cast<void **>(&k), const_cast<void **>(&v),
                  &dec, &kind, &state, &out, &Hi, &dki, &dvi, &phi, &norm};
  const void *fn = (flags & FLA_BF16) ? reinterpret_cast<const void *>(&fla::step_kernel<__bf16>)
                                      : reinterpret_cast<const void *>(&fla::step_kernel<float>);
  if (hipLaunchKernel(fn, dim3((unsigned)nbh), dim3(fla::kStepThreads), args, 0, s) != hipSuccess)
    return FLA_ERR_DEVICE;
  return FLA_OK;
}

} // extern "C"
