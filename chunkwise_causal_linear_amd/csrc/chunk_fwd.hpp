// Chunkwise causal linear attention, forward — fused gfx950 kernel.
//
// Per (b, h) and chunk n of length L (tokens t = nC + i), with b_i[c] the inclusive
// product of the decays inside the chunk (e^{lambda_i}), unrolling the recurrence
// S_t = G_t (.) S_{t-1} + v_t phi(k_t)^T (textbook chapter 1.6, "linear attention";
// RetNet gamma / GLA gate per the FLA posts; chunk mode = the chapter's remark on
// decay-masked linear attention trained in matmul-friendly chunks) gives, with the
// state H = S^T (dk x dv) before the chunk:
//   gate:  O = tril(Qt Kt^T) V + Qt H,        H <- diag(b_{L-1}) (H + Kt^T V)
//          Qt = phi(q) (.) b,  Kt = phi(k) / b
//   gamma: O = (tril(phi(q) phi(k)^T) (.) gamma^{i-j}) V + diag(gamma^{i+1}) phi(q) H,
//          H <- gamma^L H + phi(k)^T diag(gamma^{L-1-j}) V          (no overflow)
//   none:  the gamma form with gamma = 1.
// The normaliser z is the state column of an all-ones value: den = A 1 + Qt z.
//
// Workgroup = 6 or 8 waves for one (b, h, segment, 64-wide slice of dv):
//   consumer waves (2 for dk <= 128, else 4) each own 32 or 16 value columns: their
//     slice of the fp32 state H lives in MFMA accumulators for the whole sequence; per chunk they run
//     S3  A^T = Kt Qt^T tile by tile, causal / decay mask, O^T += V^T A^T,
//     S6  O^T += H^T Qt^T (H converted to MFMA operands in registers), normalise, store,
//     S4/S5  H <- decay (H + Kt^T V) (or gamma^L H + Kt^T V');
//   4 producer waves prefetch q, k, v, gate one or two chunks ahead in registers,
//     apply phi (S1) and the decay factors (S2: per-key cumulative product down the chunk
//     by a wave-level shuffle scan), and write Qt, Kt, V row-major into an LDS stage.
// With two LDS stages producers prepare chunk n+1 while consumers compute chunk n
// (one barrier per chunk).  Kt^T and V^T operands are read from the row-major tiles
// with the gfx950 LDS transpose load (ds_read_b64_tr_b16), so no tile is ever written
// transposed.  Outputs are computed transposed (O^T tiles): each lane stores 4
// adjacent values of one output row.
//
// MFMA operand convention (v_mfma_f32_16x16x32_bf16): lane l = 16 g + li supplies row
// (A) or column (B) li; its 8 K-slots hold k = 32u + 4g + s (s < 4) and
// k = 32u + 16 + 4g + (s - 4) (s >= 4).  That is the accumulator layout (lane holds
// rows 4g + r of column li) of two adjacent 16-row tiles, so result tiles become
// operands without a shuffle.  fp32 (v_mfma_f32_16x16x4_f32): four MFMAs per 16-k
// block, MFMA r using k = 16u + 4g + r in lane group g.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// DECAY_TOKEN: a per-token scalar gate alpha_t (one value per token and head), handled
// as the per-key gate with alpha_t on every key column
enum : int { DECAY_NONE = 0, DECAY_GAMMA = 1, DECAY_GATE = 2, DECAY_TOKEN = 3 };

constexpr int kMaxThreads = 512; // consumer + 4 producer waves
constexpr int kSlice = 64;      // value columns per workgroup (16 per consumer wave)
constexpr int kMaxLds = 163840; // gfx950 LDS per workgroup

struct ChunkArgs {
  const void *q, *k, *v;
  const float *decay;      // gamma [H] or gate [B][H][T][dk]
  const float *init;       // start states (or null = zeros)
  int64_t init_bh_stride;  // elements between (b,h) start states
  int64_t init_seg_stride; // elements between segment start states
  float *fin;              // end states (or null)
  int64_t fin_bh_stride, fin_seg_stride;
  float *seg_decay;        // [BH][nseg][dk]: product of the decays over each segment
  void *out;
  int64_t T;
  int64_t seg_len;         // tokens per segment (a multiple of the chunk)
  int H, dv, ncol;
  int nseg, nvs, nunits;   // nunits = B * H * nseg
  int phi_elu1;
  int state_only;          // 1: only the end state (and segment decay), no outputs
  int bthd;                // 1: q, k, v, out, gate in token-major [B][T][H][d] (or packed
                           //    [total][H][d] with cu_seqlens); 0: [B][H][T][d]
  const int64_t *cu_seqlens; // packed sequences: [B + 1] token offsets (bthd only), or null
  const int *seq_order;    // packed sequences: unit order -> sequence (longest first), or null
  int *unsafe;             // gated kinds: [B*H*nseg][4], written by value slice 0's producer
                           //   waves (one word each): 1 if a chunk's decay product fell below
                           //   kSafeDecay (the factorised form is then not used for the unit)
};

// Smallest product of the decays along one chunk (per key) for which the factorised form
// Qt = phi(q) b, Kt = phi(k) / b is used: 1 / b stays below 2^100, far from fp32 / bf16
// overflow for any reasonable |phi(k)|, and phi(q) b far above the denormal range.  A unit
// with a chunk below it is recomputed by the exact 16-token kernel (exact_fwd.hpp).
constexpr float kSafeDecay = 0x1p-100f;

// PB: bytes of padding after each Qt / Kt row (the tile's row stride is DK + PB / ES
// elements); see Cfg below for the choice.
template <typename TIn, int DK, int C, int DECAY, bool NORM, int PB>
struct CfgP {
  static constexpr int ES = sizeof(TIn);
  static constexpr bool BF = (ES == 2);
  static constexpr int PAD = PB / ES;
  static constexpr int LQ = DK + PAD;    // row stride (elements) of Qt, Kt
  static constexpr int NB = C / 16;      // 16-row blocks per chunk
  static constexpr int NCB = DK / 16;    // 16-row blocks of the state
  static constexpr int TPU = BF ? 2 : 1; // 16-blocks per MFMA K unit
  static constexpr int NU_DK = (NCB + TPU - 1) / TPU;
  static constexpr int NU_C = (NB + TPU - 1) / TPU;
  static constexpr bool HI_DK = !(BF && DK == 16);
  static constexpr bool HI_C = !(BF && C == 16);
  // consumer waves: NCW waves, each owning ET 16-column tiles of the 64-wide value slice
  // (with two tiles a wave, both share every Qt/Kt operand fragment).  Four waves of one
  // tile for every decay: two waves of two tiles ran the per-key gate at the same speed
  // (its producers and the memory system bound it) but needed scratch registers, and ran
  // the constant decays 1.4x slower (their consumer chain bounds them).
  static constexpr int NCW = 4;
  static constexpr int ET = 4 / NCW;
  static constexpr int NT = 64 * (NCW + 4);     // + 4 producer waves
  // keep the Kt fragments of earlier row blocks in registers (unrolled row-block loop)
  static constexpr bool KCACHE = DK <= 128 && C <= 64 && ET == 1;
  // producer mapping for q/k/gate: wave p owns columns [p W, (p+1) W); a lane owns G
  // consecutive columns and RPT consecutive rows; LPR lanes share a row.  The token-major
  // and packed layouts of the per-key gate at dk = 128 (bf16, 64-token chunks; RH2) split
  // the rows instead (row halves, see the producer waves).
  static constexpr bool RH2 = DECAY == DECAY_GATE && BF && DK == 128 && C == 64;
  static constexpr int W = DK / 4;
  static constexpr int G = W >= 8 ? 8 : W;
  static constexpr int LPR = W / G;
  static constexpr int RP = 64 / LPR;
  static constexpr int RPT = C >= RP ? C / RP : 1;
  static constexpr int NRG = C / RPT;
  static constexpr int PACTIVE = NRG * LPR;
  // producer mapping for v: 8 columns per lane, 8 lanes per row, 256 producer lanes
  static constexpr int RPTV = C >= 32 ? C / 32 : 1;
  static constexpr int VACTIVE = C >= 32 ? 256 : C * 8;
  // registers held per prefetched chunk (32-bit words per producer lane)
  // gated kinds: the producers scan GS columns of the gate (the token gate is one column)
  static constexpr bool GATED = DECAY == DECAY_GATE || DECAY == DECAY_TOKEN;
  static constexpr int GS = DECAY == DECAY_TOKEN ? 1 : G;
  static constexpr int STAGE_WORDS = 2 * RPT * G * ES / 4 + (GATED ? RPT * GS : 0) +
                                     RPTV * 8 * ES / 4;
  static constexpr int PF_BASE = (STAGE_WORDS <= 64 && C <= 64 && !NORM) ? 2 : 1;
  // Score tiles shared through LDS: the masked score tiles of a chunk are computed once,
  // split over the consumer waves, into an LDS buffer that every wave reads for O += A V.
  // Tile (ib, jb), jb <= ib, is number ib (ib + 1) / 2 + jb; when the slots outnumber the
  // tiles one more tile takes the writes of the idle slots.
  static constexpr int NTILES = NB * (NB + 1) / 2;
  static constexpr int SLOTS = (NTILES + NCW - 1) / NCW; // score tiles per consumer wave
  static constexpr int PTILE = 256;                      // elements per score tile
  static constexpr int PBUF_BYTES = (NTILES + (SLOTS * NCW > NTILES ? 1 : 0)) * PTILE * ES;
  static constexpr int PW_BYTES = DECAY == DECAY_GAMMA ? ((C + 4) / 4) * 16 : 0;
  // gated kinds: one word per producer wave (see OFF_FLAG); RH2 adds two words (16 bytes)
  // of first-half progress and DK floats of first-half column products
  static constexpr int FLAG_BYTES = GATED ? 16 + (RH2 ? 16 + DK * 4 : 0) : 0;
  static constexpr int QT_BYTES = C * LQ * ES; // one Qt or Kt tile
  static constexpr int EL_BYTES = GATED ? DK * 4 : 0;
  // row stride of V: 40 words (8 mod 32) keeps the transposed operand loads conflict-free;
  // 36 words where the split schedule needs the room
  static constexpr int LV_W = kSlice + (BF ? 16 : 4);
  static constexpr int LV_T = kSlice + (BF ? 8 : 4);
  static constexpr int stage_bytes(int lv) { return 2 * QT_BYTES + C * lv * ES + EL_BYTES; }
  static constexpr int split_bytes(int lv) {
    return QT_BYTES + 2 * (QT_BYTES + C * lv * ES + EL_BYTES) + PBUF_BYTES + PW_BYTES + FLAG_BYTES;
  }
  // Schedules, by the LDS they need:
  //  SHARE: three stages {Qt, Kt, V, eL} and two score buffers; iteration n computes the
  //    score tiles of chunk n and the outputs and state update of chunk n - 1 (one barrier
  //    a chunk);
  //  SPLIT: one Qt tile, two {Kt, V, eL} stages and one score buffer; two barriers a chunk:
  //    phase 1 the inter-chunk term and the score tiles, phase 2 O += A V, the output and
  //    the state update; producers write Kt and V of the next chunk during phase 1 and its
  //    Qt during phase 2;
  //  otherwise the per-wave schedule: two stages (one where two do not fit), each consumer
  //    wave computing the score tiles it needs itself.
  static constexpr bool SHARE =
      3 * stage_bytes(LV_W) + 2 * PBUF_BYTES + PW_BYTES + FLAG_BYTES <= kMaxLds;
  static constexpr bool SPLIT = !SHARE && split_bytes(LV_T) <= kMaxLds;
  static constexpr int LV = (SPLIT && split_bytes(LV_W) > kMaxLds) ? LV_T : LV_W;
  static constexpr int PF = SPLIT ? 1 : PF_BASE; // chunks the producers load ahead
  // split schedule without a gate: Qt = phi(q) is formed when the Qt tile is free, from
  // the q rows still in the staging registers (no copy held through phase 1)
  static constexpr bool Q_LATE = SPLIT && !GATED;
  // LDS map (bytes).  SHARE / per-wave: [STAGES] x {Qt, Kt, V, eL}, [2] x score tiles
  // (SHARE), gamma powers.  SPLIT: Qt, [2] x {Kt, V, eL}, score tiles, gamma powers.
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + QT_BYTES;
  static constexpr int OFF_V = OFF_K + QT_BYTES;
  static constexpr int OFF_EL = OFF_V + C * LV * ES;
  static constexpr int STAGE_BYTES = OFF_EL + EL_BYTES;
  static constexpr int KV_BYTES = QT_BYTES + C * LV * ES + EL_BYTES; // SPLIT {Kt, V, eL}
  static constexpr int STAGES =
      SHARE ? 3 : SPLIT ? 2 : (2 * STAGE_BYTES + PW_BYTES + FLAG_BYTES <= kMaxLds ? 2 : 1);
  static constexpr int OFF_P = SPLIT ? QT_BYTES + 2 * KV_BYTES : STAGES * STAGE_BYTES;
  static constexpr int OFF_PW = OFF_P + (SHARE ? 2 * PBUF_BYTES : SPLIT ? PBUF_BYTES : 0);
  // gated kinds: one word per producer wave, 1 once a chunk's decay product was unsafe
  static constexpr int OFF_FLAG = OFF_PW + PW_BYTES;
  static constexpr int LDS = OFF_FLAG + FLAG_BYTES;
  static constexpr bool FITS = LDS <= kMaxLds;
  // byte offsets of the tiles of chunk n
  __device__ static int q_at(int n) { return SPLIT ? 0 : (n % STAGES) * STAGE_BYTES + OFF_Q; }
  __device__ static int k_at(int n) {
    return SPLIT ? QT_BYTES + (n & 1) * KV_BYTES : (n % STAGES) * STAGE_BYTES + OFF_K;
  }
  __device__ static int v_at(int n) {
    return SPLIT ? 2 * QT_BYTES + (n & 1) * KV_BYTES : (n % STAGES) * STAGE_BYTES + OFF_V;
  }
  __device__ static int el_at(int n) {
    return SPLIT ? 2 * QT_BYTES + C * LV * ES + (n & 1) * KV_BYTES
                 : (n % STAGES) * STAGE_BYTES + OFF_EL;
  }
  __device__ static int p_at(int n) { return OFF_P + (SHARE ? (n & 1) * PBUF_BYTES : 0); }
  // state row order (bf16, shared score tiles): accumulator row m = 4g + r of state
  // block cb = 2u + s holds key index 32u + 8g + 4s + r, so that the bf16 operand built
  // from blocks 2u and 2u+1 has k = 32u + 8g + slot, the order of 16-byte LDS reads
  static constexpr bool PERM = (SHARE || SPLIT) && BF && HI_DK;
  // score tiles by row-block pairs: consumer wave w computes every tile of row blocks w and
  // NB-1-w (NB + 1 tiles, the same for every wave), each Qt row block and Kt column block
  // read once (code specialised per wave)
  static constexpr bool PAIRS = SPLIT && NB == 2 * NCW;
  // scheduling fences in the shared-score consumer: between row blocks and before the
  // next chunk's score tiles (needed to stay within the registers with two tiles a wave)
  static constexpr int FENCE = ET >= 2 ? 3 : 1; // bit 0: row blocks, bit 1: scores
  __device__ static constexpr int state_row(int cb, int g, int r) {
    return PERM ? 32 * (cb >> 1) + 8 * g + 4 * (cb & 1) + r : 16 * cb + 4 * g + r;
  }
};

// Row padding of the Qt / Kt tiles.  With 16 bytes (bf16 row stride = 4 words mod 64) the
// 16-byte operand reads of 16 rows collide in the LDS banks and take 1.8x the cycles of a
// stride of 8 words mod 64 (32 bytes of padding), and the transposed reads 1.1-1.3x
// (measured with an in-bounds read-pattern probe on gfx950).  bf16 tiles take the 32-byte
// padding where it leaves the schedule and the stage count unchanged; where the wider rows
// would push the tiles into a schedule with fewer stages (128-token tiles) the 16-byte
// padding stays.
template <typename TIn, int DK, int C, int DECAY, bool NORM>
constexpr int qk_pad_bytes() {
  using A = CfgP<TIn, DK, C, DECAY, NORM, 16>;
  using B = CfgP<TIn, DK, C, DECAY, NORM, 32>;
  return (A::BF && B::FITS && A::SHARE == B::SHARE && A::SPLIT == B::SPLIT &&
          A::STAGES == B::STAGES && A::LV == B::LV)
             ? 32
             : 16;
}
template <typename TIn, int DK, int C, int DECAY, bool NORM>
struct Cfg : CfgP<TIn, DK, C, DECAY, NORM, qk_pad_bytes<TIn, DK, C, DECAY, NORM>()> {};

// ---------------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ float rcp_f(float x) { return __builtin_amdgcn_rcpf(x); }

// N consecutive 32-bit words from global memory (N = 2, 4 or 8).
template <int N>
__device__ __forceinline__ void ld_words(uint32_t *w, const void *p) {
  if constexpr (N == 2) {
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    w[0] = x.x; w[1] = x.y;
  } else {
    static_assert(N % 4 == 0, "word count");
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const uint4 x = reinterpret_cast<const uint4 *>(p)[i / 4];
      w[i] = x.x; w[i + 1] = x.y; w[i + 2] = x.z; w[i + 3] = x.w;
    }
  }
}

// Unpack N elements of TIn held in 32-bit words to fp32.
template <typename TIn, int N>
__device__ __forceinline__ void unpack(float *f, const uint32_t *w) {
  if constexpr (sizeof(TIn) == 2) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// Pack N fp32 values as TIn elements into 32-bit words.
template <typename TIn, int N>
__device__ __forceinline__ void pack_words(uint32_t *w, const float *f) {
  if constexpr (sizeof(TIn) == 2) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const bf16x2 b = {(__bf16)f[2 * i], (__bf16)f[2 * i + 1]};
      w[i] = __builtin_bit_cast(uint32_t, b);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = __float_as_uint(f[i]);
  }
}
// Store N (2, 4 or 8) 32-bit words to LDS.
template <int N>
__device__ __forceinline__ void st_words_lds(void *p, const uint32_t *w) {
  if constexpr (N == 2) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      reinterpret_cast<uint4 *>(p)[i / 4] = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
  }
}

// Store N (4 or 8) fp32 values as consecutive TIn elements in LDS.
template <typename TIn, int N>
__device__ __forceinline__ void st_lds(TIn *p, const float *f) {
  if constexpr (sizeof(TIn) == 2) {
    if constexpr (N == 8) {
      bf16x8 x;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (__bf16)f[i];
      *reinterpret_cast<bf16x8 *>(p) = x;
    } else {
      static_assert(N == 4, "width");
      *reinterpret_cast<bf16x4 *>(p) = bf16x4{(__bf16)f[0], (__bf16)f[1], (__bf16)f[2], (__bf16)f[3]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<float4 *>(p + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
  }
}

// MFMA fragments ------------------------------------------------------------------
template <typename TIn>
using Frag = std::conditional_t<sizeof(TIn) == 2, bf16x8, f32x4>;

// Operand fragment from an LDS row whose K index is contiguous: K unit u.
template <typename TIn, bool HI>
__device__ __forceinline__ Frag<TIn> ld_frag(const TIn *row, int u, int g) {
  if constexpr (sizeof(TIn) == 2) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + 32 * u + 4 * g);
    bf16x4 hi;
    if constexpr (HI) hi = *reinterpret_cast<const bf16x4 *>(row + 32 * u + 16 + 4 * g);
    else hi = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return *reinterpret_cast<const f32x4 *>(row + 16 * u + 4 * g);
  }
}

// Operand fragment under the contiguous K convention (lane group g holds k = 32u + 8g + s):
// one 16-byte load.  Used where both operands of an MFMA come from LDS (the intra-chunk
// score tiles), where it avoids the bank conflicts of two 8-byte loads.
template <typename TIn, bool HI>
__device__ __forceinline__ Frag<TIn> ld_frag_c(const TIn *row, int u, int g) {
  if constexpr (sizeof(TIn) == 2) {
    if constexpr (HI) {
      return *reinterpret_cast<const bf16x8 *>(row + 32 * u + 8 * g);
    } else {
      const __bf16 z = (__bf16)0.f;
      bf16x8 r = {z, z, z, z, z, z, z, z};
      if (g < 2) r = *reinterpret_cast<const bf16x8 *>(row + 32 * u + 8 * g);
      return r;
    }
  } else {
    return *reinterpret_cast<const f32x4 *>(row + 16 * u + 4 * g);
  }
}

// Operand fragment whose K index runs down the rows of a row-major LDS tile (stride ld):
// lane (g, li) gets column col0 + CS (li/4) + li%4 at the rows of K unit u (CS = 4: the
// 16 consecutive columns from col0).  bf16: two LDS transpose loads (in each 16-lane group
// lane q addresses row r0 + q/4, columns col0 + CS (q%4) .. +3; lane p receives element
// p%4 of the group addressed by lanes 4y + p/4, y = 0..3).  fp32: four scalar loads.
template <typename TIn, bool HI, int CS = 4>
__device__ __forceinline__ Frag<TIn> ld_frag_t(const TIn *tile, int ld, int col0, int u, int g,
                                               int li) {
  if constexpr (sizeof(TIn) == 2) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int r0 = 32 * u + 4 * g + (li >> 2);
    const int c = col0 + CS * (li & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + r0 * ld + c));
    i16x4 hi = {0, 0, 0, 0};
    if constexpr (HI)
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + (r0 + 16) * ld + c));
    const bf16x4 l = __builtin_bit_cast(bf16x4, lo), h = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  } else {
    static_assert(CS == 4, "fp32 tiles use consecutive columns");
    const TIn *p = tile + (16 * u + 4 * g) * ld + col0 + li;
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
  }
}

// The same fragments from a lane base pointer (the lane-dependent part of the address
// already added), so that every other offset is a compile-time constant that the
// compiler folds into the LDS instruction.  Contiguous: base = row li, column 8g (bf16)
// or 4g (fp32); transposed: base = row 4g + li/4, column CS (li%4) (bf16) or row 4g,
// column li (fp32).
template <typename TIn, bool HI>
__device__ __forceinline__ Frag<TIn> ld_frag_c_at(const TIn *base, int u, int g) {
  if constexpr (sizeof(TIn) == 2) {
    if constexpr (HI) {
      return *reinterpret_cast<const bf16x8 *>(base + 32 * u);
    } else {
      const __bf16 z = (__bf16)0.f;
      bf16x8 r = {z, z, z, z, z, z, z, z};
      if (g < 2) r = *reinterpret_cast<const bf16x8 *>(base + 32 * u);
      return r;
    }
  } else {
    return *reinterpret_cast<const f32x4 *>(base + 16 * u);
  }
}
// split K convention (k = 32u + 4g + s, 32u + 16 + 4g + s - 4); base = row li, column 4g
template <typename TIn, bool HI>
__device__ __forceinline__ Frag<TIn> ld_frag_at(const TIn *base, int u) {
  if constexpr (sizeof(TIn) == 2) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(base + 32 * u);
    bf16x4 hi;
    if constexpr (HI) hi = *reinterpret_cast<const bf16x4 *>(base + 32 * u + 16);
    else hi = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return *reinterpret_cast<const f32x4 *>(base + 16 * u);
  }
}
template <typename TIn, bool HI>
__device__ __forceinline__ Frag<TIn> ld_frag_t_at(const TIn *base, int ld, int col0, int u) {
  if constexpr (sizeof(TIn) == 2) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const TIn *p = base + 32 * u * ld + col0;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
    i16x4 hi = {0, 0, 0, 0};
    if constexpr (HI) hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * ld));
    const bf16x4 l = __builtin_bit_cast(bf16x4, lo), h = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  } else {
    const TIn *p = base + 16 * u * ld + col0;
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
  }
}

// Score tiles in LDS (shared-score schedule): a 16 x 16 tile of A^T (rows j, columns i)
// is kept as its accumulator image, lane l = 16 g + li owning elements 4 l .. 4 l + 3 (rows
// 4g .. 4g+3 of column li), which is also where the P V operand fragment of that lane
// reads them; a wave's 64 lanes touch one contiguous 512-byte (bf16) block, free of bank
// conflicts.
template <typename TIn>
__device__ __forceinline__ void st_ptile(TIn *ltile, f32x4 x) { // ltile: + 4 (16 g + li)
  if constexpr (sizeof(TIn) == 2) {
    *reinterpret_cast<bf16x4 *>(ltile) = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  } else {
    *reinterpret_cast<f32x4 *>(ltile) = x;
  }
}
// B operand of O^T += V^T A^T for K unit (two 16-row tiles ta, tb; tb < 0: zeros);
// lbuf = score buffer + the lane's offset 4 (16 g + li).
template <typename TIn, int TA, int TB>
__device__ __forceinline__ Frag<TIn> ld_ptile(const TIn *lbuf) {
  if constexpr (sizeof(TIn) == 2) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(lbuf + TA * 256);
    bf16x4 hi = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    if constexpr (TB >= 0) hi = *reinterpret_cast<const bf16x4 *>(lbuf + TB * 256);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    static_assert(TB < 0, "fp32 K units are one tile");
    return *reinterpret_cast<const f32x4 *>(lbuf + TA * 256);
  }
}

// Output store of 4 adjacent values through a buffer resource: the hardware drops a
// store whose byte offset lies past the resource's range, which masks the rows past
// the end of a chunk and the columns past dv without a branch.
constexpr int kBufWord3 = 0x00020000; // gfx9 buffer resource: 32-bit data format
constexpr int kDropOffset = 0x7ff00000; // beyond any chunk's output range
// Keeps the vector-memory instructions on either side in program order (everything else
// may still move across).  The producers issue each chunk's loads in the order they are
// consumed; vmcnt retires loads in issue order, so a load the scheduler moved later would
// make the wait for an earlier one drain everything behind it.
__device__ __forceinline__ void vmem_order() { __builtin_amdgcn_sched_barrier(0x078F); }

// Buffer resource for [base, base + bytes).  Both must be uniform across the wave (they
// are: derived from the workgroup's unit and the chunk index); reading them through
// readfirstlane keeps them in scalar registers, where the compiler could otherwise wrap
// each load in a loop over the distinct values it cannot prove equal.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void *b = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, __builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}
// N (1, 2, 4 or 8) consecutive 32-bit words at byte offset off; zeros past the range.
template <int N>
__device__ __forceinline__ void ld_words_buf(uint32_t *w, __amdgpu_buffer_rsrc_t rs, int off) {
  if constexpr (N == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
  } else if constexpr (N == 2) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    w[0] = x[0]; w[1] = x[1];
  } else {
    static_assert(N % 4 == 0, "word count");
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * i, 0, 0);
      w[i] = x[0]; w[i + 1] = x[1]; w[i + 2] = x[2]; w[i + 3] = x[3];
    }
  }
}
// voff: the lane's byte offset; soff: the wave-uniform part (kDropOffset drops the store).
template <typename TIn>
__device__ __forceinline__ void st_out4_buf(__amdgpu_buffer_rsrc_t rs, int voff, int soff, f32x4 o) {
  if constexpr (sizeof(TIn) == 2) {
    const bf16x4 b = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), rs, voff, soff, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rs, voff, soff, 0);
  }
}

// Operand fragment from accumulator tiles (rows 4g+r of column li).
__device__ __forceinline__ bf16x8 acc_frag_bf(const f32x4 &t0, const f32x4 &t1) {
  return bf16x8{(__bf16)t0[0], (__bf16)t0[1], (__bf16)t0[2], (__bf16)t0[3],
                (__bf16)t1[0], (__bf16)t1[1], (__bf16)t1[2], (__bf16)t1[3]};
}

__device__ __forceinline__ f32x4 mma(f32x4 acc, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, f32x4 a, f32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  return acc;
}

// Scale the K-slots of a fragment by per-slot factors s[].
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 f, const float *s) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)((float)f[i] * s[i]);
  return r;
}
__device__ __forceinline__ f32x4 scale_frag(f32x4 f, const float *s) {
  return f32x4{f[0] * s[0], f[1] * s[1], f[2] * s[2], f[3] * s[3]};
}

template <typename TIn>
__device__ __forceinline__ Frag<TIn> frag_from(const float *s) {
  if constexpr (sizeof(TIn) == 2) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)s[i];
    return r;
  } else {
    return f32x4{s[0], s[1], s[2], s[3]};
  }
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (compile-time indices).
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Output store of 4 adjacent values (an O^T tile lane's rows 4g..4g+3).
template <typename TIn>
__device__ __forceinline__ void st_out4(TIn *p, f32x4 o) {
  if constexpr (sizeof(TIn) == 2) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
  } else {
    *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------------------------
// Producer: raw chunk data held in registers between its load and its preparation.

template <typename TIn, int DK, int C, int DECAY, bool NORM>
struct Staged {
  using K = Cfg<TIn, DK, C, DECAY, NORM>;
  static constexpr int QW = K::G * K::ES / 4; // words per row of q or k
  uint32_t q[K::RPT][QW], k[K::RPT][QW];
  uint32_t a[K::GATED ? K::RPT : 1][K::GS];
  uint32_t v[K::RPTV][2 * K::ES];             // 8 elements
};

// ---------------------------------------------------------------------------------
// The fused chunk kernel.

// SO: end states only (the first pass of the segment schedule; a.state_only is 1).
template <typename TIn, int DK, int C, int DECAY, bool NORM, bool SO, bool BTHD>
__global__ __launch_bounds__(kMaxThreads) void chunk_fwd_kernel(ChunkArgs a) {
  using K = Cfg<TIn, DK, C, DECAY, NORM>;
  using F = Frag<TIn>;
  using St = Staged<TIn, DK, C, DECAY, NORM>;
  static_assert(K::FITS, "tiles exceed LDS");
  // Producer rows in halves (token-major and packed layouts of the per-key gate at dk = 128):
  // wave p owns 64 key columns (64 (p % 2) ..) of 32 rows (32 (p / 2) ..), so that each
  // q/k load instruction reads whole 128-byte lines of rows H d elements apart; each half
  // scans its rows and the second half takes the first half's column products from LDS.
  // Measured on the load pattern alone (no arithmetic), token-major: 5.19 against 4.70 TB/s
  // for 32 columns of all 64 rows, whose instructions take half lines; in the forward pass
  // 0.82 against 0.99-1.04 ms (token-major) and 0.71 against 0.86-0.88 ms (packed), while
  // the head-major kernel ran 5% slower with it and keeps whole columns.
  constexpr int RH = (K::RH2 && BTHD) ? 2 : 1;
  constexpr int PW = DK * RH / 4;   // columns of one producer wave
  constexpr int LPR = PW / K::G;    // lanes sharing a row
  constexpr int CH = C / RH;        // rows of one producer wave
  constexpr int NRG = CH / K::RPT;  // row groups
  static_assert(NRG * LPR == K::PACTIVE && (CH >= 64 / LPR ? CH / (64 / LPR) : 1) == K::RPT,
                "row halves keep the lane count and the rows per lane");
  static_assert(RH == 1 || (K::PF == 1 && K::SHARE), "row halves: one prep between barriers");
  __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS];
  float *sPw = reinterpret_cast<float *>(smem + K::OFF_PW);

  // ---- which (b, h, segment, value slice): sibling slices share an XCD (id mod 8)
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vs = rest % a.nvs;
  const int unit = (rest / a.nvs) * 8 + xcd;
  if (unit >= a.nunits) return;
  const int seg = unit % a.nseg;
  int bh = unit / a.nseg;
  if (a.seq_order) bh = a.seq_order[bh / a.H] * a.H + bh % a.H; // longest sequences first
  const int h = bh % a.H;

  // wave index through readfirstlane: the compiler then keeps everything derived from it
  // (roles, value columns, tile masks) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool producer = wave >= K::NCW;
  constexpr bool state_only = SO;

  // Token addressing.  [B][H][T][d]: the unit's tokens are contiguous rows of d.
  // [B][T][H][d] / packed [total][H][d]: row t of head h of sequence b sits at token
  // s0 + t of the token-major array (s0 = b T, or cu_seqlens[b], clamped to the array),
  // so consecutive rows are H d elements apart.  Every element offset below is
  // base + t * RS + column.
  int64_t Tu = a.T, s0 = 0;
  if constexpr (BTHD) {
    const int b = bh / a.H;
    if (a.cu_seqlens) {
      s0 = a.cu_seqlens[b];
      int64_t e = a.cu_seqlens[b + 1];
      s0 = s0 < 0 ? 0 : (s0 > a.T ? a.T : s0);
      e = e < s0 ? s0 : (e > a.T ? a.T : e);
      Tu = e - s0;
    } else {
      s0 = (int64_t)b * a.T;
    }
  }
  const int RS_QK = BTHD ? a.H * DK : DK;          // row strides (elements)
  const int RS_V = BTHD ? a.H * a.dv : a.dv;
  const int RS_T = BTHD ? a.H : 1;                 // per-token decay
  const int64_t base_qk = BTHD ? (s0 * a.H + h) * DK : (int64_t)bh * a.T * DK;
  const int64_t base_v = BTHD ? (s0 * a.H + h) * a.dv : (int64_t)bh * a.T * a.dv;
  const int64_t base_t = BTHD ? s0 * a.H + h : (int64_t)bh * a.T;
  // byte range of L rows of d elements at row stride rs
  auto rows_bytes = [](int L, int rs, int d, int es) -> int {
    if constexpr (BTHD) return L > 0 ? ((L - 1) * rs + d) * es : 0;
    else return L * d * es;
  };

  const int64_t t_begin = (int64_t)seg * a.seg_len;
  int64_t t_end = t_begin + a.seg_len;
  if (t_end > Tu) t_end = Tu;
  const int nch = t_end > t_begin ? (int)((t_end - t_begin + C - 1) / C) : 0;

  if constexpr (DECAY == DECAY_GAMMA) {
    // gamma^n, n = 0..C, read by both roles
    if (tid <= C) {
      const float gm = a.decay[h];
      sPw[tid] = tid == 0 ? 1.f : exp2f((float)tid * log2f(gm));
    }
    __syncthreads();
  }

  // row-half hand-off of the gate products (RH = 2): hflag[cb] = 1 + the last chunk
  // whose first-half products sHalf[cb PW ..] hold; zero before the first chunk
  int *hflag = reinterpret_cast<int *>(smem + K::OFF_FLAG + 16);
  float *sHalf = reinterpret_cast<float *>(smem + K::OFF_FLAG + 32);
  if constexpr (RH == 2) {
    if (tid < 4) hflag[tid] = 0;
    __syncthreads();
  }

  if (producer) {
    // =========================== producer waves ===========================
    const int p = wave - K::NCW, ptid = tid - 64 * K::NCW;
    const int cgl = lane % LPR, rg = lane / LPR;
    const int cb = RH == 1 ? p : p % 2, rh = RH == 1 ? 0 : p / 2; // column block, row half
    const bool last_half = RH == 1 || rh == RH - 1;                 // holds the chunk's totals
    const int col0 = cb * PW + cgl * K::G;
    const int row0 = rh * CH + rg * K::RPT;
    const bool ld_on = lane < K::PACTIVE;
    const int vcg = ptid & 7, vrg = ptid >> 3;
    const int vrow0 = vrg * K::RPTV;
    const bool vld_on = ptid < K::VACTIVE && (vs * kSlice + 8 * vcg) < a.dv;
    float dprod[K::G];
#pragma unroll
    for (int c = 0; c < K::G; ++c) dprod[c] = 1.f;
    // gated kinds: set once a chunk's decay product (on this lane's key columns) falls below
    // kSafeDecay; published per wave in LDS (for the consumers' end-state write) and to
    // a.unsafe (for the exact kernel)
    bool unsafe = false;
    int *sFlag = reinterpret_cast<int *>(smem + K::OFF_FLAG);

    // Loads go through a buffer resource per chunk (range = the chunk's valid rows): rows
    // past the end of the sequence and idle lanes read zeros without a branch, so the
    // loads can be placed right where a row's registers fall free.
    // gate loads are issued separately so they can go out as soon as the scan has used
    // the previous chunk's gate registers; rows past L are set to 1 in prep
    // (0 past the last chunk: the prefetch of a chunk that does not exist loads nothing,
    // and staying unconditional keeps the loads' wait counts exact for the compiler)
    auto chunk_len = [&](int n) {
      const int64_t t0 = t_begin + (int64_t)n * C;
      const int64_t l = t_end - t0;
      return (int)(l < 0 ? 0 : (l < C ? l : C));
    };
    auto load_gate = [&](St &s, int n) {
      if constexpr (DECAY == DECAY_GATE) {
        const int64_t t0 = t_begin + (int64_t)n * C;
        const auto rs = make_rsrc(a.decay + base_qk + t0 * RS_QK, rows_bytes(chunk_len(n), RS_QK, DK, 4));
#pragma unroll
        for (int r = 0; r < K::RPT; ++r)
          ld_words_buf<K::G>(s.a[r], rs, ld_on ? ((row0 + r) * RS_QK + col0) * 4 : kDropOffset);
      } else if constexpr (DECAY == DECAY_TOKEN) {
        // one value per row ([B][H][T])
        const int64_t t0 = t_begin + (int64_t)n * C;
        const auto rs = make_rsrc(a.decay + base_t + t0 * RS_T, rows_bytes(chunk_len(n), RS_T, 1, 4));
#pragma unroll
        for (int r = 0; r < K::RPT; ++r)
          ld_words_buf<1>(s.a[r], rs, ld_on ? (row0 + r) * RS_T * 4 : kDropOffset);
      }
    };
    // q/k row r and v row r of chunk n
    auto load_q = [&](St &s, int n, int r) {
      const int64_t t0 = t_begin + (int64_t)n * C;
      const auto rq = make_rsrc(static_cast<const TIn *>(a.q) + base_qk + t0 * RS_QK,
                                state_only ? 0 : rows_bytes(chunk_len(n), RS_QK, DK, K::ES));
      ld_words_buf<St::QW>(s.q[r], rq, ld_on ? ((row0 + r) * RS_QK + col0) * K::ES : kDropOffset);
    };
    auto load_k = [&](St &s, int n, int r) {
      const int64_t t0 = t_begin + (int64_t)n * C;
      const auto rk = make_rsrc(static_cast<const TIn *>(a.k) + base_qk + t0 * RS_QK,
                                rows_bytes(chunk_len(n), RS_QK, DK, K::ES));
      ld_words_buf<St::QW>(s.k[r], rk, ld_on ? ((row0 + r) * RS_QK + col0) * K::ES : kDropOffset);
    };
    auto load_qk = [&](St &s, int n, int r) {
      load_q(s, n, r);
      load_k(s, n, r);
    };
    auto load_v = [&](St &s, int n, int r) {
      const int64_t t0 = t_begin + (int64_t)n * C;
      const auto rs = make_rsrc(static_cast<const TIn *>(a.v) + base_v + t0 * RS_V,
                                rows_bytes(chunk_len(n), RS_V, a.dv, K::ES));
      ld_words_buf<2 * K::ES>(s.v[r], rs, vld_on ? ((vrow0 + r) * RS_V + vs * kSlice + 8 * vcg) * K::ES : kDropOffset);
    };
    // same order as prep issues the next chunk's loads (v, gate, q/k rows): the loads
    // then retire in the order they are used
    auto load = [&](St &s, int n) {
#pragma unroll
      for (int r = 0; r < K::RPTV; ++r) load_v(s, n, r);
      vmem_order();
      load_gate(s, n);
      vmem_order();
#pragma unroll
      for (int r = 0; r < K::RPT; ++r) {
        if constexpr (K::Q_LATE) load_k(s, n, r);
        else load_qk(s, n, r);
      }
      vmem_order();
      if constexpr (K::Q_LATE) {
#pragma unroll
        for (int r = 0; r < K::RPT; ++r) load_q(s, n, r);
        vmem_order();
      }
    };

    // split schedule: Qt rows of the chunk being prepared wait here for the Qt tile
    uint32_t qkeep[K::SPLIT && !K::Q_LATE ? K::RPT : 1][St::QW];
    // (Q_LATE: s holds chunk n's q rows; they are replaced by chunk n + 1's as they go)
    auto store_q = [&](St &s, int n) {
      if constexpr (K::Q_LATE) {
        const int L = chunk_len(n);
        TIn *sQ = reinterpret_cast<TIn *>(smem + K::q_at(n));
        auto qrows = [&](auto elu_c) {
          constexpr bool ELU = decltype(elu_c)::value;
#pragma unroll
          for (int r = 0; r < K::RPT; ++r) {
            const int row = row0 + r;
            float qv[K::G];
            unpack<TIn, K::G>(qv, s.q[r]);
#pragma unroll
            for (int c = 0; c < K::G; ++c) {
              float qq = qv[c];
              if constexpr (ELU) qq = qq > 0.f ? qq + 1.f : __expf(qq);
              qv[c] = row < L ? qq : 0.f;
            }
            if (ld_on) st_lds<TIn, K::G>(sQ + row * K::LQ + col0, qv);
          }
        };
        if (a.phi_elu1) qrows(std::true_type{});
        else qrows(std::false_type{});
        // the next chunk's q rows, outside the branch so that their wait counts stay exact
#pragma unroll
        for (int r = 0; r < K::RPT; ++r) load_q(s, n + 1, r);
        vmem_order();
      } else if constexpr (K::SPLIT) {
        if (ld_on) {
          TIn *sQ = reinterpret_cast<TIn *>(smem + K::q_at(n));
#pragma unroll
          for (int r = 0; r < K::RPT; ++r) st_words_lds<St::QW>(sQ + (row0 + r) * K::LQ + col0, qkeep[r]);
        }
      }
    };

    // prepares chunk n (n may be one past the last chunk: L = 0, nothing loaded or read)
    auto prep = [&](St &s, int n) {
      const int L = chunk_len(n);
      TIn *sQ = reinterpret_cast<TIn *>(smem + K::q_at(n));
      TIn *sK = reinterpret_cast<TIn *>(smem + K::k_at(n));
      TIn *sV = reinterpret_cast<TIn *>(smem + K::v_at(n));
      float *sEL = reinterpret_cast<float *>(smem + K::el_at(n));
      // V rows are copied as they are; the next chunk's V goes out at once
      if (ptid < K::VACTIVE) {
#pragma unroll
        for (int r = 0; r < K::RPTV; ++r) {
          uint32_t *dst = reinterpret_cast<uint32_t *>(sV + (vrow0 + r) * K::LV + 8 * vcg);
#pragma unroll
          for (int i = 0; i < 2 * K::ES; i += 4)
            *reinterpret_cast<uint4 *>(dst + i) = make_uint4(s.v[r][i], s.v[r][i + 1], s.v[r][i + 2], s.v[r][i + 3]);
        }
      }
#pragma unroll
      for (int r = 0; r < K::RPTV; ++r) load_v(s, n + K::PF, r);
      vmem_order();
      // gate: b_i = local cumulative product over this lane's rows times the product of
      // the row groups above it (inclusive shuffle scan across lanes rg*LPR + cgl)
      // (token gate: one column, the same for every key)
      float bc[K::GATED ? K::RPT : 1][K::GS];
      if constexpr (K::GATED) {
        if (L < C) {
#pragma unroll
          for (int r = 0; r < K::RPT; ++r)
#pragma unroll
            for (int i = 0; i < K::GS; ++i)
              if (row0 + r >= L) s.a[r][i] = 0x3f800000u; // 1.0f: no decay past the end
        }
#pragma unroll
        for (int r = 0; r < K::RPT; ++r) {
          unpack<float, K::GS>(bc[r], s.a[r]);
          if (r > 0) {
#pragma unroll
            for (int c = 0; c < K::GS; ++c) bc[r][c] *= bc[r - 1][c];
          }
        }
        float inc[K::GS];
#pragma unroll
        for (int c = 0; c < K::GS; ++c) inc[c] = bc[K::RPT - 1][c];
#pragma unroll
        for (int d = 1; d < NRG; d *= 2) {
          const int src = (lane - d * LPR) < 0 ? 0 : 4 * (lane - d * LPR);
#pragma unroll
          for (int c = 0; c < K::GS; ++c) {
            const float o = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(inc[c])));
            inc[c] = rg >= d ? inc[c] * o : inc[c];
          }
        }
        const int src_last = 4 * ((NRG - 1) * LPR + cgl);
        const int src_prev = (lane - LPR) < 0 ? 0 : 4 * (lane - LPR);
        float tot[K::GS];
#pragma unroll
        for (int c = 0; c < K::GS; ++c) {
          tot[c] = __int_as_float(__builtin_amdgcn_ds_bpermute(src_last, __float_as_int(inc[c])));
          const float pv = __int_as_float(__builtin_amdgcn_ds_bpermute(src_prev, __float_as_int(inc[c])));
          const float ex = rg == 0 ? 1.f : pv;
#pragma unroll
          for (int r = 0; r < K::RPT; ++r) bc[r][c] *= ex;
          if constexpr (RH == 1) {
            dprod[c] *= tot[c];
            unsafe = unsafe || (ld_on && !(tot[c] >= kSafeDecay)); // (a NaN gate counts as unsafe)
          }
        }
        if constexpr (RH == 2) {
          if (rh == 0) {
            // publish this half's column products, then the chunk index (release: the
            // compiler waits for the LDS writes before the flag store)
            if (rg == 0) st_lds<float, K::G>(sHalf + col0, tot);
            if (lane == 0)
              __hip_atomic_store(&hflag[cb], n + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          } else {
            // the first-half wave of this column block publishes before it reaches the
            // chunk's barrier and waits for nothing of this wave, so the wait ends
            while (__hip_atomic_load(&hflag[cb], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <= n)
              __builtin_amdgcn_s_sleep(1);
            const f32x4 h0 = *reinterpret_cast<const f32x4 *>(sHalf + col0);
            const f32x4 h1 = *reinterpret_cast<const f32x4 *>(sHalf + col0 + 4);
#pragma unroll
            for (int c = 0; c < K::G; ++c) {
              const float f = c < 4 ? h0[c] : h1[c - 4];
              tot[c] *= f;
#pragma unroll
              for (int r = 0; r < K::RPT; ++r) bc[r][c] *= f;
            }
          }
          if (last_half) {
#pragma unroll
            for (int c = 0; c < K::GS; ++c) {
              dprod[c] *= tot[c];
              unsafe = unsafe || (ld_on && !(tot[c] >= kSafeDecay));
            }
          }
        }
        // (the ballot outside the lane-0 branch: inside it only lane 0 would vote)
        const int wave_unsafe = __builtin_amdgcn_ballot_w64(unsafe) != 0 ? 1 : 0;
        if (lane == 0) sFlag[p] = wave_unsafe;
        if (ld_on && rg == 0 && last_half) {
          float totg[K::G];
#pragma unroll
          for (int c = 0; c < K::G; ++c) totg[c] = tot[K::GS == 1 ? 0 : c];
          st_lds<float, K::G>(sEL + col0, totg);
        }
        load_gate(s, n + K::PF);
        vmem_order();
      } else if constexpr (DECAY == DECAY_GAMMA) {
        dprod[0] *= sPw[L];
      }
      // feature map (compile-time choice), decay factors, bf16/fp32 tiles -> LDS
      auto rows = [&](auto elu_c, auto full_c) {
        constexpr bool ELU = decltype(elu_c)::value, FULL = decltype(full_c)::value;
#pragma unroll
        for (int r = 0; r < K::RPT; ++r) {
          const int row = row0 + r;
          float qv[K::G], kv[K::G];
          unpack<TIn, K::G>(kv, s.k[r]);
          if constexpr (!K::Q_LATE) unpack<TIn, K::G>(qv, s.q[r]);
          else {
#pragma unroll
            for (int c = 0; c < K::G; ++c) qv[c] = 0.f; // formed later from s.q
          }
#pragma unroll
          for (int c = 0; c < K::G; ++c) {
            float kk = kv[c], qq = qv[c];
            if constexpr (ELU) {
              kk = kk > 0.f ? kk + 1.f : __expf(kk);
              qq = qq > 0.f ? qq + 1.f : __expf(qq);
            }
            if constexpr (!FULL) {
              kk = row < L ? kk : 0.f;
              qq = row < L ? qq : 0.f;
            }
            if constexpr (K::GATED) {
              // 1 / b formed here, row by row, so no second array of reciprocals stays live
              qq *= bc[r][K::GS == 1 ? 0 : c];
              kk *= rcp_f(bc[r][K::GS == 1 ? 0 : c]);
            }
            kv[c] = kk;
            qv[c] = qq;
          }
          st_lds<TIn, K::G>(sK + row * K::LQ + col0, kv);
          if constexpr (K::Q_LATE) {
          } else if constexpr (K::SPLIT) pack_words<TIn, K::G>(qkeep[r], qv);
          else if (!state_only) st_lds<TIn, K::G>(sQ + row * K::LQ + col0, qv);
          if constexpr (!K::SPLIT) {
            load_qk(s, n + K::PF, r); // this row's registers are free
            vmem_order();
          }
        }
      };
      if (ld_on) {
        using T_ = std::true_type;
        using F_ = std::false_type;
        if (a.phi_elu1) {
          if (L == C) rows(T_{}, T_{});
          else rows(T_{}, F_{});
        } else {
          if (L == C) rows(F_{}, T_{});
          else rows(F_{}, F_{});
        }
      }
      // Split schedule: the next chunk's q/k rows after the branches above (inside them,
      // the compiler's wait counts for these loads turn conservative across that loop's
      // two barriers; the one-barrier loops keep exact counts with the loads per row).
      if constexpr (K::SPLIT) {
#pragma unroll
        for (int r = 0; r < K::RPT; ++r) {
          if constexpr (K::Q_LATE) load_k(s, n + K::PF, r);
          else load_qk(s, n + K::PF, r);
        }
        vmem_order();
      }
    };

    if constexpr (K::SPLIT) {
      // barriers: A_n (chunk n in place) and B_n (phase 1 of chunk n done) for every chunk
      St s0;
      if (nch > 0) {
        load(s0, 0);
        prep(s0, 0);
        store_q(s0, 0);
      }
      for (int n = 0; n < nch; ++n) {
        __syncthreads(); // A_n
        prep(s0, n + 1); // Kt, V of chunk n + 1 into the stage chunk n - 1 used
        __syncthreads(); // B_n: Qt of chunk n read
        store_q(s0, n + 1);
      }
    } else if constexpr (K::PF == 2) {
      St s0, s1;
      if (nch > 0) load(s0, 0);
      if (nch > 1) load(s1, 1);
      static_assert(K::STAGES >= 2, "two chunks ahead needs two stages");
      for (int n = 0; n < nch; n += 2) {
        prep(s0, n);
        __syncthreads();
        // unconditional: past the last chunk it loads nothing and fills a stage no consumer
        // reads (keeps the loads' wait counts exact); only the barrier follows the chunks
        prep(s1, n + 1);
        if (n + 1 < nch) __syncthreads();
      }
    } else {
      St s0;
      if (nch > 0) load(s0, 0);
      for (int n = 0; n < nch; ++n) {
        prep(s0, n);
        __syncthreads();
        if constexpr (K::STAGES == 1) __syncthreads();
      }
    }
    // shared-score schedule: consumers finish the last chunk one barrier later
    if constexpr (K::SHARE) {
      if (nch > 0) __syncthreads();
    }
    if (a.seg_decay && vs == 0 && ld_on && rg == 0 && last_half) {
      float *sd = a.seg_decay + ((int64_t)bh * a.nseg + seg) * DK + col0;
#pragma unroll
      for (int c = 0; c < K::G; ++c) sd[c] = (DECAY == DECAY_GATE) ? dprod[c] : dprod[0];
    }
    if constexpr (K::GATED) {
      const bool any = __builtin_amdgcn_ballot_w64(unsafe) != 0;
      if (a.unsafe && vs == 0 && lane == 0) a.unsafe[((int64_t)bh * a.nseg + seg) * 4 + p] = any ? 1 : 0;
    }
    return;
  }

  // =========================== consumer waves ===========================
  const int g = lane >> 4, li = lane & 15;
  const int e0 = vs * kSlice + 16 * K::ET * wave; // first value column of this wave
  bool tile_on[K::ET];
#pragma unroll
  for (int t = 0; t < K::ET; ++t) tile_on[t] = e0 + 16 * t < a.dv;
  const bool wave_on = tile_on[0];
  TIn *gout = static_cast<TIn *>(a.out) + base_v;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  f32x4 Hs[K::ET][K::NCB];
  f32x4 Zs[NORM ? K::NCB : 1];
  {
    const float *ini = a.init ? a.init + (int64_t)bh * a.init_bh_stride + (int64_t)seg * a.init_seg_stride
                              : nullptr;
#pragma unroll
    for (int cb = 0; cb < K::NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = K::state_row(cb, g, r);
#pragma unroll
        for (int t = 0; t < K::ET; ++t) {
          const int e = e0 + 16 * t + li;
          Hs[t][cb][r] = (ini && e < a.dv) ? ini[(int64_t)c * a.ncol + e] : 0.f;
        }
        if constexpr (NORM) Zs[cb][r] = ini ? ini[(int64_t)c * a.ncol + a.dv] : 0.f;
      }
    }
  }

  if constexpr (K::SHARE || K::SPLIT) {
    // ---------------- consumer waves, score tiles shared through LDS ----------------
    const int cw = wave;
    // score tiles of this wave: tile k = s * NCW + cw of slot s; a slot past the last tile
    // computes tile 0 into the discard tile
    int sib[K::SLOTS], sjb[K::SLOTS], sdst[K::SLOTS];
    const int dl = li - 4 * g;
    // Gamma powers in the loop.  Split schedule: no table reads; each power is a lane part
    // gamma^0..31 (vector registers) times gamma^{16k} (uniform: scalar registers).
    // Shared-score schedule (which runs at the register limit, where the compiler's schedule
    // measured best this way): mask factors in registers, V' factors and row scales from the
    // power table.
    auto uni = [](float x) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
    };
    constexpr bool GM = DECAY == DECAY_GAMMA;
    constexpr bool GF = GM && K::SPLIT;
    float g16[GF ? K::NB + 1 : 1];  // gamma^{16k}, k = 0..NB (gamma^C = g16[NB])
    float vpl[4], fdiag[4], foff[4], lrow = 1.f;
    float smul[K::SLOTS];
    bool sdiag[K::SLOTS];
    float fac[GM && !GF ? K::SLOTS : 1][4]; // gamma^{i-j} (0 above the diagonal) per element
    if constexpr (GF) {
#pragma unroll
      for (int k = 0; k <= K::NB; ++k) g16[k] = uni(sPw[16 * k]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) vpl[qq] = sPw[15 - 4 * g - qq]; // V' lane part
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = dl - r; // i - j inside a diagonal tile
        fdiag[r] = d >= 0 ? sPw[d] : 0.f;
        foff[r] = K::NB >= 2 ? sPw[16 + d] : 0.f; // off-diagonal: times gamma^{16 (ib - jb - 1)}
      }
      lrow = sPw[li + 1];
    }
#pragma unroll
    for (int s = 0; s < K::SLOTS; ++s) {
      const int k = s * K::NCW + cw;
      const int kk = k < K::NTILES ? k : 0;
      int ib = 0;
      while ((ib + 1) * (ib + 2) / 2 <= kk) ++ib;
      sib[s] = ib;
      sjb[s] = kk - ib * (ib + 1) / 2;
      sdst[s] = k < K::NTILES ? k : K::NTILES;
      sdiag[s] = sib[s] == sjb[s];
      smul[s] = 0.f;
      if constexpr (GF) smul[s] = uni(sdiag[s] ? 0.f : sPw[16 * (sib[s] - sjb[s] - 1)]);
      if constexpr (GM && !GF) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int dij = 16 * (sib[s] - sjb[s]) + dl - r;
          fac[s][r] = dij >= 0 ? sPw[dij] : 0.f;
        }
      }
    }

    // this wave's masked score tiles of chunk n -> its score buffer
    // Lane parts of the LDS addresses (elements).  Every access is tile base (uniform) +
    // lane part + a compile-time offset; for the score slots the uniform part is formed per
    // chunk in scalar registers and kept opaque, so that the compiler holds no per-slot
    // vector registers through the loop.
    const int lc = li * K::LQ + (K::BF ? 8 : 4) * g;                  // contiguous rows
    const int ls = li * K::LQ + 4 * g;                                // split-convention rows
    const int lkt = K::BF ? (4 * g + (li >> 2)) * K::LQ + (K::PERM ? 8 : 4) * (li & 3)
                          : 4 * g * K::LQ + li;                       // Kt^T
    const int lvt = K::BF ? (4 * g + (li >> 2)) * K::LV + 4 * (li & 3)
                          : 4 * g * K::LV + li;                       // V^T
    const int lp = (16 * g + li) * 4;                                   // score tiles
    const int lel = K::PERM ? 8 * g : 4 * g;                          // eL
    auto scores = [&](int n) {
#pragma unroll
      for (int s = 0; s < K::SLOTS; ++s) {
        const int qo = __builtin_amdgcn_readfirstlane(K::q_at(n) + 16 * sib[s] * K::LQ * K::ES);
        const int ko = __builtin_amdgcn_readfirstlane(K::k_at(n) + 16 * sjb[s] * K::LQ * K::ES);
        const int po = __builtin_amdgcn_readfirstlane(K::p_at(n) + sdst[s] * K::PTILE * K::ES);
        const TIn *qrow = reinterpret_cast<const TIn *>(smem + qo) + lc;
        const TIn *krow = reinterpret_cast<const TIn *>(smem + ko) + lc;
        TIn *ptile = reinterpret_cast<TIn *>(smem + po) + lp;
        f32x4 x = zero4;
#pragma unroll
        for (int u = 0; u < K::NU_DK; ++u)
          x = mma(x, ld_frag_c_at<TIn, K::HI_DK>(krow, u, g), ld_frag_c_at<TIn, K::HI_DK>(qrow, u, g));
        // element (j = 16 jb + 4g + r, i = 16 ib + li): keep i >= j (gamma: times gamma^{i-j})
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (GF) {
            x[r] *= sdiag[s] ? fdiag[r] : smul[s] * foff[r];
          } else if constexpr (GM) {
            x[r] *= fac[s][r];
          } else {
            const int dij = 16 * (sib[s] - sjb[s]) + dl - r;
            x[r] = dij >= 0 ? x[r] : 0.f;
          }
        }
        st_ptile<TIn>(ptile, x);
      }
    };

    // Row-block-pair variant (K::PAIRS): wave W computes tiles (B, jb), jb <= B, and
    // (A, jb), jb <= A, with A = W, B = NB - 1 - W; each Kt block is read once for both.
    auto scores_pair = [&](int n, auto W_c) {
      constexpr int A = decltype(W_c)::value, B = K::NB - 1 - A;
      const TIn *sQ = reinterpret_cast<const TIn *>(smem + K::q_at(n)) + lc;
      const TIn *sK = reinterpret_cast<const TIn *>(smem + K::k_at(n)) + lc;
      TIn *pb = reinterpret_cast<TIn *>(smem + K::p_at(n)) + lp;
      // row block B's fragments stay in registers; A's (at most NB / 2 tiles) are re-read
      F qb[K::NU_DK];
#pragma unroll
      for (int u = 0; u < K::NU_DK; ++u) qb[u] = ld_frag_c_at<TIn, K::HI_DK>(sQ + 16 * B * K::LQ, u, g);
      auto tile = [&](const F *qf, const F *kf, auto IB, auto JB) {
        constexpr int ib = decltype(IB)::value, jb = decltype(JB)::value;
        f32x4 x = zero4;
#pragma unroll
        for (int u = 0; u < K::NU_DK; ++u) x = mma(x, kf[u], qf[u]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (ib == jb) {
            if constexpr (GF) x[r] *= fdiag[r];
            else if constexpr (GM) x[r] = dl - r >= 0 ? x[r] * sPw[dl - r < 0 ? 0 : dl - r] : 0.f;
            else x[r] = dl - r >= 0 ? x[r] : 0.f;
          } else if constexpr (GF) {
            // (x * a) * b: a precomputed product would be a loop invariant per (ib - jb, r)
            x[r] = (x[r] * g16[ib - jb - 1]) * foff[r];
          } else if constexpr (GM) {
            x[r] *= sPw[16 * (ib - jb) + dl - r];
          }
        }
        st_ptile<TIn>(pb + (ib * (ib + 1) / 2 + jb) * K::PTILE, x);
      };
      static_for<0, B + 1>([&](auto JB) {
        constexpr int jb = decltype(JB)::value;
        F kf[K::NU_DK];
#pragma unroll
        for (int u = 0; u < K::NU_DK; ++u) kf[u] = ld_frag_c_at<TIn, K::HI_DK>(sK + 16 * jb * K::LQ, u, g);
        tile(qb, kf, std::integral_constant<int, B>{}, JB);
        if constexpr (jb <= A) {
          F qa[K::NU_DK];
#pragma unroll
          for (int u = 0; u < K::NU_DK; ++u) qa[u] = ld_frag_c_at<TIn, K::HI_DK>(sQ + 16 * A * K::LQ, u, g);
          tile(qa, kf, std::integral_constant<int, A>{}, JB);
        }
      });
    };
    auto scores_any = [&](int n) {
      if constexpr (K::PAIRS) {
        static_assert(K::NCW == 2 || K::NCW == 4, "pairs");
        switch (cw) {
        case 0: scores_pair(n, std::integral_constant<int, 0>{}); break;
        case 1: scores_pair(n, std::integral_constant<int, 1>{}); break;
        case 2: if constexpr (K::NCW == 4) scores_pair(n, std::integral_constant<int, 2>{}); break;
        default: if constexpr (K::NCW == 4) scores_pair(n, std::integral_constant<int, 3>{}); break;
        }
      } else {
        scores(n);
      }
    };

    // V^T operand fragments of chunk m (rows e, K = tokens j; columns past dv hold zeros)
    // and the state-update operands (gamma: V' = diag(gamma^{L-1-j}) V; z: the all-ones
    // or decay column)
    F vf[K::ET][K::NU_C], vu[K::ET][K::NU_C], wz[NORM ? K::NU_C : 1];
    auto v_operands = [&](const TIn *sV) {
      const TIn *vb = sV + lvt + 16 * K::ET * wave;
#pragma unroll
      for (int t = 0; t < K::ET; ++t)
#pragma unroll
        for (int u = 0; u < K::NU_C; ++u)
          vf[t][u] = ld_frag_t_at<TIn, K::HI_C>(vb, K::LV, 16 * t, u);
    };
    // (formed right before the state update: the scaling need not wait for vf earlier)
    auto update_operands = [&](int L, auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int u = 0; u < K::NU_C; ++u) {
        if constexpr (DECAY == DECAY_GAMMA) {
          float sc[8];
#pragma unroll
          for (int q = 0; q < (K::BF ? 8 : 4); ++q) {
            const int j = K::BF ? (32 * u + (q < 4 ? 0 : 16) + 4 * g + (q & 3)) : (16 * u + 4 * g + q);
            if constexpr (FULL && GF) {
              // gamma^{C-1-j} = gamma^{15-4g-(q%4)} gamma^{16k}
              const int kq = K::BF ? C / 16 - 1 - 2 * u - (q >> 2) : C / 16 - 1 - u;
              sc[q] = kq >= 0 ? vpl[q & 3] * g16[kq < 0 ? 0 : kq] : 0.f;
            } else if constexpr (FULL) {
              sc[q] = sPw[C - 1 - j];
            } else {
              sc[q] = j < L ? sPw[L - 1 - j] : 0.f;
            }
          }
#pragma unroll
          for (int t = 0; t < K::ET; ++t) vu[t][u] = scale_frag(vf[t][u], sc);
          if constexpr (NORM) wz[u] = frag_from<TIn>(sc);
        } else {
#pragma unroll
          for (int t = 0; t < K::ET; ++t) vu[t][u] = vf[t][u];
          if constexpr (NORM) {
            const float one[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
            wz[u] = frag_from<TIn>(one);
          }
        }
      }
    };

    // the state before a chunk as operands of the inter-chunk term
    F hf[K::ET][K::NU_DK], zf[NORM ? K::NU_DK : 1];
    auto state_operands = [&]() {
#pragma unroll
      for (int u = 0; u < K::NU_DK; ++u) {
        if constexpr (K::BF) {
#pragma unroll
          for (int t = 0; t < K::ET; ++t) {
            if constexpr (K::HI_DK) hf[t][u] = acc_frag_bf(Hs[t][2 * u], Hs[t][2 * u + 1]);
            else hf[t][u] = acc_frag_bf(Hs[t][0], zero4);
          }
          if constexpr (NORM) {
            if constexpr (K::HI_DK) zf[u] = acc_frag_bf(Zs[2 * u], Zs[2 * u + 1]);
            else zf[u] = acc_frag_bf(Zs[0], zero4);
          }
        } else {
#pragma unroll
          for (int t = 0; t < K::ET; ++t) hf[t][u] = Hs[t][u];
          if constexpr (NORM) zf[u] = Zs[u];
        }
      }
    };

    // Qt operand fragments of row block ib (the order matching hf)
    auto q_operands = [&](F *qc, const TIn *sQ, int ib) {
#pragma unroll
      for (int u = 0; u < K::NU_DK; ++u) {
        if constexpr (K::PERM) qc[u] = ld_frag_c_at<TIn, true>(sQ + lc + 16 * ib * K::LQ, u, g);
        else qc[u] = ld_frag_at<TIn, K::HI_DK>(sQ + ls + 16 * ib * K::LQ, u);
      }
    };

    // O^T += V^T A^T for row block IB from the score buffer pb
    auto intra = [&](f32x4 *acc, f32x4 &accd, const TIn *pb, auto IB) {
      constexpr int ib = decltype(IB)::value;
#pragma unroll
      for (int t = 0; t < K::ET; ++t) acc[t] = zero4;
      accd = zero4;
      static_for<0, K::NU_C>([&](auto JU) {
        constexpr int ju = decltype(JU)::value;
        constexpr int jb = ju * K::TPU;
        if constexpr (jb <= ib) {
          constexpr int ta = ib * (ib + 1) / 2 + jb;
          constexpr int tb = (K::TPU == 2 && jb + 1 <= ib) ? ta + 1 : -1;
          const F pf = ld_ptile<TIn, ta, tb>(pb + lp);
#pragma unroll
          for (int t = 0; t < K::ET; ++t) acc[t] = mma(acc[t], vf[t][ju], pf);
          if constexpr (NORM) {
            const float one[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
            accd = mma(accd, frag_from<TIn>(one), pf);
          }
        }
      });
    };

    // S4 + S5 for chunk m: H <- decay (H + Kt^T V) (gamma: gamma^L H + Kt^T V')
    auto state_update = [&](const TIn *sK, const float *sEL, float gl) {
      static_for<0, K::NCB>([&](auto CB) {
        constexpr int cb = decltype(CB)::value;
        if constexpr (DECAY == DECAY_GAMMA) {
#pragma unroll
          for (int t = 0; t < K::ET; ++t) Hs[t][cb] *= gl;
          if constexpr (NORM) Zs[cb] *= gl;
        }
        constexpr int kcol = K::PERM ? 32 * (cb >> 1) + 4 * (cb & 1) : 16 * cb;
#pragma unroll
        for (int u = 0; u < K::NU_C; ++u) {
          const F kf = ld_frag_t_at<TIn, K::HI_C>(sK + lkt, K::LQ, kcol, u);
#pragma unroll
          for (int t = 0; t < K::ET; ++t) Hs[t][cb] = mma(Hs[t][cb], kf, vu[t][u]);
          if constexpr (NORM) Zs[cb] = mma(Zs[cb], kf, wz[u]);
        }
        if constexpr (K::GATED) {
          const float4 el = *reinterpret_cast<const float4 *>(sEL + lel + K::state_row(cb, 0, 0));
#pragma unroll
          for (int t = 0; t < K::ET; ++t) {
            Hs[t][cb][0] *= el.x; Hs[t][cb][1] *= el.y; Hs[t][cb][2] *= el.z; Hs[t][cb][3] *= el.w;
          }
          if constexpr (NORM) {
            Zs[cb][0] *= el.x; Zs[cb][1] *= el.y; Zs[cb][2] *= el.z; Zs[cb][3] *= el.w;
          }
        }
      });
    };

    // output rows of chunk m: stores past row L or column dv fall outside the range
    auto out_rsrc = [&](int64_t t0, int L) {
      return make_rsrc(gout + t0 * RS_V, state_only ? 0 : rows_bytes(L, RS_V, a.dv, K::ES));
    };
    // lane part of an output offset in a vector register, the row block and tile part
    // (uniform) in the scalar offset
    const int out_lane = (li * RS_V + 4 * g) * K::ES;
    auto store_out = [&](__amdgpu_buffer_rsrc_t ors, int ib, int t, f32x4 o) {
      const int soff = __builtin_amdgcn_readfirstlane(
          tile_on[t] ? (16 * ib * RS_V + e0 + 16 * t) * K::ES : kDropOffset);
      st_out4_buf<TIn>(ors, out_lane, soff, o);
    };

    // end states only (first pass of the segment schedule): the state update of every
    // chunk, with the same barriers as the producers
    auto state_only_loop = [&]() {
      for (int n = 0; n < nch; ++n) {
        const int64_t t0 = t_begin + (int64_t)n * C;
        const int L = (int)((t_end - t0) < C ? (t_end - t0) : C);
        __syncthreads();
        v_operands(reinterpret_cast<const TIn *>(smem + K::v_at(n)));
        update_operands(L, std::false_type{});
        state_update(reinterpret_cast<const TIn *>(smem + K::k_at(n)),
                     reinterpret_cast<const float *>(smem + K::el_at(n)),
                     (DECAY == DECAY_GAMMA) ? sPw[L] : 1.f);
        if constexpr (K::SPLIT) __syncthreads();
      }
      if constexpr (K::SHARE) {
        if (nch > 0) __syncthreads();
      }
    };

    if constexpr (SO) {
      state_only_loop();
    } else if constexpr (K::SHARE) {
      // Iteration n computes this wave's score tiles of chunk n (stage n % 3) into score
      // buffer n % 2, and the outputs and state update of chunk n - 1, whose tiles every
      // consumer wave finished before this iteration's barrier.  mid() runs between the
      // outputs and the state update (the next chunk's score tiles, scheduled with it).
      auto rest = [&](int m, auto full_c, auto &&mid) {
        constexpr bool FULL = decltype(full_c)::value;
        const int64_t t0 = t_begin + (int64_t)m * C;
        const int L = FULL ? C : (int)((t_end - t0) < C ? (t_end - t0) : C);
        const TIn *sQ = reinterpret_cast<const TIn *>(smem + K::q_at(m));
        const TIn *pb = reinterpret_cast<const TIn *>(smem + K::p_at(m));
        v_operands(reinterpret_cast<const TIn *>(smem + K::v_at(m)));
        const float gl = GM ? (FULL ? sPw[C] : sPw[L]) : 1.f;
        state_operands();
        const auto ors = out_rsrc(t0, L);
        static_for<0, K::NB>([&](auto IB) {
          constexpr int ib = decltype(IB)::value;
          // one row block's operands at a time (hoisting them all exceeds the registers)
          if constexpr (K::FENCE & 1) __builtin_amdgcn_sched_barrier(0);
          F qc[K::NU_DK];
          q_operands(qc, sQ, ib);
          f32x4 acc[K::ET], accd;
          intra(acc, accd, pb, IB);
          // inter-chunk: O^T += H^T Qt^T
          float rsc = 1.f;
          if constexpr (GM) rsc = sPw[16 * ib + li + 1];
          float inv = 1.f;
          if constexpr (NORM) {
            f32x4 accd2 = zero4;
#pragma unroll
            for (int u = 0; u < K::NU_DK; ++u) accd2 = mma(accd2, zf[u], qc[u]);
            if constexpr (DECAY == DECAY_GAMMA) accd2 *= rsc;
            accd += accd2;
            inv = rcp_f(accd[0]); // every row of the ones tile holds the denominator
          }
#pragma unroll
          for (int t = 0; t < K::ET; ++t) {
            f32x4 acc2 = zero4;
#pragma unroll
            for (int u = 0; u < K::NU_DK; ++u) acc2 = mma(acc2, hf[t][u], qc[u]);
            if constexpr (DECAY == DECAY_GAMMA) acc2 *= rsc;
            f32x4 o = acc[t] + acc2;
            if constexpr (NORM) o *= inv;
            store_out(ors, ib, t, o);
          }
        });
        mid();
        update_operands(L, full_c);
        state_update(reinterpret_cast<const TIn *>(smem + K::k_at(m)),
                     reinterpret_cast<const float *>(smem + K::el_at(m)), gl);
      };

      if (nch > 0) {
        __syncthreads(); // stage 0 holds chunk 0
        scores_any(0);
        for (int n = 1; n < nch; ++n) {
          __syncthreads(); // stage n % 3 holds chunk n; score tiles of chunk n - 1 complete
          rest(n - 1, std::true_type{}, [&] {
            if constexpr (K::FENCE & 2) __builtin_amdgcn_sched_barrier(0);
            scores_any(n);
          });
        }
        __syncthreads();
        rest(nch - 1, std::false_type{}, [] {});
      }
    } else {
      // Split schedule, two barriers a chunk.  Phase 1: the inter-chunk term of every row
      // block from the state before the chunk, and this wave's score tiles.  Phase 2:
      // O += A V, the outputs, the state update.
      for (int n = 0; n < nch; ++n) {
        const int64_t t0 = t_begin + (int64_t)n * C;
        const int L = (int)((t_end - t0) < C ? (t_end - t0) : C);
        const TIn *sQ = reinterpret_cast<const TIn *>(smem + K::q_at(n));
        const TIn *pb = reinterpret_cast<const TIn *>(smem + K::p_at(n));
        __syncthreads(); // Qt, Kt, V of chunk n in place
        // score tiles first: the inter-chunk results below then live only from there to
        // phase 2, not through the score tiles
        scores_any(n);
        state_operands();
        f32x4 inter[K::NB][K::ET];
        f32x4 dinter[NORM ? K::NB : 1];
        static_for<0, K::NB>([&](auto IB) {
          constexpr int ib = decltype(IB)::value;
          F qc[K::NU_DK];
          q_operands(qc, sQ, ib);
          float rsc = 1.f;
          if constexpr (GM) rsc = g16[ib] * lrow; // gamma^{16 ib + li + 1}
#pragma unroll
          for (int t = 0; t < K::ET; ++t) {
            f32x4 x = zero4;
#pragma unroll
            for (int u = 0; u < K::NU_DK; ++u) x = mma(x, hf[t][u], qc[u]);
            if constexpr (DECAY == DECAY_GAMMA) x *= rsc;
            inter[ib][t] = x;
          }
          if constexpr (NORM) {
            f32x4 x = zero4;
#pragma unroll
            for (int u = 0; u < K::NU_DK; ++u) x = mma(x, zf[u], qc[u]);
            if constexpr (DECAY == DECAY_GAMMA) x *= rsc;
            dinter[ib] = x;
          }
        });
        __syncthreads(); // score tiles complete; Qt free for the next chunk
        v_operands(reinterpret_cast<const TIn *>(smem + K::v_at(n)));
        const float gl = GM ? (L == C ? g16[K::NB] : sPw[L]) : 1.f;
        const auto ors = out_rsrc(t0, L);
        static_for<0, K::NB>([&](auto IB) {
          constexpr int ib = decltype(IB)::value;
          if constexpr (K::FENCE & 1) __builtin_amdgcn_sched_barrier(0);
          f32x4 acc[K::ET], accd;
          intra(acc, accd, pb, IB);
          float inv = 1.f;
          if constexpr (NORM) {
            accd += dinter[ib];
            inv = rcp_f(accd[0]);
          }
#pragma unroll
          for (int t = 0; t < K::ET; ++t) {
            f32x4 o = acc[t] + inter[ib][t];
            if constexpr (NORM) o *= inv;
            store_out(ors, ib, t, o);
          }
        });
        if (L == C) update_operands(L, std::true_type{});
        else update_operands(L, std::false_type{});
        state_update(reinterpret_cast<const TIn *>(smem + K::k_at(n)),
                     reinterpret_cast<const float *>(smem + K::el_at(n)), gl);
      }
    }
  } else {
  for (int n = 0; n < nch; ++n) {
    __syncthreads(); // stage n % STAGES holds chunk n
    const int64_t t0 = t_begin + (int64_t)n * C;
    const int L = (int)((t_end - t0) < C ? (t_end - t0) : C);
    const unsigned char *base = smem + (n % K::STAGES) * K::STAGE_BYTES;
    const TIn *sQ = reinterpret_cast<const TIn *>(base + K::OFF_Q);
    const TIn *sK = reinterpret_cast<const TIn *>(base + K::OFF_K);
    const TIn *sV = reinterpret_cast<const TIn *>(base + K::OFF_V);
    const float *sEL = reinterpret_cast<const float *>(base + K::OFF_EL);

    if (wave_on) {
      // V^T operand fragments (rows e, K = tokens); tiles past dv hold zeros
      F vf[K::ET][K::NU_C];
#pragma unroll
      for (int t = 0; t < K::ET; ++t)
#pragma unroll
        for (int u = 0; u < K::NU_C; ++u)
          vf[t][u] = ld_frag_t<TIn, K::HI_C>(sV, K::LV, 16 * (K::ET * wave + t), u, g, li);

      // operands of the state update: V (gamma: V' = diag(gamma^{L-1-j}) V) and, for z,
      // the all-ones (gamma: decay) column
      F vu[K::ET][K::NU_C], wz[NORM ? K::NU_C : 1];
#pragma unroll
      for (int u = 0; u < K::NU_C; ++u) {
        if constexpr (DECAY == DECAY_GAMMA) {
          float sc[8];
#pragma unroll
          for (int q = 0; q < (K::BF ? 8 : 4); ++q) {
            const int j = K::BF ? (32 * u + (q < 4 ? 0 : 16) + 4 * g + (q & 3)) : (16 * u + 4 * g + q);
            sc[q] = j < L ? sPw[L - 1 - j] : 0.f;
          }
#pragma unroll
          for (int t = 0; t < K::ET; ++t) vu[t][u] = scale_frag(vf[t][u], sc);
          if constexpr (NORM) wz[u] = frag_from<TIn>(sc);
        } else {
#pragma unroll
          for (int t = 0; t < K::ET; ++t) vu[t][u] = vf[t][u];
          if constexpr (NORM) {
            const float one[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
            wz[u] = frag_from<TIn>(one);
          }
        }
      }
      const float gl = (DECAY == DECAY_GAMMA) ? sPw[L] : 1.f;

      // S4 + S5 for state row block cb: H <- decay (H + Kt^T V) (gamma: gamma^L H + Kt^T V')
      auto state_block = [&](const int cb) {
        if constexpr (DECAY == DECAY_GAMMA) {
#pragma unroll
          for (int t = 0; t < K::ET; ++t) Hs[t][cb] *= gl;
          if constexpr (NORM) Zs[cb] *= gl;
        }
#pragma unroll
        for (int u = 0; u < K::NU_C; ++u) {
          const F kf = ld_frag_t<TIn, K::HI_C>(sK, K::LQ, 16 * cb, u, g, li);
#pragma unroll
          for (int t = 0; t < K::ET; ++t) Hs[t][cb] = mma(Hs[t][cb], kf, vu[t][u]);
          if constexpr (NORM) Zs[cb] = mma(Zs[cb], kf, wz[u]);
        }
        if constexpr (K::GATED) {
          const float4 el = *reinterpret_cast<const float4 *>(sEL + 16 * cb + 4 * g);
#pragma unroll
          for (int t = 0; t < K::ET; ++t) {
            Hs[t][cb][0] *= el.x; Hs[t][cb][1] *= el.y; Hs[t][cb][2] *= el.z; Hs[t][cb][3] *= el.w;
          }
          if constexpr (NORM) {
            Zs[cb][0] *= el.x; Zs[cb][1] *= el.y; Zs[cb][2] *= el.z; Zs[cb][3] *= el.w;
          }
        }
      };

      // operand copies of the state before this chunk (for the inter-chunk term)
      F hf[K::ET][K::NU_DK], zf[NORM ? K::NU_DK : 1];
      if (!state_only) {
#pragma unroll
        for (int u = 0; u < K::NU_DK; ++u) {
          if constexpr (K::BF) {
#pragma unroll
            for (int t = 0; t < K::ET; ++t) {
              if constexpr (K::HI_DK) hf[t][u] = acc_frag_bf(Hs[t][2 * u], Hs[t][2 * u + 1]);
              else hf[t][u] = acc_frag_bf(Hs[t][0], zero4);
            }
            if constexpr (NORM) {
              if constexpr (K::HI_DK) zf[u] = acc_frag_bf(Zs[2 * u], Zs[2 * u + 1]);
              else zf[u] = acc_frag_bf(Zs[0], zero4);
            }
          } else {
#pragma unroll
            for (int t = 0; t < K::ET; ++t) hf[t][u] = Hs[t][u];
            if constexpr (NORM) zf[u] = Zs[u];
          }
        }
      }

      // ---------------- S3 + S6 for row block ib (outputs of this chunk)
      F kc[K::KCACHE ? K::NB : 1][K::NU_DK]; // Kt fragments of row blocks seen so far
      auto row_block = [&](const int ib) {
        const TIn *qrow = sQ + (16 * ib + li) * K::LQ;
        // qf: split K convention (pairs with the state operand); qc: contiguous convention
        // (pairs with Kt in the score tiles)
        F qf[K::NU_DK], qc[K::NU_DK];
#pragma unroll
        for (int u = 0; u < K::NU_DK; ++u) {
          qf[u] = ld_frag<TIn, K::HI_DK>(qrow, u, g);
          if constexpr (K::BF) qc[u] = ld_frag_c<TIn, K::HI_DK>(qrow, u, g);
          else qc[u] = qf[u];
        }
        if constexpr (K::KCACHE) {
          const TIn *krow = sK + (16 * ib + li) * K::LQ;
#pragma unroll
          for (int u = 0; u < K::NU_DK; ++u) kc[ib][u] = ld_frag_c<TIn, K::HI_DK>(krow, u, g);
        }

        f32x4 acc[K::ET];
#pragma unroll
        for (int t = 0; t < K::ET; ++t) acc[t] = zero4;
        f32x4 accd = zero4;
        // intra-chunk: A^T tiles (rows j, cols i) for j-blocks <= ib
#pragma unroll
        for (int ju = 0; ju < K::NU_C; ++ju) {
          if (ju * K::TPU > ib) break;
          f32x4 st[K::TPU];
#pragma unroll
          for (int s = 0; s < K::TPU; ++s) {
            const int jb = ju * K::TPU + s;
            f32x4 x = zero4;
            if (jb <= ib) {
              const TIn *krow = sK + (16 * jb + li) * K::LQ;
#pragma unroll
              for (int u = 0; u < K::NU_DK; ++u) {
                F kfr;
                if constexpr (K::KCACHE) kfr = kc[jb][u];
                else kfr = ld_frag_c<TIn, K::HI_DK>(krow, u, g);
                x = mma(x, kfr, qc[u]);
              }
              // element (j = 16 jb + 4g + r, i = 16 ib + li)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int dij = 16 * (ib - jb) + li - 4 * g - r; // i - j
                if constexpr (DECAY == DECAY_GAMMA) {
                  x[r] = dij >= 0 ? x[r] * sPw[dij] : 0.f;
                } else {
                  if (dij < 0) x[r] = 0.f;
                }
              }
            }
            st[s] = x;
          }
          F af;
          if constexpr (K::BF) af = acc_frag_bf(st[0], st[1]);
          else af = st[0];
#pragma unroll
          for (int t = 0; t < K::ET; ++t) acc[t] = mma(acc[t], vf[t][ju], af);
          if constexpr (NORM) {
            const float one[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
            accd = mma(accd, frag_from<TIn>(one), af);
          }
        }
        // inter-chunk: H^T Qt^T
        float rsc = 1.f;
        if constexpr (DECAY == DECAY_GAMMA) rsc = sPw[16 * ib + li + 1];
        float inv = 1.f;
        if constexpr (NORM) {
          f32x4 accd2 = zero4;
#pragma unroll
          for (int u = 0; u < K::NU_DK; ++u) accd2 = mma(accd2, zf[u], qf[u]);
          if constexpr (DECAY == DECAY_GAMMA) accd2 *= rsc;
          accd += accd2;
          inv = rcp_f(accd[0]); // every row of the ones tile holds the denominator
        }
        const int i = 16 * ib + li;
#pragma unroll
        for (int t = 0; t < K::ET; ++t) {
          f32x4 acc2 = zero4;
#pragma unroll
          for (int u = 0; u < K::NU_DK; ++u) acc2 = mma(acc2, hf[t][u], qf[u]);
          if constexpr (DECAY == DECAY_GAMMA) acc2 *= rsc;
          f32x4 o = acc[t] + acc2;
          if constexpr (NORM) o *= inv;
          if (i < L && tile_on[t]) st_out4<TIn>(gout + (t0 + i) * RS_V + e0 + 16 * t + 4 * g, o);
        }
      };

      if (!state_only) {
        if constexpr (K::KCACHE) {
#pragma unroll
          for (int ib = 0; ib < K::NB; ++ib) {
            if (16 * ib >= L) break;
            row_block(ib);
          }
        } else {
          // not unrolled: keeps the compiler from hoisting every row block's operand loads
#pragma unroll 1
          for (int ib = 0; ib < K::NB; ++ib) {
            if (16 * ib >= L) break;
            row_block(ib);
          }
        }
      }
      // compile-time block indices: a runtime index into the accumulator array would
      // move it to scratch memory
      static_for<0, K::NCB>([&](auto CB) { state_block(decltype(CB)::value); });
    }
    if constexpr (K::STAGES == 1) __syncthreads(); // stage free for the next chunk
  }
  }

  // ---- end state (not written for a unit the exact kernel recomputes: with an in-place
  // resume its start state must survive)
  bool unsafe_unit = false;
  if constexpr (K::GATED) {
    if (nch > 0) {
      const int *sFlag = reinterpret_cast<const int *>(smem + K::OFF_FLAG);
      unsafe_unit = (sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3]) != 0;
    }
  }
  if (a.fin && wave_on && !unsafe_unit) {
    float *fo = a.fin + (int64_t)bh * a.fin_bh_stride + (int64_t)seg * a.fin_seg_stride;
#pragma unroll
    for (int cb = 0; cb < K::NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = K::state_row(cb, g, r);
#pragma unroll
        for (int t = 0; t < K::ET; ++t) {
          const int e = e0 + 16 * t + li;
          if (e < a.dv) fo[(int64_t)c * a.ncol + e] = Hs[t][cb][r];
        }
        if constexpr (NORM) {
          if (vs == 0 && wave == 0 && li == 0) fo[(int64_t)c * a.ncol + a.dv] = Zs[cb][r];
        }
      }
    }
  }
}

} // namespace fla
