// Chunkwise causal linear attention, backward — gfx950 kernels.
//
// Reverse-mode derivative of the recurrence h_t = diag(g_t) h_{t-1} + phi(k_t) v_t^T,
// o_t = h_t^T phi(q_t) (h = S^T, dk x dv; the decayed linear attention of the textbook
// chapter 1.6 "linear attention" section with the RetNet / GLA decays of the FLA posts),
// for the loss L = sum dout . o + sum dfinal (.) h_T.  Per chunk of C rows with b the
// inclusive product of the decays inside the chunk, bL = b[L-1], Qb = phi(q) b,
// Kb = phi(k) / b, and H (dH) the state (its gradient) at the chunk's start (end):
//   dphi(q) = b (.) ( tril(dO V^T) Kb + dO H^T ),         H  <- diag(bL) (H + Kb^T V)
//   dv      = triu(Kb Qb^T) dO + Kb diag(bL) dH,           dH <- diag(bL) dH + Qb^T dO
//   dphi(k) = (1/b) (.) ( triu(V dO^T) Qb + V (diag(bL) dH)^T )
// (triu: query rows at or after the key row).  The gate's gradient follows from
// d log b_t = phi(q_t) dphi(q_t) - phi(k_t) dphi(k_t) summed over later tokens, plus the
// final state's term sum_e dfinal (.) h_T; d alpha = d log alpha / alpha.
//
// All three are one scan pattern, "role" R:
//   out[r][x] = post[r][x] * ( sum_{s ~ r} (X_r . Y_s) Z[s][x] + sum_y X[r][y] S[y][x] ),
//   S (fp32, [DY][64] per workgroup, in MFMA accumulators) updated with Y^T Z per chunk,
// with  DQ: X = dO, Y = V, Z = Kb, S = H^T, forward in time, post = b;
//       DK: X = V, Y = dO, Z = Qb, S = dH^T, reverse, post = 1/b;
//       DV: X = Kb, Y = Qb, Z = dO, S = dH,  reverse, post = 1.
// One workgroup owns one (b, h, 64-wide slice of the output dimension).  An operand group
// of 4 waves scans the decay down each chunk and forms the chunk's operand tiles in LDS
// from registers loaded ahead; an output group of 4 waves computes the C x C score tiles
// once (shared through LDS), then wave w forms the output tiles of columns 16w..16w+15,
// updates its state columns and (dk role) sums the decay gradient in registers.  Where two
// operand stages fit in LDS the groups are separate waves working one chunk apart (two
// barriers per chunk); otherwise one group of 4 waves does both in turn (four barriers).
// MFMA conventions are the forward kernel's.
#pragma once

#include "chunk_fwd.hpp"

namespace fla {

enum : int { BWD_DQ = 0, BWD_DK = 1, BWD_DV = 2 };

struct BwdArgs {
  const void *q, *k, *v, *dout;
  const float *decay;  // gamma [H], gate (laid out like q), per-token decay (one per token
                       // and head, [B][H][T] or token-major [tokens][H]), or null
  const float *init;   // [B][H][dk][dv] or null (read by DQ)
  const float *dfinal; // [B][H][dk][dv] or null (read by DV, DK, and DQ for its term)
  void *grad_q, *grad_k, *grad_v; // outputs in the input dtype
  float *dgate;        // gate: laid out like the gate (written by DK) or null
  float *dinit;        // [B][H][dk][dv] (written by DV) or null
  float *rq;           // workspace laid out like q: phi(q) dphi(q) (DQ writes, DK reads) or null
  float *fterm;        // workspace [B][H][dk]: sum_e dfinal h_T (DQ writes, DK reads) or null
  float *tpart;        // workspace [H][nsl][4][ntok]: d log a_t per slice and wave (token) or null
  int64_t T;           // tokens per sequence (packed: the total)
  int64_t ntok;        // tokens over all sequences (B T, or the packed total)
  int bthd;            // 1: q, k, v, dout, gate and their gradients token-major [B][T][H][d]
                       //    (packed [total][H][d] with cu_seqlens); 0: [B][H][T][d]
  const int64_t *cu_seqlens; // packed sequences: [B + 1] token offsets (bthd only), or null
  int H, dk, dv;
  int nsl;             // 64-wide slices of the output dimension
  int nunits;          // B * H * nsl
  int phi_elu1;
  int want_dg;         // DQ: write rq (and fterm with dfinal); DK: write the decay gradient
};

template <typename TIn, int ROLE, int DY, int DECAY>
struct BwdCfg {
  static constexpr int C = 64, XW = 64;
  static constexpr int NTG = 256;                // threads of one wave group (4 waves)
  static constexpr int ES = sizeof(TIn);
  static constexpr int VE = 16 / ES;             // elements per 16-byte vector
  static constexpr int KU = ES == 2 ? 32 : 16;   // MFMA K unit
  static constexpr int LDX = DY + VE;            // X, Y row stride (elements)
  static constexpr int LDZ = XW + VE;            // Z row stride
  static constexpr bool REV = ROLE != BWD_DQ;
  static constexpr bool HAS_B = DECAY != DECAY_NONE;
  static constexpr bool GATE = DECAY == DECAY_GATE;
  static constexpr bool TOKEN = DECAY == DECAY_TOKEN;
  static constexpr bool GAMMA = DECAY == DECAY_GAMMA;
  // b tile columns: per-key gate over the decayed dimension, else one column
  static constexpr int GW = GATE ? (ROLE == BWD_DV ? DY : XW) : 1;
  static constexpr bool HAS_AUX = ROLE != BWD_DV; // phi(q) (DQ) / phi(k) (DK) read per lane
  static constexpr bool HAS_RQ = ROLE == BWD_DK && (GATE || TOKEN);
  // bf16 dq / dk roles carry the rounded MFMA operands as hi + lo pairs (scores, Z, state)
  // so their outputs, and the decay gradient summed from them over the sequence, keep
  // close to fp32 accuracy; the dv role rounds once, like the forward pass
  static constexpr bool SPLIT = ES == 2 && ROLE != BWD_DV;
  // register prefetch: 16-byte vectors per thread of the operand group
  static constexpr int NVX = C * DY / VE / NTG;
  static constexpr int NVZ = C * XW / VE / NTG;
  static_assert(NVX >= 1 && NVZ >= 1, "tile too small for the thread count");
  // gate scan: NSEG row segments of SEGR rows; a thread scans GC adjacent columns of one
  // segment (two for the dv role's gate of 128 columns or more, so its segments stay short)
  static constexpr int GC = (GATE && ROLE == BWD_DV && GW >= 128) ? 2 : 1;
  static constexpr int NSEG = GATE ? NTG * GC / GW : 1;
  static constexpr int SEGR = C / NSEG;
  static_assert(!GATE || ROLE == BWD_DV || SEGR == 16, "dq / dk read segment prefixes per row block");
  // a wave's 16-byte vectors of a decayed tile cover 64 / (row vectors) consecutive rows,
  // starting at a multiple of that count: they lie in one gate segment
  static constexpr int DEC_VPR = (ROLE == BWD_DV ? DY : XW) / VE;
  static_assert(!GATE || (DEC_VPR <= 64 && SEGR % (64 / DEC_VPR) == 0), "segment uniform per wave");
  // b as the output tiles read it (dq, dk): gate local products [C][GW] with the segment
  // prefixes [NSEG][GW]; per-token decay: b [C]
  static constexpr bool B_OUT = (GATE && ROLE != BWD_DV) || TOKEN;
  static constexpr int B_BYTES = (GATE && ROLE != BWD_DV) ? C * GW * 4 : TOKEN ? C * 4 : 0;
  static constexpr int PRE_BYTES = (GATE && ROLE != BWD_DV) ? NSEG * GW * 4 : 0;
  static constexpr int BL_BYTES = GATE ? GW * 4 : TOKEN ? 16 : 0;
  // one stage of chunk operands (bytes)
  static constexpr int ST_X = 0;
  static constexpr int ST_Y = ST_X + C * LDX * ES;
  static constexpr int ST_Z = ST_Y + C * LDX * ES;
  static constexpr int ST_ZL = ST_Z + C * LDZ * ES;                 // Z lo (SPLIT)
  static constexpr int ST_B = ST_ZL + (SPLIT ? C * LDZ * ES : 0);
  static constexpr int ST_PRE = ST_B + B_BYTES;
  static constexpr int ST_BL = ST_PRE + PRE_BYTES;                  // chunk decay bL
  static constexpr int STAGE = (ST_BL + BL_BYTES + 15) / 16 * 16;
  // shared by the stages: score tiles, the dv role's gate products (gamma: its powers), the
  // gate's segment totals
  static constexpr int SH_P = 0;
  static constexpr int SH_PL = SH_P + 16 * 256 * ES;                 // score lo (SPLIT)
  static constexpr int SH_BS = SH_PL + (SPLIT ? 16 * 256 * ES : 0);
  static constexpr int SH_TOT = SH_BS + ((GATE && ROLE == BWD_DV) ? C * GW * 4 : GAMMA ? C * 4 : 0);
  static constexpr int SHARED = SH_TOT + (GATE ? NSEG * GW * 4 : 0);
  // two stages fit: a producer wave group forms chunk n + 1 while the consumer group works
  // on chunk n; else one group does both in turn
  static constexpr bool PC = 2 * STAGE + SHARED <= kMaxLds;
  static constexpr int NST = PC ? 2 : 1;
  static constexpr int NT = NST * NTG;
  static constexpr int OFF_SH = NST * STAGE;
  static constexpr int LDS = OFF_SH + SHARED;
  static constexpr bool FITS = LDS <= kMaxLds;
};


// fp32 values rounded to bf16 and back (the hi part of a hi + lo split)
__device__ __forceinline__ f32x4 bf_round4(f32x4 x) {
  return f32x4{(float)(__bf16)x[0], (float)(__bf16)x[1], (float)(__bf16)x[2], (float)(__bf16)x[3]};
}

// phi as a compile-time choice; elu + 1 without a branch: max(x, 0) + e^min(x, 0)
template <bool ELU>
__device__ __forceinline__ float phi_c(float x) {
  if constexpr (ELU) return fmaxf(x, 0.f) + __expf(fminf(x, 0.f));
  else return x;
}

__device__ __forceinline__ float phi_d(float phi_val, int elu1) {
  // derivative of phi in terms of phi(x): identity -> 1; elu+1 -> 1 (x > 0, phi > 1)
  // or e^x = phi(x) (x <= 0)
  return elu1 ? fminf(phi_val, 1.f) : 1.f;
}

// Score-tile operand (A, row r = li, K = s) for K unit u of row block RB: tiles TA, TB of
// the row-major 16x16 score images (negative = zeros).  bf16: two tiles per unit.
template <typename TIn, int TA, int TB>
__device__ __forceinline__ Frag<TIn> ld_ptile2(const TIn *lbuf) {
  if constexpr (sizeof(TIn) == 2) {
    const __bf16 z = (__bf16)0.f;
    bf16x4 lo = {z, z, z, z}, hi = {z, z, z, z};
    if constexpr (TA >= 0) lo = *reinterpret_cast<const bf16x4 *>(lbuf + TA * 256);
    if constexpr (TB >= 0) hi = *reinterpret_cast<const bf16x4 *>(lbuf + TB * 256);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    static_assert(TB < 0, "fp32 K units are one tile");
    if constexpr (TA >= 0) return *reinterpret_cast<const f32x4 *>(lbuf + TA * 256);
    else return f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Allowed score tiles (row block rb of the output rows r, column block sb of the summed
// rows s): s <= r (forward roles) or s >= r (reverse roles).
template <bool REV>
__host__ __device__ constexpr bool tile_on(int rb, int sb) { return REV ? sb >= rb : sb <= rb; }
template <bool REV>
__host__ __device__ constexpr int tile_pos(int rb, int sb) { // index among the allowed tiles
  int n = 0;
  for (int i = 0; i < 16; ++i) {
    if (i == rb * 4 + sb) return n;
    if (tile_on<REV>(i / 4, i % 4)) ++n;
  }
  return -1;
}


// The value of lane li + D of the same 16-lane row (DPP row shift), 0 past the row's end.
template <int D>
__device__ __forceinline__ float from_row_next(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + D, 0xf, 0xf, true));
}

// Suffix sums over the 64 rows r = 16 rb + li of a chunk held as v[rb] by the 16 lanes of
// lane group g: on return v[rb] = sum over rows r' >= r; returns the sum of all 64 rows.
__device__ __forceinline__ float suffix_rows64(float (&v)[4], int g) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    v[rb] += from_row_next<1>(v[rb]);
    v[rb] += from_row_next<2>(v[rb]);
    v[rb] += from_row_next<4>(v[rb]);
    v[rb] += from_row_next<8>(v[rb]);
  }
  float t[4]; // row block totals (lane li = 0 of the group)
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) t[rb] = __shfl(v[rb], 16 * g);
  v[2] += t[3];
  v[1] += t[2] + t[3];
  v[0] += t[1] + t[2] + t[3];
  return t[0] + t[1] + t[2] + t[3];
}

template <typename TIn, int ROLE, int DY, int DECAY>
__global__ void __launch_bounds__((BwdCfg<TIn, ROLE, DY, DECAY>::NT)) chunk_bwd_kernel(BwdArgs a) {
  using K = BwdCfg<TIn, ROLE, DY, DECAY>;
  constexpr int C = K::C, XW = K::XW, VE = K::VE, KU = K::KU;
  constexpr int LDX = K::LDX, LDZ = K::LDZ, GW = K::GW;
  constexpr bool REV = K::REV;
  constexpr int NYB = DY / 16;         // 16-row blocks of the state
  constexpr int NZU = C / KU;          // K units over the chunk rows
  __shared__ __attribute__((aligned(16))) unsigned char lds[K::LDS];
  auto stX = [&](int s) { return reinterpret_cast<TIn *>(lds + s * K::STAGE + K::ST_X); };
  auto stY = [&](int s) { return reinterpret_cast<TIn *>(lds + s * K::STAGE + K::ST_Y); };
  auto stZ = [&](int s) { return reinterpret_cast<TIn *>(lds + s * K::STAGE + K::ST_Z); };
  auto stZL = [&](int s) { return reinterpret_cast<TIn *>(lds + s * K::STAGE + K::ST_ZL); };
  auto stB = [&](int s) { return reinterpret_cast<float *>(lds + s * K::STAGE + K::ST_B); };
  auto stPre = [&](int s) { return reinterpret_cast<float *>(lds + s * K::STAGE + K::ST_PRE); };
  auto stBL = [&](int s) { return reinterpret_cast<float *>(lds + s * K::STAGE + K::ST_BL); };
  TIn *sP = reinterpret_cast<TIn *>(lds + K::OFF_SH + K::SH_P);
  TIn *sPL = reinterpret_cast<TIn *>(lds + K::OFF_SH + K::SH_PL);
  float *sBS = reinterpret_cast<float *>(lds + K::OFF_SH + K::SH_BS);
  float *sTot = reinterpret_cast<float *>(lds + K::OFF_SH + K::SH_TOT);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, li = lane & 15;

  // unit -> (b h, slice); sibling slices of one head on the same XCD (ids = mod 8)
  int unit = blockIdx.x;
  if ((a.nunits & 7) == 0) unit = (unit & 7) * (a.nunits >> 3) + (unit >> 3);
  const int slice = unit % a.nsl;
  const int64_t bh = unit / a.nsl;
  const int h = (int)(bh % a.H);
  const int dk = a.dk, dv = a.dv;

  // Token addressing.  [B][H][T][d]: the unit's rows are contiguous rows of d.  [B][T][H][d]
  // / packed [total][H][d]: row t of this head of sequence b is token tok0 + t of the
  // token-major array (tok0 = b T, or cu_seqlens[b] clamped to the array), rows H d apart.
  const int64_t b = bh / a.H;
  int64_t T = a.T, tok0 = b * a.T;
  if (a.cu_seqlens) {
    int64_t s = a.cu_seqlens[b], e = a.cu_seqlens[b + 1];
    s = s < 0 ? 0 : (s > a.T ? a.T : s);
    e = e < s ? s : (e > a.T ? a.T : e);
    tok0 = s;
    T = e - s;
  }
  const int64_t rsK = a.bthd ? (int64_t)a.H * dk : dk;  // rows of q, k, dq, dk, the gate
  const int64_t rsV = a.bthd ? (int64_t)a.H * dv : dv;  // rows of v, dout, dv
  const int64_t rsT = a.bthd ? a.H : 1;                 // per-token decay
  const int64_t baseK = a.bthd ? (tok0 * a.H + h) * dk : bh * a.T * dk;
  const int64_t baseV = a.bthd ? (tok0 * a.H + h) * dv : bh * a.T * dv;
  const int64_t baseT = a.bthd ? tok0 * a.H + h : bh * a.T;
  const int nchunks = (int)((T + C - 1) / C);
  const int elu1 = a.phi_elu1;
  const bool want_dg = a.want_dg != 0;

  // sources: X, Y rows of DY elements; Z and AUX 64-column slices; row strides rsXY, rsZ
  const TIn *srcX, *srcY, *srcZ, *srcA = nullptr;
  int64_t rsXY, rsZ;
  if constexpr (ROLE == BWD_DQ) {
    srcX = (const TIn *)a.dout + baseV; srcY = (const TIn *)a.v + baseV;
    srcZ = (const TIn *)a.k + baseK; srcA = (const TIn *)a.q + baseK;
    rsXY = rsV; rsZ = rsK;
  } else if constexpr (ROLE == BWD_DK) {
    srcX = (const TIn *)a.v + baseV; srcY = (const TIn *)a.dout + baseV;
    srcZ = (const TIn *)a.q + baseK; srcA = (const TIn *)a.k + baseK;
    rsXY = rsV; rsZ = rsK;
  } else {
    srcX = (const TIn *)a.k + baseK; srcY = (const TIn *)a.q + baseK;
    srcZ = (const TIn *)a.dout + baseV;
    rsXY = rsK; rsZ = rsV;
  }
  const int zoff = slice * XW;                      // first output column
  const int goff = (ROLE == BWD_DV) ? 0 : zoff;     // first gate column

  auto chunk_len = [&](int n) -> int {
    const int64_t l = T - (int64_t)n * C;
    return (int)(l < C ? l : C);
  };
  auto chunk_at = [&](int it) -> int { return REV ? nchunks - 1 - it : it; };

  // ---- gamma: b[r] = gamma^(r+1) for the whole kernel -----------------------------
  if constexpr (K::GAMMA) {
    if (wave == 0) {
      float x = a.decay[h];
      for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(x, d);
        if (lane >= d) x *= o;
      }
      sBS[lane] = x;
    }
  }

  // =========================== operand group ===========================================
  // Forms the operand tiles of a chunk in a stage: phase 1 scans the decay down the chunk
  // and copies the tiles that need no decay; phase 2 (after a barrier) completes the scan
  // with the segment prefixes and forms the decayed tiles.  Registers hold the next
  // chunk's inputs, loaded as the current ones fall free.
  const int ptid = K::PC ? tid - K::NTG : tid;
  const int pwave = K::PC ? wave - 4 : wave;
  uint32_t rX[K::NVX][4], rY[K::NVX][4], rZ[K::NVZ][4];
  float rG[K::GATE ? K::SEGR : 1][K::GC]; // gate rows of this thread's (columns, segment) in scan order
  float rTok = 1.f;
  auto ld_xy = [&](int n) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;
    constexpr int VPRX = DY / VE;
#pragma unroll
    for (int j = 0; j < K::NVX; ++j) {
      const int vi = ptid + K::NTG * j, r = vi / VPRX, c = (vi % VPRX) * VE;
      // rows past the end read the last row and are masked where the tiles are formed
      // (a select here would make the compiler wait for the load)
      const int rc = r < L ? r : L - 1;
      const uint4 x = *reinterpret_cast<const uint4 *>(srcX + (t0 + rc) * rsXY + c);
      const uint4 y = *reinterpret_cast<const uint4 *>(srcY + (t0 + rc) * rsXY + c);
      rX[j][0] = x.x; rX[j][1] = x.y; rX[j][2] = x.z; rX[j][3] = x.w;
      rY[j][0] = y.x; rY[j][1] = y.y; rY[j][2] = y.z; rY[j][3] = y.w;
    }
  };
  auto ld_z = [&](int n) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;
    constexpr int VPRZ = XW / VE;
#pragma unroll
    for (int j = 0; j < K::NVZ; ++j) {
      const int vi = ptid + K::NTG * j, r = vi / VPRZ, c = (vi % VPRZ) * VE;
      const int rc = r < L ? r : L - 1;
      const uint4 z = *reinterpret_cast<const uint4 *>(srcZ + (t0 + rc) * rsZ + zoff + c);
      rZ[j][0] = z.x; rZ[j][1] = z.y; rZ[j][2] = z.z; rZ[j][3] = z.w;
    }
  };
  auto ld_g = [&](int n) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;
    if constexpr (K::GATE) {
      // thread (columns GC (ptid % (GW / GC)) + 0 .. GC - 1, segment ptid / (GW / GC)) reads
      // its SEGR rows: for each row the lanes of a wave read consecutive columns
      constexpr int NCOL = GW / K::GC;
      const float *gsrc = a.decay + baseK + goff + K::GC * (ptid % NCOL);
      const int r0 = (ptid / NCOL) * K::SEGR;
#pragma unroll
      for (int i = 0; i < K::SEGR; ++i) {
        const float *src = gsrc + (t0 + (r0 + i < L ? r0 + i : L - 1)) * rsK;
        if constexpr (K::GC == 2) {
          const float2 v = *reinterpret_cast<const float2 *>(src);
          rG[i][0] = v.x;
          rG[i][1] = v.y;
        } else {
          rG[i][0] = *src;
        }
      }
    }
    if constexpr (K::TOKEN) {
      if (pwave == 0) rTok = a.decay[baseT + (t0 + (ptid < L ? ptid : L - 1)) * rsT];
    }
  };
  // phase-1 inputs: the decay and the tiles copied unconverted; phase-2: the decayed tiles
  auto load1 = [&](int n) {
    ld_g(n);
    if constexpr (ROLE == BWD_DV) ld_z(n);
    else ld_xy(n);
  };
  auto load2 = [&](int n) {
    if constexpr (ROLE == BWD_DV) ld_xy(n);
    else ld_z(n);
  };

  auto phase1 = [&](int n, int s) {
    const int L = chunk_len(n);
    if constexpr (K::GATE) {
      // local products down this thread's segment, and the segment's total; rows past the
      // end carry no decay
      constexpr int NCOL = GW / K::GC;
      const int col = K::GC * (ptid % NCOL), seg = ptid / NCOL;
      float *loc = (ROLE == BWD_DV) ? sBS : stB(s);
      float p[K::GC];
#pragma unroll
      for (int c = 0; c < K::GC; ++c) p[c] = 1.f;
#pragma unroll
      for (int i = 0; i < K::SEGR; ++i) {
        const bool in = seg * K::SEGR + i < L;
#pragma unroll
        for (int c = 0; c < K::GC; ++c) p[c] *= in ? rG[i][c] : 1.f;
        float *dst = loc + (seg * K::SEGR + i) * GW + col;
        if constexpr (K::GC == 2) *reinterpret_cast<float2 *>(dst) = make_float2(p[0], p[1]);
        else *dst = p[0];
      }
#pragma unroll
      for (int c = 0; c < K::GC; ++c) sTot[seg * GW + col + c] = p[c];
    } else if constexpr (K::TOKEN) {
      if (pwave == 0) {
        float x = lane < L ? rTok : 1.f;
        for (int d = 1; d < 64; d <<= 1) {
          const float o = __shfl_up(x, d);
          if (lane >= d) x *= o;
        }
        stB(s)[lane] = x;
        if (lane == 63) stBL(s)[0] = x; // padded rows carry 1: b[63] = b[L-1]
      }
    }
    if constexpr (ROLE == BWD_DV) {
      constexpr int VPRZ = XW / VE;
#pragma unroll
      for (int j = 0; j < K::NVZ; ++j) {
        const int vi = ptid + K::NTG * j, r = vi / VPRZ, c = (vi % VPRZ) * VE;
        const uint32_t m = r < L ? ~0u : 0u; // rows past the end: zeros
        const uint32_t w[4] = {rZ[j][0] & m, rZ[j][1] & m, rZ[j][2] & m, rZ[j][3] & m};
        st_words_lds<4>(stZ(s) + r * LDZ + c, w);
      }
    } else {
      constexpr int VPRX = DY / VE;
#pragma unroll
      for (int j = 0; j < K::NVX; ++j) {
        const int vi = ptid + K::NTG * j, r = vi / VPRX, c = (vi % VPRX) * VE;
        const uint32_t m = r < L ? ~0u : 0u; // rows past the end: zeros
        const uint32_t wx[4] = {rX[j][0] & m, rX[j][1] & m, rX[j][2] & m, rX[j][3] & m};
        const uint32_t wy[4] = {rY[j][0] & m, rY[j][1] & m, rY[j][2] & m, rY[j][3] & m};
        st_words_lds<4>(stX(s) + r * LDX + c, wx);
        st_words_lds<4>(stY(s) + r * LDX + c, wy);
      }
    }
  };

  auto phase2 = [&](int n, int s) {
    const int L = chunk_len(n);
    if constexpr (K::GATE) {
      // prefix of the earlier segments; the chunk decay bL from the last segment
      constexpr int NCOL = GW / K::GC;
      const int col0 = K::GC * (ptid % NCOL), seg = ptid / NCOL;
#pragma unroll
      for (int c = 0; c < K::GC; ++c) {
        const int col = col0 + c;
        float pre = 1.f;
        for (int s2 = 0; s2 < seg; ++s2) pre *= sTot[s2 * GW + col];
        if constexpr (ROLE != BWD_DV) stPre(s)[seg * GW + col] = pre;
        if (seg == K::NSEG - 1) stBL(s)[col] = pre * sTot[seg * GW + col];
      }
    }
    // b at row r, columns c .. c + VE - 1
    auto b_vec = [&](float *bb, int r, int c) {
      if constexpr (K::GATE) {
        const float *loc = ((ROLE == BWD_DV) ? sBS : stB(s)) + r * GW + c;
        // the rows of one wave's vector lie in one segment (static_assert below): a scalar loop
        const int seg = __builtin_amdgcn_readfirstlane(r / K::SEGR);
#pragma unroll
        for (int e = 0; e < VE; e += 4) {
          f32x4 pre = {1.f, 1.f, 1.f, 1.f};
          for (int s2 = 0; s2 < seg; ++s2) pre *= *reinterpret_cast<const f32x4 *>(sTot + s2 * GW + c + e);
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(loc + e);
          bb[e] = l4[0] * pre[0]; bb[e + 1] = l4[1] * pre[1];
          bb[e + 2] = l4[2] * pre[2]; bb[e + 3] = l4[3] * pre[3];
        }
      } else {
        float x = 1.f;
        if constexpr (K::TOKEN) x = stB(s)[r];
        else if constexpr (K::GAMMA) x = sBS[r];
#pragma unroll
        for (int e = 0; e < VE; ++e) bb[e] = x;
      }
    };
    // the decayed tiles, with phi chosen once for the whole chunk
    auto transform = [&](auto elu_c) {
      constexpr bool ELU = decltype(elu_c)::value;
      if constexpr (ROLE == BWD_DV) {
        constexpr int VPRX = DY / VE;
        // when vector j of every thread lies in gate segment j, the segment prefix is a
        // running product over j (the same products, in the same order, as b_vec's loop)
        constexpr bool RUN = K::GATE && K::NTG / VPRX == K::SEGR;
        float pre[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) pre[e] = 1.f;
#pragma unroll
        for (int j = 0; j < K::NVX; ++j) {
          const int vi = ptid + K::NTG * j, r = vi / VPRX, c = (vi % VPRX) * VE;
          float fx[VE], fy[VE], bb[VE];
          unpack<TIn, VE>(fx, rX[j]);
          unpack<TIn, VE>(fy, rY[j]);
          if constexpr (RUN) {
#pragma unroll
            for (int e = 0; e < VE; e += 4) {
              const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sBS + r * GW + c + e);
              bb[e] = l4[0] * pre[e]; bb[e + 1] = l4[1] * pre[e + 1];
              bb[e + 2] = l4[2] * pre[e + 2]; bb[e + 3] = l4[3] * pre[e + 3];
            }
            if (j + 1 < K::NVX) {
#pragma unroll
              for (int e = 0; e < VE; e += 4) {
                const f32x4 t4 = *reinterpret_cast<const f32x4 *>(sTot + j * GW + c + e);
                pre[e] *= t4[0]; pre[e + 1] *= t4[1]; pre[e + 2] *= t4[2]; pre[e + 3] *= t4[3];
              }
            }
          } else {
            b_vec(bb, r, c);
          }
          const float ok = r < L ? 1.f : 0.f; // rows past the end (finite values): zeros
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            fx[e] = phi_c<ELU>(fx[e]) * rcp_f(bb[e]) * ok;
            fy[e] = phi_c<ELU>(fy[e]) * bb[e] * ok;
          }
          st_lds<TIn, VE>(stX(s) + r * LDX + c, fx);
          st_lds<TIn, VE>(stY(s) + r * LDX + c, fy);
        }
      } else {
        constexpr int VPRZ = XW / VE;
#pragma unroll
        for (int j = 0; j < K::NVZ; ++j) {
          const int vi = ptid + K::NTG * j, r = vi / VPRZ, c = (vi % VPRZ) * VE;
          float fz[VE], bb[VE];
          unpack<TIn, VE>(fz, rZ[j]);
          b_vec(bb, r, c);
          const float ok = r < L ? 1.f : 0.f; // rows past the end (finite values): zeros
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            const float pz = phi_c<ELU>(fz[e]);
            fz[e] = (ROLE == BWD_DQ ? pz * rcp_f(bb[e]) : pz * bb[e]) * ok;
          }
          st_lds<TIn, VE>(stZ(s) + r * LDZ + c, fz);
          if constexpr (K::SPLIT) {
            float fl[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) fl[e] = fz[e] - (float)(TIn)fz[e];
            st_lds<TIn, VE>(stZL(s) + r * LDZ + c, fl);
          }
        }
      }
    };
    if (elu1) transform(std::true_type{});
    else transform(std::false_type{});
  };

  if constexpr (K::PC) {
    if (wave >= 4) {
      // ----- producer waves: stage (it + 1) & 1 while the consumers work on it & 1 -----
      if (nchunks > 0) {
        load1(chunk_at(0));
        load2(chunk_at(0));
        phase1(chunk_at(0), 0);
        if (nchunks > 1) load1(chunk_at(1));
      }
      __syncthreads();
      if (nchunks > 0) {
        phase2(chunk_at(0), 0);
        if (nchunks > 1) load2(chunk_at(1));
      }
      __syncthreads();
      for (int it = 0; it < nchunks; ++it) {
        const int s = (it + 1) & 1;
        if (it + 1 < nchunks) {
          phase1(chunk_at(it + 1), s);
          if (it + 2 < nchunks) load1(chunk_at(it + 2));
        }
        __syncthreads(); // consumers: score tiles of chunk it written
        if (it + 1 < nchunks) {
          phase2(chunk_at(it + 1), s);
          if (it + 2 < nchunks) load2(chunk_at(it + 2));
        }
        __syncthreads(); // consumers: chunk it done; stage s complete
      }
      return;
    }
  }

  // =========================== output group (waves 0-3) =================================
  // state: S[y][x] for y in DY, x = 16 wave + li; tile yb holds rows 16yb + 4g + q
  f32x4 S[NYB];
  {
    const float *s0 = (ROLE == BWD_DQ) ? a.init : a.dfinal;
#pragma unroll
    for (int yb = 0; yb < NYB; ++yb) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int y = 16 * yb + 4 * g + qq, x = 16 * wave + li;
        float val = 0.f;
        if (s0) {
          if constexpr (ROLE == BWD_DV) val = s0[(bh * dk + y) * dv + zoff + x];
          else val = s0[(bh * dk + zoff + x) * dv + y];
        }
        S[yb][qq] = val;
      }
    }
  }

  const int xc = 16 * wave + 4 * g; // first of this lane's 4 output columns
  // decay-gradient carry (DK): the sum over later chunks, per column (gate) or over this
  // wave's 16 columns (token); starts from the final state's term
  f32x4 carry4 = {0.f, 0.f, 0.f, 0.f};
  float carry = 0.f;
  if constexpr (ROLE == BWD_DK && K::GATE) {
    if (want_dg && a.fterm) carry4 = *reinterpret_cast<const f32x4 *>(a.fterm + bh * dk + goff + xc);
  }
  if constexpr (ROLE == BWD_DK && K::TOKEN) {
    if (want_dg && a.fterm) {
      float x = a.fterm[bh * dk + goff + 16 * wave + li];
      for (int d = 8; d >= 1; d >>= 1) x += __shfl_xor(x, d);
      carry = x;
    }
  }

  // this lane's rows 16 rb + li, columns xc .. xc+3: raw q (dq role) or k (dk role) for
  // phi and phi', and phi(q) dphi(q) from the dq pass (dk role) - read from global memory
  // at the start of the chunk, used by the output tiles
  uint32_t raux[4][K::ES]; // 4 elements of the input type
  f32x4 rqv[4];
  // the next chunk's per-lane values, loaded one chunk ahead (two-group schedule)
  uint32_t naux[4][K::ES];
  f32x4 nrqv[4];
  auto load_lane = [&](int n, uint32_t (&raux)[4][K::ES], f32x4 (&rqv)[4]) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;
    if constexpr (K::HAS_AUX) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        // rows past the end read the last row (no branch); their outputs are not stored
        const int r = 16 * rb + li, rc = r < L ? r : L - 1;
        const TIn *pa = srcA + (t0 + rc) * rsK + zoff + xc;
        if constexpr (K::ES == 2) {
          const uint2 w2 = *reinterpret_cast<const uint2 *>(pa);
          raux[rb][0] = w2.x; raux[rb][1] = w2.y;
        } else {
          const uint4 w4 = *reinterpret_cast<const uint4 *>(pa);
          raux[rb][0] = w4.x; raux[rb][1] = w4.y; raux[rb][2] = w4.z; raux[rb][3] = w4.w;
        }
        rqv[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (K::HAS_RQ) {
          if (want_dg) rqv[rb] = *reinterpret_cast<const f32x4 *>(a.rq + baseK + (t0 + rc) * rsK + zoff + xc);
        }
      }
    }
  };

  // ---- score tiles: image of tile (rb, sb) holds P[r][s] = X_r . Y_s, masked --------
  auto scores = [&](int s) {
    const TIn *sX = stX(s), *sY = stY(s);
    static_for<0, 16>([&](auto I) {
      constexpr int rb = I / 4, sb = I % 4;
      if constexpr (tile_on<REV>(rb, sb)) {
        if (tile_pos<REV>(rb, sb) % 4 == wave) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const TIn *ya = sY + (16 * sb + li) * LDX + (sizeof(TIn) == 2 ? 8 : 4) * g;
          const TIn *xb = sX + (16 * rb + li) * LDX + (sizeof(TIn) == 2 ? 8 : 4) * g;
#pragma unroll
          for (int u = 0; u < DY / KU; ++u)
            acc = mma(acc, ld_frag_c_at<TIn, true>(ya, u, g), ld_frag_c_at<TIn, true>(xb, u, g));
          // acc[qq] = P[r = 16 rb + li][s = 16 sb + 4g + qq]
          if constexpr (rb == sb) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int s2 = 4 * g + qq;
              const bool keep = REV ? (s2 >= li) : (s2 <= li);
              if (!keep) acc[qq] = 0.f;
            }
          }
          st_ptile<TIn>(sP + I * 256 + (16 * g + li) * 4, acc);
          if constexpr (K::SPLIT) {
            f32x4 lo;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) lo[qq] = acc[qq] - (float)(TIn)acc[qq];
            st_ptile<TIn>(sPL + I * 256 + (16 * g + li) * 4, lo);
          }
        }
      }
    });
  };

  // ---- output tiles, the state, and (dk) the decay gradient --------------------------
  auto finish = [&](int n, int s) {
    const int L = chunk_len(n);
    const int64_t t0 = (int64_t)n * C;
    const TIn *sX = stX(s), *sY = stY(s), *sZ = stZ(s), *sZL = stZL(s);
    const float *sB = stB(s), *sBL = stBL(s);
    (void)sB; (void)sBL; (void)sZL;
    // chunk decay bL of a column (gate) or of the chunk
    auto bl_at = [&](int idx) -> float {
      if constexpr (K::GATE) return sBL[idx];
      else if constexpr (K::TOKEN) return sBL[0];
      else if constexpr (K::GAMMA) return sBS[L - 1];
      else return 1.f;
    };
    const int x = 16 * wave + li; // this lane's state column in the slice
    if constexpr (ROLE == BWD_DK) {
      const float d = bl_at(x);
#pragma unroll
      for (int yb = 0; yb < NYB; ++yb) S[yb] *= d;
    } else if constexpr (ROLE == BWD_DV) {
#pragma unroll
      for (int yb = 0; yb < NYB; ++yb)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) S[yb][qq] *= bl_at(16 * yb + 4 * g + qq);
    }
    Frag<TIn> zf[NZU], zl[K::SPLIT ? NZU : 1];
#pragma unroll
    for (int u = 0; u < NZU; ++u) {
      zf[u] = ld_frag_t<TIn, true>(sZ, LDZ, 16 * wave, u, g, li);
      if constexpr (K::SPLIT) zl[u] = ld_frag_t<TIn, true>(sZL, LDZ, 16 * wave, u, g, li);
    }

    // Output tiles are formed transposed (out^T = Z^T P^T + S^T X^T: the same fragments with
    // the operands swapped), so a lane holds 4 adjacent columns of one row: 16-byte LDS
    // reads of the per-element factors and 8-byte (bf16) stores.
    f32x4 pre4[4]; // gate: prefix of the earlier segments, row block rb, columns xc..
    if constexpr (K::GATE && ROLE != BWD_DV) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) pre4[rb] = *reinterpret_cast<const f32x4 *>(stPre(s) + rb * GW + xc);
    }
    auto b_at4 = [&](int r, int rb) -> f32x4 {
      if constexpr (K::GATE) return *reinterpret_cast<const f32x4 *>(sB + r * GW + xc) * pre4[rb];
      else if constexpr (K::TOKEN) return f32x4{sB[r], sB[r], sB[r], sB[r]};
      else if constexpr (K::GAMMA) return f32x4{sBS[r], sBS[r], sBS[r], sBS[r]};
      else return f32x4{1.f, 1.f, 1.f, 1.f};
    };
    auto phi4 = [&](int rb) -> f32x4 {
      float f[4];
      unpack<TIn, 4>(f, raux[rb]);
      f32x4 p;
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = elu1 ? phi_c<true>(f[e]) : f[e];
      return p;
    };
    (void)phi4;
    (void)b_at4;
    // the state as MFMA fragments (hi and, for split roles, lo parts), once per chunk
    Frag<TIn> sfh[DY / KU], sfl[K::SPLIT ? DY / KU : 1];
#pragma unroll
    for (int u = 0; u < DY / KU; ++u) {
      if constexpr (sizeof(TIn) == 2) {
        sfh[u] = acc_frag_bf(S[2 * u], S[2 * u + 1]);
        if constexpr (K::SPLIT)
          sfl[u] = acc_frag_bf(S[2 * u] - bf_round4(S[2 * u]), S[2 * u + 1] - bf_round4(S[2 * u + 1]));
      } else {
        sfh[u] = S[u];
      }
    }
    f32x4 rr[4]; // dk: phi(q) dphi(q) - phi(k) dphi(k) of this lane's rows and columns
    static_for<0, 4>([&](auto RB) {
      constexpr int rb = RB;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      // intra-chunk: sum over allowed s of P[r][s] Z[s][x]
      static_for<0, NZU>([&](auto U) {
        constexpr int u = U;
        if constexpr (sizeof(TIn) == 2) {
          constexpr int TA = tile_on<REV>(rb, 2 * u) ? rb * 4 + 2 * u : -1;
          constexpr int TB = tile_on<REV>(rb, 2 * u + 1) ? rb * 4 + 2 * u + 1 : -1;
          if constexpr (TA >= 0 || TB >= 0) {
            const Frag<TIn> ph = ld_ptile2<TIn, TA, TB>(sP + (16 * g + li) * 4);
            acc = mma(acc, zf[u], ph);
            if constexpr (K::SPLIT) {
              acc = mma(acc, zf[u], ld_ptile2<TIn, TA, TB>(sPL + (16 * g + li) * 4));
              acc = mma(acc, zl[u], ph);
            }
          }
        } else {
          constexpr int TA = tile_on<REV>(rb, u) ? rb * 4 + u : -1;
          if constexpr (TA >= 0) acc = mma(acc, zf[u], ld_ptile2<TIn, TA, -1>(sP + (16 * g + li) * 4));
        }
      });
      // inter-chunk: sum over y of X[r][y] S[y][x]
      const TIn *xa = sX + (16 * rb + li) * LDX + 4 * g;
#pragma unroll
      for (int u = 0; u < DY / KU; ++u) {
        const Frag<TIn> xf = ld_frag_at<TIn, true>(xa, u);
        acc = mma(acc, sfh[u], xf);
        if constexpr (K::SPLIT) acc = mma(acc, sfl[u], xf);
      }
      // acc[qq] = out[r = 16 rb + li][xc + qq]
      const int r = 16 * rb + li;
      const int64_t t = t0 + r;
      if constexpr (ROLE == BWD_DQ) {
        const f32x4 dqb = acc * b_at4(r, rb);
        const f32x4 qb = phi4(rb);
        if (r < L) {
          f32x4 dq4;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dq4[qq] = dqb[qq] * phi_d(qb[qq], elu1);
          st_out4<TIn>((TIn *)a.grad_q + baseK + t * rsK + zoff + xc, dq4);
          if (want_dg) *reinterpret_cast<f32x4 *>(a.rq + baseK + t * rsK + zoff + xc) = qb * dqb;
        }
      } else if constexpr (ROLE == BWD_DK) {
        const f32x4 bb = b_at4(r, rb);
        f32x4 dkb;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) dkb[qq] = acc[qq] * rcp_f(bb[qq]);
        const f32x4 kb = phi4(rb);
        if (r < L) {
          f32x4 dk4;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dk4[qq] = dkb[qq] * phi_d(kb[qq], elu1);
          st_out4<TIn>((TIn *)a.grad_k + baseK + t * rsK + zoff + xc, dk4);
        }
        rr[rb] = (r < L) ? rqv[rb] - kb * dkb : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        if (r < L) st_out4<TIn>((TIn *)a.grad_v + baseV + t * rsV + zoff + xc, acc);
      }
    });
    (void)rr;

    // state update: S[y][x] += sum_s Y[s][y] Z[s][x]
#pragma unroll
    for (int yb = 0; yb < NYB; ++yb) {
#pragma unroll
      for (int u = 0; u < NZU; ++u) {
        const Frag<TIn> yf = ld_frag_t<TIn, true>(sY, LDX, 16 * yb, u, g, li);
        S[yb] = mma(S[yb], yf, zf[u]);
        if constexpr (K::SPLIT) S[yb] = mma(S[yb], yf, zl[u]);
      }
    }
    if constexpr (ROLE == BWD_DQ) {
      const float d = bl_at(x);
#pragma unroll
      for (int yb = 0; yb < NYB; ++yb) S[yb] *= d;
    }

    // decay gradient (DK): sums of r over the later tokens, in registers (rows across the
    // 16 lanes of a group and the 4 row blocks of a lane)
    if constexpr (ROLE == BWD_DK && K::GATE) {
      if (want_dg) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          float v[4] = {rr[0][qq], rr[1][qq], rr[2][qq], rr[3][qq]};
          const float tot = suffix_rows64(v, g);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) rr[rb][qq] = v[rb] + carry4[qq];
          carry4[qq] += tot;
        }
        // d alpha = d log alpha / alpha, with alpha_r = l_r / l_{r-1} from the local
        // products l down each 16-row segment (l_{r-1} = 1 at a segment's first row): exact
        // to an ulp or two where the products do not underflow, which the 1/b scaling of
        // the output tiles requires anyway
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int r = 16 * rb + li;
          const f32x4 lc = *reinterpret_cast<const f32x4 *>(sB + r * GW + xc);
          const f32x4 lp = *reinterpret_cast<const f32x4 *>(sB + (li ? r - 1 : r) * GW + xc);
          f32x4 dg;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dg[qq] = rr[rb][qq] * (li ? lp[qq] : 1.f) * rcp_f(lc[qq]);
          if (r < L) *reinterpret_cast<f32x4 *>(a.dgate + baseK + (t0 + r) * rsK + goff + xc) = dg;
        }
      }
    }
    if constexpr (ROLE == BWD_DK && K::TOKEN) {
      if (want_dg) {
        // row sums over this wave's 16 columns, then suffix sums over the rows
        float v[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          float sum = rr[rb][0] + rr[rb][1] + rr[rb][2] + rr[rb][3];
          sum += __shfl_xor(sum, 16);
          sum += __shfl_xor(sum, 32);
          v[rb] = sum;
        }
        const float tot = suffix_rows64(v, g);
        if (g == 0) {
          float *tp = a.tpart + ((int64_t)(h * a.nsl + slice) * 4 + wave) * a.ntok + tok0 + t0;
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int r = 16 * rb + li;
            if (r < L) tp[r] = v[rb] + carry;
          }
        }
        carry += tot;
      }
    }
  };

  if constexpr (K::PC) {
    // per-lane values one chunk ahead where that measured faster (dk; dq without the per-key
    // gate, whose dq output group waits on them later in the chunk)
    constexpr bool AHEAD = ROLE == BWD_DK || (ROLE == BWD_DQ && DECAY != DECAY_GATE);
    if constexpr (AHEAD) {
      if (nchunks > 0) load_lane(chunk_at(0), naux, nrqv);
    }
    __syncthreads(); // stage 0: phase 1 done
    __syncthreads(); // stage 0 complete
    for (int it = 0; it < nchunks; ++it) {
      const int n = chunk_at(it);
      if constexpr (AHEAD) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
          for (int e = 0; e < K::ES; ++e) raux[rb][e] = naux[rb][e];
          rqv[rb] = nrqv[rb];
        }
        // clamped past the last chunk: loads an existing chunk, values unused
        load_lane(chunk_at(it + 1 < nchunks ? it + 1 : it), naux, nrqv);
      } else {
        load_lane(n, raux, rqv);
      }
      scores(it & 1);
      __syncthreads();
      finish(n, it & 1);
      __syncthreads();
    }
  } else {
    // one wave group forms the operands and then the outputs of each chunk
    if (nchunks > 0) {
      load1(chunk_at(0));
      load2(chunk_at(0));
    }
    for (int it = 0; it < nchunks; ++it) {
      const int n = chunk_at(it);
      load_lane(n, raux, rqv);
      phase1(n, 0);
      if (it + 1 < nchunks) load1(chunk_at(it + 1));
      __syncthreads();
      phase2(n, 0);
      if (it + 1 < nchunks) load2(chunk_at(it + 1));
      __syncthreads();
      scores(0);
      __syncthreads();
      finish(n, 0);
      __syncthreads();
    }
  }

  // ---- epilogue ---------------------------------------------------------------------
  const int x = 16 * wave + li;
  if constexpr (ROLE == BWD_DQ) {
    if (want_dg && a.fterm) {
      float part = 0.f;
      if (a.dfinal) {
#pragma unroll
        for (int yb = 0; yb < NYB; ++yb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            part += a.dfinal[(bh * dk + zoff + x) * dv + 16 * yb + 4 * g + qq] * S[yb][qq];
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (g == 0) a.fterm[bh * dk + zoff + x] = part;
    }
  } else if constexpr (ROLE == BWD_DV) {
    if (a.dinit) {
#pragma unroll
      for (int yb = 0; yb < NYB; ++yb)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          a.dinit[(bh * dk + 16 * yb + 4 * g + qq) * dv + zoff + x] = S[yb][qq];
    }
  }
}

} // namespace fla
