/*
 * fla_linattn.h — C ABI of the MI355X (gfx950) chunkwise causal linear attention library.
 *
 * The operation (forward pass, "chunk" mode) is causal linear attention with an
 * optional decay, per (batch b, head h):
 *
 *     S_t = G_t (.) S_{t-1} + v_t phi(k_t)^T          (state, d_v x d_k)
 *     z_t = G_t (.) z_{t-1} + phi(k_t)                 (normaliser, only with FLA_NORMALIZE)
 *     o_t = S_t phi(q_t)            or   S_t phi(q_t) / (z_t^T phi(q_t))
 *
 * Sources: the textbook chapter 1.6 "Long context and efficient attention", section
 * "linear attention" (recurrence, normaliser, elu+1 feature map, parallel = recurrent),
 * and the Flash Linear Attention posts (RetNet retention with a per-head decay gamma,
 * GLA with a per-token per-key gate alpha_t, "chunk" mode forward).  G_t is 1 (plain
 * linear attention), gamma_h (FLA_DECAY_GAMMA), alpha_t (FLA_DECAY_GATE) or a per-token
 * scalar a_t (FLA_DECAY_TOKEN: one decay per token and head, the data-dependent form of
 * the retention decay); the gate multiplies key column c of S for every value row, the
 * old state is decayed before the current token is added, and z decays with the same G_t.
 *
 * Layouts (all row-major, contiguous, device memory of the current HIP device):
 *   q, k    [B][H][T][dk]   bf16 (FLA_BF16) or fp32
 *   v, out  [B][H][T][dv]   same dtype as q
 *   gamma   [H]             fp32, values in [0, 1]
 *   gate    [B][H][T][dk]   fp32, values in [0, 1]
 *   token   [B][H][T]       fp32, values in [0, 1] (per-token scalar decay)
 *   state   [B][H][dk][dv + n] fp32, n = 1 with FLA_NORMALIZE (column dv holds z);
 *           this is h = S^T, so state[b][h][c][e] = S[e][c].
 * With FLA_LAYOUT_BTHD (forward calls) the per-token tensors are token-major instead, as
 * the projections of a [B][T][hidden] activation produce them: q, k, gate [B][T][H][dk],
 * v, out [B][T][H][dv], per-token decay [B][T][H]; gamma and the states are unchanged.
 *
 * Ownership: every pointer belongs to the caller; the library keeps none after a call
 * returns and holds no global mutable state.  Calls are asynchronous on `stream`
 * (a hipStream_t; NULL = the default stream) and never synchronise the host.  Inputs
 * are read-only.  Errors found on the host are returned before anything is enqueued;
 * faults during execution surface at the caller's next synchronisation.
 */
#ifndef FLA_LINATTN_H
#define FLA_LINATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
enum fla_status {
  FLA_OK = 0,
  FLA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad or conflicting flags */
  FLA_ERR_UNSUPPORTED = -2, /* valid request outside the built shape set */
  FLA_ERR_DEVICE = -3,      /* a HIP launch or stream-ordered allocation failed */
  FLA_ERR_SCRATCH = -4      /* the no-allocation entry point's scratch array is too small */
};

/* Flag bits. */
#define FLA_BF16 (1u << 0)        /* q, k, v, out are bf16; otherwise fp32 */
#define FLA_DECAY_GAMMA (1u << 1) /* gate_or_gamma = const float[H] */
#define FLA_DECAY_GATE (1u << 2)  /* gate_or_gamma = const float[B][H][T][dk] */
#define FLA_PHI_ELU1 (1u << 3)    /* phi(x) = elu(x) + 1 on q and k; otherwise identity */
#define FLA_NORMALIZE (1u << 4)   /* divide by z_t^T phi(q_t); the state carries z */
#define FLA_DECAY_TOKEN (1u << 5) /* gate_or_gamma = const float[B][H][T] (scalar per token) */
#define FLA_LAYOUT_BTHD (1u << 6) /* token-major q, k, v, out, gate: [B][T][H][d] (see below) */
#define FLA_ALL_FLAGS                                                                      \
  (FLA_BF16 | FLA_DECAY_GAMMA | FLA_DECAY_GATE | FLA_PHI_ELU1 | FLA_NORMALIZE |           \
   FLA_DECAY_TOKEN | FLA_LAYOUT_BTHD)

/*
 * fla_linattn_fwd — chunkwise forward pass over T tokens.
 * Defined by the token recurrence above (textbook chapter 1.6, "linear attention": the
 * state update and read-out, trained "in parallel or in chunks"), evaluated in chunk mode
 * (the FLA posts' chunk-mode forward; chapter 1.6, "state-space models and Mamba": linear
 * attention with a decay mask, trained in matmul-friendly chunks).
 *
 *   q, k, v, out : see layouts above; 16-byte aligned.  May be NULL only when T == 0.
 *   gate_or_gamma: gamma [H] with FLA_DECAY_GAMMA (4-byte aligned), gate [B][H][T][dk]
 *                  with FLA_DECAY_GATE (16-byte aligned), token [B][H][T] with
 *                  FLA_DECAY_TOKEN (4-byte aligned), NULL with no decay bit.
 *   init_state   : [B][H][dk][dv+n] fp32, or NULL for a zero initial state (16-byte aligned).
 *   final_state  : [B][H][dk][dv+n] fp32 written with the state after token T-1, or NULL.
 *                  May alias init_state (in-place resume).
 *   B, H >= 1; T >= 0; dk, dv in {16, 32, 64, 128, 256}; chunk in {16, 32, 64, 128,
 *                  256, 512, 1024}: the tile sizes are 16..128; a larger chunk (the FLA
 *                  posts advise chunk_size = 512 for long-sequence training) is evaluated
 *                  as consecutive 64-token sub-chunks (the fastest tile), which is exact
 *                  in real arithmetic; so is chunk 128 with FLA_DECAY_GATE or dk = 256,
 *                  whose 128-token tiles measured 4-8x slower, bf16 chunk 128 with
 *                  FLA_DECAY_GAMMA at dk = 128 (about 4% slower at long sequences), and
 *                  fp32 chunk 128 at dk >= 128, whose 128-token tile does not fit the
 *                  160 KiB LDS.
 *   flags        : FLA_* bits; at most one decay bit.
 *   stream       : hipStream_t or NULL.
 *
 * T == 0 leaves out untouched and writes init_state (or zeros) to final_state.
 * The chunk size changes the rounding, never the mathematical result.  Every (dtype, dk,
 * dv, chunk) combination listed above is supported; other values return
 * FLA_ERR_UNSUPPORTED.
 * Decay range (FLA_DECAY_GATE and FLA_DECAY_TOKEN): any decay in [0, 1].  The fused
 * kernel factors a chunk's decays as phi(q) b and phi(k) / b (b: the product of the
 * decays from the chunk start), which is used while every chunk's product stays at or
 * above 2^-100; it flags the (b, h) units where one does not, and an exact 16-token kernel
 * (running products only, fp32) then recomputes those units' outputs and final states
 * (a few times slower per unit; units that stay in range pay one extra launch that exits
 * at once, plus a stream-ordered buffer of 16 B*H*segments bytes for the flags).
 */
int fla_linattn_fwd(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                    const float *init_state, void *out, float *final_state, int64_t B,
                    int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk,
                    uint32_t flags, void *stream);

/*
 * fla_linattn_fwd_segments — fla_linattn_fwd with an explicit choice of schedule.
 * The segment schedule splits the sequence like the context parallelism textbook chapter
 * 1.6 mentions for long contexts, with the recurrence's state as the only thing carried
 * between pieces (end state from zero, then a scan of the pieces' decays and end states).
 *   n_segments == 0: automatic (same as fla_linattn_fwd).
 *   n_segments == 1: one workgroup per (b, h, 64-wide value slice) streams all chunks.
 *   n_segments  > 1: the sequence is cut into that many segments of whole chunks; the
 *                    segments' end states are combined by a scan, then every segment
 *                    produces its outputs from its own start state (three launches and a
 *                    stream-ordered workspace of B*H*n_segments*dk*(dv+n+1)*4 bytes).
 * Both schedules compute the same function; they differ in rounding only.
 */
int fla_linattn_fwd_segments(const void *q, const void *k, const void *v,
                             const float *gate_or_gamma, const float *init_state, void *out,
                             float *final_state, int64_t B, int64_t H, int64_t T, int64_t dk,
                             int64_t dv, int64_t chunk, uint32_t flags, int64_t n_segments,
                             void *stream);

/*
 * fla_linattn_fwd_noalloc — fla_linattn_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, layouts, validation and results as fla_linattn_fwd; it calls no
 * hipMalloc / hipMallocAsync / hipFree and no allocating library routine.
 *   The workspaces the forward pass needs (the gated kinds' range flags, the segment
 *   schedule's per-segment end states and decay products, and the private start-state
 *   copy of an in-place resume with the normaliser) come from a static device array of
 *   64 MiB that each GPU the library runs on holds until the process ends.  The automatic segment count is halved
 *   until its workspace fits (so long sequences may run with fewer segments than
 *   fla_linattn_fwd chooses: same function, different rounding); a request that still
 *   does not fit returns FLA_ERR_SCRATCH before anything is enqueued.
 *   Every call on a GPU shares that GPU's array: calls that overlap on one GPU (on
 *   different streams, or from different host threads) race and must be serialised by
 *   the caller.  Nothing in the array needs to start at zero.
 * The first call on a device looks up the array's device address (hipGetSymbolAddress).
 */
int fla_linattn_fwd_noalloc(const void *q, const void *k, const void *v,
                            const float *gate_or_gamma, const float *init_state, void *out,
                            float *final_state, int64_t B, int64_t H, int64_t T, int64_t dk,
                            int64_t dv, int64_t chunk, uint32_t flags, void *stream);

/*
 * fla_linattn_fwd_proj — the layer's input side fused with the feature map, then the
 * forward pass: a linear-attention layer maps activations x [B][T][hidden] to per-head
 * q, k, v (the FLA guide's layers), and the FLA Triton post fuses the Q/K/V projections
 * with the phi computation.  Per token and head h:
 *     q = phi(x W_q)[h d_k .. h d_k + d_k),  k = phi(x W_k)[...],  v = (x W_v)[h d_v ..],
 * then the recurrence of fla_linattn_fwd on them.
 *   x      : [B][T][hidden]; w_q, w_k: [hidden][H*dk]; w_v: [hidden][H*dv]; row-major, the
 *            input dtype (bf16 with FLA_BF16, else fp32), 16-byte aligned.
 *   out    : [B][T][H][dv] (token-major), the input dtype.
 *   gate_or_gamma: gamma [H], gate [B][T][H][dk] or per-token decay [B][T][H] (token-major),
 *            or NULL; init_state / final_state: [B][H][dk][dv + n] fp32 as fla_linattn_fwd.
 *   hidden : a multiple of 32; H*dk and H*dv multiples of 16; other limits as
 *            fla_linattn_fwd with FLA_LAYOUT_BTHD (implied).  FLA_PHI_ELU1 applies phi to
 *            the projected q and k, inside the projection kernel.
 * The projections are MFMA GEMMs with phi in their epilogue (one launch per projection),
 * written to stream-ordered workspaces (B T H (2 dk + dv) elements of the input dtype),
 * then read by the chunk kernel.  Everything is validated before the first launch.
 */
int fla_linattn_fwd_proj(const void *x, const void *w_q, const void *w_k, const void *w_v,
                         const float *gate_or_gamma, const float *init_state, void *out,
                         float *final_state, int64_t B, int64_t T, int64_t hidden, int64_t H,
                         int64_t dk, int64_t dv, int64_t chunk, uint32_t flags, void *stream);

/*
 * fla_linattn_fwd_varlen — fla_linattn_fwd over packed variable-length sequences (the
 * Triton fused-kernel post recommends chunk mode for variable-length input; the FLA
 * guide's layers take [B][T][hidden] activations, hence the token-major layout).
 *   q, k, gate: [total_T][H][dk]; v, out: [total_T][H][dv]; per-token decay [total_T][H]
 *   (token-major, FLA_LAYOUT_BTHD implied); sequence s owns tokens cu_seqlens[s] ..
 *   cu_seqlens[s+1]-1.
 *   cu_seqlens   : device int64 [n_seqs + 1], 8-byte aligned, non-decreasing from 0 to
 *                  total_T.  Values are clamped to [0, total_T] on the device, so a bad array
 *                  gives wrong results, never an out-of-range access.
 *   init_state, final_state: [n_seqs][H][dk][dv + n] fp32 (one state per sequence), or NULL.
 *   Other arguments as fla_linattn_fwd (B = n_seqs, T = total_T).  One streaming workgroup
 *   per (sequence, head, 64-wide value slice); sequences are independent.  For 2 to 8192
 *   sequences a small kernel first ranks them by chunk count (a stream-ordered buffer of
 *   n_seqs*4 bytes) so the workgroups of the longest sequences are dispatched first; the
 *   order changes no result.
 */
int fla_linattn_fwd_varlen(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                           const float *init_state, void *out, float *final_state,
                           const int64_t *cu_seqlens, int64_t n_seqs, int64_t total_T, int64_t H,
                           int64_t dk, int64_t dv, int64_t chunk, uint32_t flags, void *stream);

/*
 * fla_linattn_step — one token of recurrent decoding (the T == 1 case of the forward
 * pass), updating the state in place: the recurrent form of textbook chapter 1.6, "linear
 * attention" (constant memory per generated token, as the chapter contrasts with a
 * growing KV cache).
 *   q, k : [B][H][dk]; v, out: [B][H][dv] (bf16 with FLA_BF16, else fp32); 16-byte aligned.
 *   gate_or_gamma: gamma [H], gate [B][H][dk] or token [B][H] per the decay bit, else NULL.
 *   state: fp32 [B][H][dk][dv+n], read and written (required).
 *   dk, dv in {16, 32, 64, 128, 256}.  One token is laid out the same way in either
 *   layout, so FLA_LAYOUT_BTHD changes nothing here.
 */
int fla_linattn_step(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                     float *state, void *out, int64_t B, int64_t H, int64_t dk, int64_t dv,
                     uint32_t flags, void *stream);

/*
 * fla_linattn_bwd — gradients of the forward pass (chunkwise backward), for the loss
 * L = sum(dout (.) out) + sum(dfinal_state (.) final_state), by the reverse-mode chain rule
 * through the recurrence above (no normaliser).  The FLA posts time chunk mode forward
 * and backward together for training; this is the backward half.
 *
 *   q, k, v, gate_or_gamma, init_state: the forward call's inputs (layouts above, including
 *                  token-major [B][T][H][d] with FLA_LAYOUT_BTHD).
 *   dout         : laid out like v (dtype of q); the gradient arriving at out.
 *   dfinal_state : fp32 [B][H][dk][dv] gradient arriving at final_state, or NULL (zero).
 *   dq, dk, dv   : written, shaped and typed like q, k, v.
 *   dgate        : fp32, written with the gradient of the per-key gate [B][H][T][dk]
 *                  (FLA_DECAY_GATE) or of the per-token decay [B][H][T] (FLA_DECAY_TOKEN);
 *                  NULL skips it.  Must be NULL with FLA_DECAY_GAMMA (gamma is a constant
 *                  of the model here) or without a decay.
 *   dinit_state  : fp32 [B][H][dk][dv] written with the gradient of init_state (whether or
 *                  not init_state was given), or NULL.
 *   All pointers 16-byte aligned, except gamma and the per-token decay (4 bytes).
 *   dk, dv in {64, 128, 256} (fp32: up to 128); chunk: any value the forward call takes
 *   (the backward always tiles by 64 tokens, the same function); FLA_NORMALIZE is not supported;
 *   token-major: H * max(dk, dv) <= 2^20.
 *   Three chunk-scan launches (dq forward in time; dv, then dk and dgate in reverse) and,
 *   when dgate is requested, a stream-ordered workspace of 4 (B H T dk + B H dk) bytes
 *   (+ 4 B H T dk/16 for the per-token decay, and a fourth small launch that sums it).
 * Returns FLA_ERR_UNSUPPORTED for shapes or flags outside that set.  Decay range: the
 * backward kernels use the factorised form only, so every chunk's product of the decays
 * (per key) must stay at or above 2^-100 (the GLA workload's is about 2^-5).
 */
int fla_linattn_bwd(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                    const float *init_state, const void *dout, const float *dfinal_state,
                    void *dq, void *dk, void *dv, float *dgate, float *dinit_state, int64_t B,
                    int64_t H, int64_t T, int64_t dk_dim, int64_t dv_dim, int64_t chunk,
                    uint32_t flags, void *stream);

/*
 * fla_linattn_bwd_varlen — fla_linattn_bwd over packed variable-length sequences: the
 * gradients of fla_linattn_fwd_varlen.  Tensors as in that call (token-major [total_T][H][d];
 * dout and dv like v; dq, dk like q, k; dgate like the gate or per-token decay); states
 * init_state, dfinal_state, dinit_state: [n_seqs][H][dk][dv] fp32.  cu_seqlens as in
 * fla_linattn_fwd_varlen (device int64 [n_seqs + 1], clamped to [0, total_T] on the device).
 * Other arguments and limits as fla_linattn_bwd (B = n_seqs, T = total_T); sequences are
 * independent, and an empty sequence gets dinit_state = dfinal_state.
 */
int fla_linattn_bwd_varlen(const void *q, const void *k, const void *v, const float *gate_or_gamma,
                           const float *init_state, const void *dout, const float *dfinal_state,
                           void *dq, void *dk, void *dv, float *dgate, float *dinit_state,
                           const int64_t *cu_seqlens, int64_t n_seqs, int64_t total_T, int64_t H,
                           int64_t dk_dim, int64_t dv_dim, int64_t chunk, uint32_t flags,
                           void *stream);

/*
 * fla_gdn_fwd — gated delta rule, chunkwise forward (textbook chapter 1.6, section "gated
 * delta rule"; the Gated DeltaNet op the FLA posts list).  Per (b, h), with the unit-norm
 * key k^_t = k_t / max(|k_t|, 1e-12) (normalised inside the call, as the chapter's reference
 * code does) and q used as given:
 *     S_t = alpha_t S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T,   o_t = S_t q_t,
 * i.e. decay the memory, replace a beta_t share of what it stores under k^_t by v_t.
 *   q, k  : [B][H][T][dk]; v, out: [B][H][T][dv] (bf16 with FLA_BF16, else fp32); 16-byte aligned.
 *   alpha : fp32 [B][H][T], the decay in [0, 1] (the in-chunk decay ratios are formed in
 *           mantissa-exponent form, so any product is exact or negligibly small);
 *   beta  : fp32 [B][H][T], the write strength in [0, 1]; 4-byte aligned.
 *   init_state, final_state: fp32 [B][H][dk][dv] (h = S^T as above) or NULL; may alias.
 *   dk in {64, 128} (fp32: 64); dv a multiple of 64 up to 256; chunk: any value fla_linattn_fwd
 *   takes (64-token tiles are used for all of them); flags: FLA_BF16 only.
 * Two launches: a pre-pass forms, for every chunk at once, the part that does not depend
 * on the state (Tb = T diag(beta) with T the inverse of the chunk's unit lower-triangular
 * delta system; its ten lower-triangle 16 x 16 blocks), into a stream-ordered workspace
 * of B H ceil(T / 64) 2560 elem bytes;
 * then one workgroup per (b, h, 64-wide value slice) streams the chunks with the state on
 * chip, forming U = Tb (V - diag(g) K^ H) per chunk.
 */
int fla_gdn_fwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                const float *init_state, void *out, float *final_state, int64_t B, int64_t H,
                int64_t T, int64_t dk, int64_t dv, int64_t chunk, uint32_t flags, void *stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char *fla_status_string(int status);

/*
 * fla_linattn_segments_for — the segment count fla_linattn_fwd would choose for a shape
 * (1 = single streaming launch; the schedule of fla_linattn_fwd_segments).  Returns a
 * status; *n_segments is set on FLA_OK.
 */
int fla_linattn_segments_for(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                             int64_t chunk, uint32_t flags, int64_t *n_segments);

#ifdef __cplusplus
}
#endif

#endif /* FLA_LINATTN_H */
