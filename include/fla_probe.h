/*
 * fla_probe.h — measurement probes of the chunkwise linear attention library.
 *
 * They are not part of the attention path.  The benchmark runs them beside it to measure
 * what this GPU reaches with plain streaming and plain MFMA kernels, so the attention
 * kernel's roofline fraction can be read against a measured ceiling as well as the
 * published peaks (HBM3E 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).
 *
 * Both calls are asynchronous on `stream` (a hipStream_t, NULL = default stream); the
 * caller times them with events on that stream.  Pointers are device pointers owned by
 * the caller.  Return 0, -1 for an invalid argument (nothing enqueued), -3 when the
 * launch fails.
 */
#ifndef FLA_PROBE_H
#define FLA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLA_PROBE_READ 0 /* read `bytes` of src; dst receives one word per workgroup (16 KiB suffices) */
#define FLA_PROBE_COPY 1 /* copy `bytes` from src to dst */
#define FLA_PROBE_MIX5 2 /* read 5/6 of `bytes` from src, write 1/6 to dst (bytes % 96 == 0) */

/*
 * fla_probe_stream — one streaming pass with 16-byte non-temporal vector loads and stores.
 *   src, dst: 16-byte aligned.  bytes: a positive multiple of 16 (of 96 for MIX5).
 *   READ moves `bytes`; COPY moves 2 * `bytes` (read + write); MIX5 moves `bytes`
 *   (5/6 read from src, 1/6 written to dst; src holds 5/6 * bytes, dst 1/6 * bytes).
 */
int fla_probe_stream(const void *src, void *dst, int64_t bytes, int pattern, void *stream);

/*
 * fla_probe_mfma — `workgroups` workgroups of four waves, each wave running `iters`
 * iterations of four independent v_mfma_f32_32x32x16_bf16 chains on register operands.
 *   out: fp32, one word per wave (4 * workgroups words), written with the chains' sums.
 * fla_probe_mfma_flops gives the dense FLOPs such a launch performs.
 */
int fla_probe_mfma(float *out, int64_t workgroups, int64_t iters, void *stream);
double fla_probe_mfma_flops(int64_t workgroups, int64_t iters);

/*
 * fla_probe_chunk_pattern — the access pattern of the gated forward pass (fla_linattn_fwd
 * with FLA_BF16 | FLA_DECAY_GATE, dk = 128, 64-token chunks) with none of its arithmetic:
 * one workgroup per (b, h, 64-wide value slice), sibling slices of a head on one XCD,
 * walking the chunks in order; per chunk it reads the chunk's q, k and gate rows and its
 * value slice and writes its output slice, one chunk of loads in flight ahead of the
 * stores.  It moves the forward pass's bytes without its final state (B H T (4 dk + 4 dk
 * + 4 dv) bytes), so its rate is the ceiling of that pattern on this GPU.
 *   q, k: bf16 [B][H][T][128]; gate: fp32 [B][H][T][128]; v, out: bf16 [B][H][T][dv],
 *   dv a multiple of 64 up to 256; 1 <= T <= 2^36; all 16-byte aligned.  out[b][h][t] receives, per 16-byte
 *   vector, the value vector XOR the XOR of the q, k and gate vectors its lane read (lane
 *   t of a workgroup reads vectors t + 256 i of the chunk's q, k and gate rows and vectors
 *   j = t + 256 i of the value slice, vector j being row j / 8, bytes 16 (j % 8) of the
 *   slice).
 */
int fla_probe_chunk_pattern(const void *q, const void *k, const float *gate, const void *v,
                            void *out, int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FLA_PROBE_H */
