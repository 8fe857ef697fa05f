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

#ifdef __cplusplus
}
#endif

#endif /* FLA_PROBE_H */
