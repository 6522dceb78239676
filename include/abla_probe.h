/*
 * abla_probe -- measurement probes used by the benchmark, not part of the attention path.
 *
 * abla_probe_mfma: one launch of `grid` workgroups of four waves, each wave issuing `iters`
 * rounds of four independent matrix-core products with no memory traffic: kind 0 =
 * v_mfma_f32_32x32x16_bf16 (bf16 inputs, float32 accumulation), kind 1 =
 * v_mfma_f32_32x32x2_f32 (float32). Timing it on a board gives the sustained matrix rate there
 * (power and clock limits included). `sink` is a device buffer of `grid` floats that is never
 * written in practice (it keeps the loop alive). Returns 0, 1 for a bad argument, 4 for a
 * failed launch. abla_probe_mfma_flops: the floating-point operations of such a launch.
 *
 * abla_probe_stream: one launch streaming `bytes` bytes (a multiple of 32 KiB) of the device
 * buffer `src`, one contiguous 32 KiB span per 256-thread workgroup, eight 16-byte loads in
 * flight per thread: copy = 0 only reads (dst receives at most one 16-byte word, and only for a
 * value no ordinary input produces), copy = 1 writes the same bytes to dst. Timing it gives the
 * HBM rate the board sustains for reads, and for an equal read/write mix.
 * Returns 0, 1 for a bad argument (null, misaligned, size), 4 for a failed launch.
 */
#ifndef ABLA_PROBE_H
#define ABLA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t abla_probe_mfma(int32_t kind, int32_t grid, int32_t iters, float* sink, void* stream);
double abla_probe_mfma_flops(int32_t kind, int32_t grid, int32_t iters);
int32_t abla_probe_stream(int32_t copy, const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ABLA_PROBE_H */
