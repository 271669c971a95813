/*
 * la_probe.h - measurement probe library (libla_probe.so) for gfx950.  Not
 * part of the attention path: it measures what the chip's matrix cores and
 * memory give in the same run as the attention kernels, so that their
 * utilisation can be stated against measured peaks as well as datasheet ones.
 *
 * la_probe_mfma - every wave of a grid of `grid` workgroups (256 threads, four
 * waves) runs `iters` rounds of eight independent matrix-core instructions
 * back to back (eight accumulators, so no instruction waits for the one
 * before it):
 *   kind 0: v_mfma_f32_16x16x32_bf16 (2 * 16 * 16 * 32 = 16,384 flops each);
 *   kind 1: v_mfma_i32_16x16x64_i8   (2 * 16 * 16 * 64 = 32,768 ops each).
 * Total work: grid * 4 * iters * 8 * (flops per instruction).
 *
 *   out   [grid * 256] float, device: one value per thread (the accumulators
 *         summed), written so that the work is not optimised away.
 *   stream  the HIP stream to enqueue on (0 = the null stream).
 * Returns 0, or -1 on a non-positive iters or grid, an unknown kind or a NULL
 * out (nothing launched), or the HIP error code of the launch.
 *
 * la_probe_read - the read bandwidth the memory system gives a plain stream:
 * a grid of `grid` workgroups (256 threads) reads the n16 16-byte vectors of x
 * `reps` times over, grid-stride (thread i reads vectors i, i + 256 grid,
 * ...), and folds them into one value per thread.  Read back to back, a set
 * larger than the last-level cache streams from HBM; a smaller one is re-read
 * from the cache after its first pass.
 *
 *   x     [n16] 16-byte vectors, device, 16-byte aligned (read only).
 *   out   [grid * 256] float, device: one value per thread.
 *   stream  the HIP stream to enqueue on (0 = the null stream).
 * Bytes read: 16 * n16 * reps.  Returns 0, or -1 on a NULL x or out, a
 * non-positive n16, reps or grid, or an x not 16-byte aligned (nothing
 * launched), or the HIP error code of the launch.
 */
#ifndef LIBLINATTN_LA_PROBE_H
#define LIBLINATTN_LA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int la_probe_mfma(int kind, int64_t iters, int64_t grid, float* out, struct ihipStream_t* stream);
int la_probe_read(const void* x, int64_t n16, int64_t reps, int64_t grid, float* out, struct ihipStream_t* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBLINATTN_LA_PROBE_H */
