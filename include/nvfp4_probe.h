/*
 * nvfp4_probe.h -- C ABI of libnvfp4_probe: the measured walls the NVFP4
 * products are reported against.  A measurement aid, not part of the
 * product: the bw24 README (performance notes) reports its best kernel as a
 * fraction of a measured DRAM wall beside the nominal peak, and these
 * kernels measure that wall on this GPU in the same process as the
 * products, at their byte counts and launch counts.
 *
 * Conventions as in nvfp4.h: caller-owned device pointers, asynchronous and
 * stream-ordered calls, int status (0 or a negative NVFP4_E* code), no
 * allocation.
 */
#ifndef NVFP4_PROBE_H
#define NVFP4_PROBE_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One plain streaming read of `bytes` bytes at `buf` (16-byte aligned,
 * bytes < 2^31): `groups` workgroups of 256 threads each read one
 * contiguous share with 128-bit nontemporal loads, eight in flight per
 * thread, and fold them with XOR; nothing is stored unless the fold hits a
 * fixed 32-bit value (then one word to sink[0]).  1 <= groups <= 65536. */
int nvfp4_probe_stream_read(const void *buf, size_t bytes, int groups, uint32_t *sink, hipStream_t stream);

/* The same read of `rbytes` bytes at `buf`, then each workgroup stores its
 * contiguous share of the `obytes`-byte output at `out` (16-byte aligned,
 * obytes a multiple of 16, both sizes < 2^31) with 128-bit stores whose
 * values come from its loads, as a product stores its outputs after its
 * sums: the wall of a launch that reads a product's inputs and writes its
 * outputs.  1 <= groups <= 65536. */
int nvfp4_probe_stream_read_store(const void *buf, size_t rbytes, void *out, size_t obytes, int groups,
                                  hipStream_t stream);

/* A bare loop of v_mfma_f32_16x16x32_bf16: `groups` workgroups of
 * `waves` waves (1..16), each wave `iters` rounds of eight independent
 * accumulator chains.  Stores only if the sum hits a fixed value.
 * FLOPs of one launch: groups * waves * iters * 8 * 16384. */
int nvfp4_probe_mfma_bf16(int groups, int waves, int iters, float *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_PROBE_H */
