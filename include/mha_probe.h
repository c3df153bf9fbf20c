/*
 * mha_probe.h -- measurement aids of libmha (not part of the attention path).
 *
 * The short-sequence attention launch (the encoder block's 32 x 8 heads of
 * 100 queries) moves 13.1 MB in a few microseconds, where the fixed cost of
 * a launch is a large part of the time.  These two kernels give the floor
 * against which such a launch is judged, on the same stream and with the
 * same launch shape: a kernel that does nothing, and a kernel that does
 * nothing but move the same bytes.
 *
 *   kind MHA_PROBE_EMPTY: `grid` workgroups of 256 threads that return at once.
 *   kind MHA_PROBE_XOR3:  dst[i] = a[i] ^ b[i] ^ c[i] over `bytes` bytes
 *                         (16-byte chunks), i.e. reads 3 * bytes and writes
 *                         bytes, spread over `grid` workgroups of 256 threads.
 *
 * All pointers are caller-owned device memory, 16-byte aligned, each
 * holding `bytes` bytes (a, b, c, dst unused for MHA_PROBE_EMPTY);
 * `bytes` must be a positive multiple of 16 for MHA_PROBE_XOR3 and `grid`
 * in [1, 2^20].  Returns MHA_OK, or a negative MHA_ERR_* status (checked
 * on the host before any HIP call; MHA_ERR_HIP on a launch error).  Work
 * is enqueued on `stream`.
 *
 * mha_mfma_probe -- the dense bf16 matrix-core throughput the device
 * sustains as it runs (the shader clock under that load included, which the
 * nominal peak does not): `grid` workgroups of 256 threads (four waves),
 * each wave running four independent chains of `iters`
 * v_mfma_f32_32x32x16_bf16 (2 * 32 * 32 * 16 flops each) with no memory
 * traffic, then writing one float per thread to sink[grid][256] (every
 * workgroup writes the same 256 values).  flops per launch =
 * grid * 4 * 4 * iters * 32768.  The operands are fixed per lane: mode
 * MHA_PROBE_MFMA_DENSE, pseudo-random sign and mantissa bits with exponents
 * in [1/4, 2) (the bit activity of normally distributed data); mode
 * MHA_PROBE_MFMA_SPARSE, small multiples of 1/1024 (few set bits) -- the
 * products' power draw, and so the clock, depends on the operand bits.
 * sink: caller-owned device floats, 4-byte aligned; grid in [1, 2^20],
 * iters in [1, 2^24].  Returns MHA_OK, or MHA_ERR_UNSUPPORTED (unknown
 * mode, misaligned sink), MHA_ERR_DIM, MHA_ERR_NULL, checked on the host
 * before any HIP call, or MHA_ERR_HIP on a launch error.
 */
#ifndef MHA_PROBE_H
#define MHA_PROBE_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHA_PROBE_EMPTY 0
#define MHA_PROBE_XOR3 1
#define MHA_PROBE_MFMA_DENSE 0
#define MHA_PROBE_MFMA_SPARSE 1

int mha_floor_probe(int kind, const void* a, const void* b, const void* c, void* dst,
                    size_t bytes, int grid, hipStream_t stream);

/* mha_floor_probe with launch events: events[0], events[1] are recorded at
 * the start and end of the kernel's execution; *n_launches = 1. */
int mha_floor_probe_timed(int kind, const void* a, const void* b, const void* c, void* dst,
                          size_t bytes, int grid, hipStream_t stream, hipEvent_t* events,
                          int capacity, int* n_launches);

int mha_mfma_probe(int mode, int grid, int iters, float* sink, hipStream_t stream);

/* mha_mfma_probe with launch events, as mha_floor_probe_timed. */
int mha_mfma_probe_timed(int mode, int grid, int iters, float* sink, hipStream_t stream,
                         hipEvent_t* events, int capacity, int* n_launches);

#ifdef __cplusplus
}
#endif

#endif /* MHA_PROBE_H */
