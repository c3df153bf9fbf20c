// Measurement aids declared in include/mha_probe.h: an empty kernel and a
// kernel that only moves bytes, launched like the attention kernels (256
// threads per workgroup, hipExtLaunchKernel with optional events), so that
// the fixed cost of a launch and the time to move a launch's bytes can be
// measured on the same stream, the same way, as the kernels they bound; and
// a kernel that only issues bf16 matrix products, for the dense throughput
// the matrix cores sustain on the device as it runs (its clock under that
// load included).
#include "kernels.h"
#include "../../include/mha_probe.h"

namespace mha {
namespace {

__global__ __launch_bounds__(256) void floor_empty_kernel() {}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// dst = a ^ b ^ c over n 16-byte chunks, grid-stride: each pass issues the
// three loads of a chunk before its store.
__global__ __launch_bounds__(256) void floor_xor3_kernel(const u32x4_t* __restrict__ a,
                                                         const u32x4_t* __restrict__ b,
                                                         const u32x4_t* __restrict__ c,
                                                         u32x4_t* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = a[i] ^ b[i] ^ c[i];
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Operand j (0..7) of lane l for the matrix-core probe.  mode 0: bf16 with
// pseudo-random sign and mantissa bits and exponents spanning [1/4, 2) (the
// bit activity of normally distributed data); mode 1: multiples of 1/1024
// below 1/64 (few set bits).  The operand values change how much power the
// products draw, and so the clock the device holds.
__host__ __device__ inline unsigned short probe_operand_bits(int mode, int l, int j, int which) {
  if (mode == 1) {
    const int v = which == 0 ? ((l + j) & 15) : ((3 * l + j) & 15);  // v / 1024 in bf16
    if (v == 0) return 0;
    int e = 0;
    while ((v >> e) > 1) ++e;                                         // v = 2^e * (1 + f)
    const unsigned mant = ((unsigned)v << (7 - e)) & 0x7fu;
    return (unsigned short)(((unsigned)(127 - 10 + e) << 7) | mant);
  }
  unsigned x = (unsigned)(l * 64 + j * 8 + which) * 2654435761u;
  x ^= x >> 15;
  x *= 2246822519u;
  x ^= x >> 13;
  const unsigned sign = (x >> 31) & 1u;
  const unsigned expo = 125u + ((x >> 7) % 3u);   // 2^-2 .. 2^0
  return (unsigned short)((sign << 15) | (expo << 7) | (x & 0x7fu));
}

// Four independent chains of `iters` v_mfma_f32_32x32x16_bf16 per wave (no
// memory traffic between the first and the last instruction); one float per
// thread written so that the chains stay live.  Every workgroup computes the
// same values.
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ sink, int iters, int mode) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(__bf16, probe_operand_bits(mode, lane, i, 0));
    b[i] = __builtin_bit_cast(__bf16, probe_operand_bits(mode, lane, i, 1));
  }
  f32x16_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

int mfma_probe_impl(int mode, int grid, int iters, float* sink, hipStream_t stream, LaunchEvents ev) {
  if (mode != 0 && mode != 1) return MHA_ERR_UNSUPPORTED;
  if (grid < 1 || grid > (1 << 20) || iters < 1 || iters > (1 << 24)) return MHA_ERR_DIM;
  if (!sink) return MHA_ERR_NULL;
  if (((uintptr_t)sink & 3u) != 0) return MHA_ERR_UNSUPPORTED;
  void* args[] = {(void*)&sink, (void*)&iters, (void*)&mode};
  const hipError_t e = launch_kernel((const void*)probe_mfma_kernel, dim3(grid), dim3(256), args, 0, stream,
                                     ev.start, ev.stop, 0);
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

int probe_impl(int kind, const void* a, const void* b, const void* c, void* dst, size_t bytes,
               int grid, hipStream_t stream, LaunchEvents ev) {
  if (grid < 1 || grid > (1 << 20)) return MHA_ERR_DIM;
  hipError_t e;
  if (kind == MHA_PROBE_EMPTY) {
    e = launch_kernel((const void*)floor_empty_kernel, dim3(grid), dim3(256), nullptr, 0, stream,
                           ev.start, ev.stop, 0);
  } else if (kind == MHA_PROBE_XOR3) {
    if (!a || !b || !c || !dst) return MHA_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0) return MHA_ERR_DIM;
    if ((((uintptr_t)a | (uintptr_t)b | (uintptr_t)c | (uintptr_t)dst) & 15u) != 0) return MHA_ERR_UNSUPPORTED;
    int64_t n = (int64_t)(bytes / 16);
    void* args[] = {(void*)&a, (void*)&b, (void*)&c, (void*)&dst, (void*)&n};
    e = launch_kernel((const void*)floor_xor3_kernel, dim3(grid), dim3(256), args, 0, stream,
                           ev.start, ev.stop, 0);
  } else {
    return MHA_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

}  // namespace
}  // namespace mha

extern "C" int mha_floor_probe(int kind, const void* a, const void* b, const void* c, void* dst,
                               size_t bytes, int grid, hipStream_t stream) {
  return mha::probe_impl(kind, a, b, c, dst, bytes, grid, stream, {});
}

extern "C" int mha_floor_probe_timed(int kind, const void* a, const void* b, const void* c, void* dst,
                                     size_t bytes, int grid, hipStream_t stream, hipEvent_t* events,
                                     int capacity, int* n_launches) {
  if (events == nullptr || capacity < 2 || events[0] == nullptr || events[1] == nullptr)
    return MHA_ERR_EVENTS;
  mha::LaunchEvents ev;
  ev.start = events[0];
  ev.stop = events[1];
  const int st = mha::probe_impl(kind, a, b, c, dst, bytes, grid, stream, ev);
  if (n_launches) *n_launches = st == MHA_OK ? 1 : 0;
  return st;
}

extern "C" int mha_mfma_probe(int mode, int grid, int iters, float* sink, hipStream_t stream) {
  return mha::mfma_probe_impl(mode, grid, iters, sink, stream, {});
}

extern "C" int mha_mfma_probe_timed(int mode, int grid, int iters, float* sink, hipStream_t stream,
                                    hipEvent_t* events, int capacity, int* n_launches) {
  if (events == nullptr || capacity < 2 || events[0] == nullptr || events[1] == nullptr)
    return MHA_ERR_EVENTS;
  mha::LaunchEvents ev;
  ev.start = events[0];
  ev.stop = events[1];
  const int st = mha::mfma_probe_impl(mode, grid, iters, sink, stream, ev);
  if (n_launches) *n_launches = st == MHA_OK ? 1 : 0;
  return st;
}
