// Measurement aids declared in include/mha_probe.h: an empty kernel and a
// kernel that only moves bytes, launched like the attention kernels (256
// threads per workgroup, hipExtLaunchKernel with optional events), so that
// the fixed cost of a launch and the time to move a launch's bytes can be
// measured on the same stream, the same way, as the kernels they bound.
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
