// Dense bf16 matrix transpose, dst[c][r] = src[r][c], for gfx950.  The
// gradients of the projections X W need X^T and W^T as row-major operands of
// the projection GEMM (dW = X^T dY, dX = dY W^T); this kernel materialises
// them.
//
// One workgroup per 64 x 64 tile: 256 threads read the tile as 16-byte row
// chunks (rows 32 apart per thread), store it in LDS with the row padded by
// one element pair, and write the transposed tile as 16-byte chunks of
// eight consecutive source rows.  Bandwidth-bound; R and C multiples of 8.
#include "device.h"

namespace mha {
namespace {

using namespace dev;

constexpr int TB = 64;          // tile rows and columns
constexpr int LD = TB + 2;      // LDS row length (elements): 132 bytes, odd word count

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const __bf16* __restrict__ src,
                                                             __bf16* __restrict__ dst, int R, int C) {
  __shared__ __bf16 t[TB * LD];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.y * TB, c0 = blockIdx.x * TB;
  const int cc = (tid & 7) * 8;  // chunk column within the tile
  // read: thread covers rows (tid >> 3) and (tid >> 3) + 32, 8 columns each
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = (tid >> 3) + 32 * i;
    bf16x8 v = {};
    if (r0 + rr < R && c0 + cc < C) v = *(const bf16x8*)(src + (int64_t)(r0 + rr) * C + c0 + cc);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[rr * LD + cc + e] = v[e];
  }
  __syncthreads();
  // write: output row c0 + oc holds source column oc; 8 consecutive source rows
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int oc = (tid >> 3) + 32 * i;
    const int rr = (tid & 7) * 8;
    if (c0 + oc < C && r0 + rr < R) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = t[(rr + e) * LD + oc];
      *(bf16x8*)(dst + (int64_t)(c0 + oc) * R + r0 + rr) = v;
    }
  }
}

}  // namespace

hipError_t launch_transpose_bf16(const void* src, void* dst, int R, int C, hipStream_t s, LaunchEvents ev) {
  if (R <= 0 || C <= 0 || R % 8 != 0 || C % 8 != 0) return hipErrorInvalidValue;
  const __bf16* sp = (const __bf16*)src;
  __bf16* dp = (__bf16*)dst;
  void* args[] = {(void*)&sp, (void*)&dp, (void*)&R, (void*)&C};
  dim3 grid((C + TB - 1) / TB, (R + TB - 1) / TB);
  if (grid.y > 65535) return hipErrorInvalidValue;
  return hipExtLaunchKernel((const void*)transpose_bf16_kernel, grid, dim3(256), args, 0, s, ev.start,
                            ev.stop, 0);
}

}  // namespace mha
