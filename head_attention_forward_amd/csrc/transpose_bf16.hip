// Dense bf16 matrix transpose, dst[c][r] = src[r][c], for gfx950.  The
// gradients of the projections X W need X^T and W^T as row-major operands of
// the projection GEMM (dW = X^T dY, dX = dY W^T); this kernel materialises
// them.
//
// Up to eight matrices per launch (grid.z).  One workgroup per 64 x 64
// tile: 256 threads read the tile as 16-byte row chunks (rows 32 apart per
// thread), store it in LDS with the row padded by one element pair, and
// write the transposed tile as 16-byte chunks of eight consecutive source
// rows.  Bandwidth-bound; R and C multiples of 8.
#include "device.h"

namespace mha {
namespace {

using namespace dev;

constexpr int TB = 64;          // tile rows and columns
constexpr int LD = TB + 2;      // LDS row length (elements): 132 bytes, odd word count

// Matrix z of a batched launch: blockIdx.z selects it (by selects on the
// uniform z, so the argument block is never indexed dynamically); workgroups
// past its tiles return at once (the grid covers the largest matrix).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const TransposeBatch tb) {
  __shared__ __bf16 t[TB * LD];
  const int z = blockIdx.z;
  const void* sp = tb.src[0];
  void* dp = tb.dst[0];
  int R = tb.R[0], C = tb.C[0];
#pragma unroll
  for (int i = 1; i < kMaxTransposeBatch; ++i)
    if (z == i) {
      sp = tb.src[i];
      dp = tb.dst[i];
      R = tb.R[i];
      C = tb.C[i];
    }
  const __bf16* __restrict__ src = (const __bf16*)sp;
  __bf16* __restrict__ dst = (__bf16*)dp;
  const int tid = threadIdx.x;
  const int r0 = blockIdx.y * TB, c0 = blockIdx.x * TB;
  if (r0 >= R || c0 >= C) return;  // whole workgroup: no barrier is skipped by part of it
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

hipError_t launch_transpose_bf16(const TransposeBatch& tb, hipStream_t s, LaunchEvents ev) {
  if (tb.n < 1 || tb.n > kMaxTransposeBatch) return hipErrorInvalidValue;
  int maxR = 0, maxC = 0;
  for (int i = 0; i < tb.n; ++i) {
    if (tb.R[i] <= 0 || tb.C[i] <= 0 || tb.R[i] % 8 != 0 || tb.C[i] % 8 != 0) return hipErrorInvalidValue;
    maxR = max(maxR, tb.R[i]);
    maxC = max(maxC, tb.C[i]);
  }
  dim3 grid((maxC + TB - 1) / TB, (maxR + TB - 1) / TB, tb.n);
  if (grid.y > 65535) return hipErrorInvalidValue;
  void* args[] = {(void*)&tb};
  return launch_kernel((const void*)transpose_bf16_kernel, grid, dim3(256), args, 0, s, ev.start,
                            ev.stop, 0);
}

}  // namespace mha
