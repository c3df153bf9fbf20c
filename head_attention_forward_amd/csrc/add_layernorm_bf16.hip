// Residual + LayerNorm (the Post-LN sublayer wrapper), bf16 in / bf16 out,
// fp32 arithmetic, for gfx950:
//
//   u = x + F(x),  y = gamma * (u - mean(u)) / sqrt(var(u) + eps) + beta
//
// per row, mean and (population) variance over the row's d features
// (hex4c59.cc "读懂 Attention Is All You Need", section "Add & Norm 里究竟
// 发生了什么？": the sublayer output is added back to its input and the sum is
// normalised over one token's features, then scaled and shifted per
// feature; devpress.csdn.net "【深度学习】Transformer", section 2.3, the
// encoder block's x + sublayer(x) followed by the norm).
//
// One wave per row: lane l holds the 16-byte chunks l, l + 64, ... of the
// row (8 features each, CH chunks per lane), so every load and store is a
// fully coalesced 1 KB wave access.  The row stays in registers between the
// two reductions (sum, then the sum of squared deviations -- the two-pass
// variance, no cancellation) and the normalised write, so Y may be the same
// buffer as X or F.  Bandwidth-bound: per row 2 d bytes read from each input,
// 2 d written.
#include "device.h"

namespace mha {
namespace {

using namespace dev;

constexpr int kRowsPerBlock = 4;  // waves per workgroup, one row each

// Butterfly sum over the 64 lanes: every lane adds the same two partial sums
// at each step (in commuted order), so all lanes end with the same value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int CH>
__global__ __launch_bounds__(64 * kRowsPerBlock) void add_layernorm_bf16_kernel(const LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const int nch = a.d >> 3;  // 16-byte chunks per row
  const int64_t base = (int64_t)row * a.d;
  const __bf16* X = (const __bf16*)a.X + base;
  const __bf16* F = (const __bf16*)a.F + base;

  // Every load of the row (inputs, gamma, beta) is issued before the first
  // use, so their latencies overlap.  Chunks past the row read chunk 0.
  bf16x8 xv[CH], fv[CH], gv[CH], bv[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j < nch ? lane + 64 * j : 0;
    xv[j] = *(const bf16x8*)(X + 8 * c);
    fv[j] = *(const bf16x8*)(F + 8 * c);
    gv[j] = *(const bf16x8*)((const __bf16*)a.gamma + 8 * c);
    bv[j] = *(const bf16x8*)((const __bf16*)a.beta + 8 * c);
  }
  float u[CH][8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const bool in = lane + 64 * j < nch;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u[j][e] = in ? (float)xv[j][e] + (float)fv[j][e] : 0.f;
      s += u[j][e];
    }
  }
  const float inv_d = 1.0f / (float)a.d;
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (lane + 64 * j < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u[j][e] -= mean;
        q += u[j][e] * u[j][e];
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_d + a.eps);

  __bf16* Y = (__bf16*)a.Y + base;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      f32x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (float)gv[j][e] * (u[j][e] * rstd) + (float)bv[j][e];
      *(bf16x8*)(Y + 8 * c) = __builtin_convertvector(y, bf16x8);
    }
  }
}

template <int CH>
hipError_t launch_ch(const LnArgs& a, hipStream_t s, LaunchEvents ev) {
  void* args[] = {(void*)&a};
  const int blocks = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
  return launch_kernel((const void*)add_layernorm_bf16_kernel<CH>, dim3(blocks),
                            dim3(64 * kRowsPerBlock), args, 0, s, ev.start, ev.stop, 0);
}

}  // namespace

hipError_t launch_add_layernorm_bf16(const LnArgs& a, hipStream_t s, LaunchEvents ev) {
  if (a.d <= 0 || a.d % 8 != 0 || a.d > kLnMaxWidth || a.M <= 0) return hipErrorInvalidValue;
  const int chunks = (a.d / 8 + 63) / 64;  // chunks per lane
  if (chunks <= 1) return launch_ch<1>(a, s, ev);
  if (chunks <= 2) return launch_ch<2>(a, s, ev);
  if (chunks <= 4) return launch_ch<4>(a, s, ev);
  return launch_ch<8>(a, s, ev);
}

}  // namespace mha
