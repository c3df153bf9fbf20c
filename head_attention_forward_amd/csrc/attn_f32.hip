// Fused scaled dot-product attention, forward, fp32 in / fp32 out, head
// size 64, for gfx950.  Same definition and streaming row softmax as the
// bf16 kernel (devpress.csdn.net "【深度学习】Transformer", section 2.1,
// equation (2.4); hex4c59.cc "读懂 Attention Is All You Need", section
// "掩码必须在 softmax 之前生效" for the mask), with no reduced-precision step:
// fp32 products on the vector ALU and the accurate expf.
//
// One thread owns one query row (its q and accumulator live in registers);
// a workgroup of 128 threads shares 32-key K and V tiles in LDS, read as
// wave-wide broadcasts.
#include "kernels.h"

#include <math.h>

namespace mha {
namespace {

constexpr int D = 64;
constexpr int QB = 128;  // queries per workgroup (one per thread)
constexpr int KT = 32;   // keys per tile

__global__ __launch_bounds__(QB) void attn_fwd_f32_d64_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float Ks[KT * D];
  __shared__ __attribute__((aligned(16))) float Vs[KT * D];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.h;
  const int hh = bh - b * a.h;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int q0 = qt * QB;
  const int my_q = q0 + tid;

  const float* Qp = (const float*)a.Q + b * a.q_sb + hh * a.q_sh;
  const float* Kp = (const float*)a.K + b * a.k_sb + hh * a.k_sh;
  const float* Vp = (const float*)a.V + b * a.v_sb + hh * a.v_sh;
  float* Op = (float*)a.O + b * a.o_sb + hh * a.o_sh;

  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int wg_last = min(q0 + QB, a.n_q) - 1;
  const int wg_keys = a.causal ? min(L, wg_last + 1) : L;
  const int lim = (my_q < a.n_q) ? (a.causal ? min(L, my_q + 1) : L) : 0;

  float q[D];
  if (my_q < a.n_q) {
    const float4* src = (const float4*)(Qp + (int64_t)my_q * a.q_sr);
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      const float4 v = src[j];
      q[4 * j] = v.x; q[4 * j + 1] = v.y; q[4 * j + 2] = v.z; q[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) q[j] = 0.f;
  }

  float acc[D];
#pragma unroll
  for (int j = 0; j < D; ++j) acc[j] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int k0 = 0; k0 < wg_keys; k0 += KT) {
    __syncthreads();
    for (int c = tid; c < KT * D / 4; c += QB) {
      const int key = k0 + c / (D / 4);
      const int dc = c % (D / 4);
      float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < a.n_k) {
        kv = *(const float4*)(Kp + (int64_t)key * a.k_sr + 4 * dc);
        vv = *(const float4*)(Vp + (int64_t)key * a.v_sr + 4 * dc);
      }
      *(float4*)&Ks[4 * c] = kv;
      *(float4*)&Vs[4 * c] = vv;
    }
    __syncthreads();
    if (k0 >= lim) continue;  // every key of this tile is hidden from this query

    float s[KT];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], Ks[j * D + d], dot);
      s[j] = (k0 + j < lim) ? dot * a.scale : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = expf(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vs[j * D + d], acc[d]);
    }
  }

  if (my_q < a.n_q) {
    float* orow = Op + (int64_t)my_q * a.o_sr;
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      float4 v;
      v.x = acc[4 * j] / l; v.y = acc[4 * j + 1] / l; v.z = acc[4 * j + 2] / l; v.w = acc[4 * j + 3] / l;
      *(float4*)(orow + 4 * j) = v;
    }
  }
}

}  // namespace

hipError_t launch_attn_f32_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  const int nqt = (a.n_q + QB - 1) / QB;
  dim3 grid(a.B * a.h, nqt);
  void* args[] = {(void*)&a};
  return hipExtLaunchKernel((const void*)attn_fwd_f32_d64_kernel, grid, dim3(QB), args, 0, s, ev.start,
                            ev.stop, 0);
}

}  // namespace mha
