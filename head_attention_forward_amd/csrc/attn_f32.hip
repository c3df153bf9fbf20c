// Fused scaled dot-product attention, forward, fp32 in / fp32 out, head
// size 64, for gfx950.  Same definition and streaming row softmax as the
// bf16 kernel (devpress.csdn.net "【深度学习】Transformer", section 2.1,
// equation (2.4); hex4c59.cc "读懂 Attention Is All You Need", section
// "掩码必须在 softmax 之前生效" for the mask), with no reduced-precision step:
// fp32 products on the vector ALU and the accurate expf.
//
// Eight lanes share one query row: lane r of the group streams keys r, r + 8,
// r + 16, ... with its own running maximum, sum and accumulator, and the
// eight partial softmaxes are merged at the end (for a common reference m,
// sum_r l_r e^(m_r - m) and sum_r acc_r e^(m_r - m) are the row's sum and
// accumulator).  A workgroup of 256 threads (32 queries) shares 64-key K and
// V tiles in LDS; rows are padded to 68 floats so that the keys a group
// reads at once fall in different banks.
#include "kernels.h"

#include <math.h>

namespace mha {
namespace {

constexpr int D = 64;
constexpr int SPLIT = 8;            // lanes per query
constexpr int QB = 32;              // queries per workgroup
constexpr int NT = QB * SPLIT;      // threads per workgroup
constexpr int KT = 64;              // keys per tile
constexpr int RS = D + 4;           // padded LDS row stride (floats)

// Sum and maximum over the 8 lanes of a group (lanes 8g .. 8g + 7) with DPP
// moves instead of LDS permutes: exchange with lane ^ 1, then lane ^ 2 (quad
// permutes), then the mirrored lane of the 8 (lane 7 - i, which after the
// first two steps holds the same value as lane i ^ 4).  The same additions
// in the same order as a butterfly over lane ^ 1, ^ 2, ^ 4.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141; // row_half_mirror
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp<kXor1>(v);
  v += dpp<kXor2>(v);
  return v + dpp<kHalfMirror>(v);
}
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp<kXor1>(v));
  v = fmaxf(v, dpp<kXor2>(v));
  return fmaxf(v, dpp<kHalfMirror>(v));
}
__global__ __launch_bounds__(NT) void attn_fwd_f32_d64_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float Ks[KT * RS];
  __shared__ __attribute__((aligned(16))) float Vs[KT * RS];

  const int tid = threadIdx.x;
  const int r = tid & (SPLIT - 1);  // this lane's key residue
  const int bh = blockIdx.x;
  const int b = bh / a.h;
  const int hh = bh - b * a.h;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int q0 = qt * QB;
  const int my_q = q0 + tid / SPLIT;

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
  float m = -INFINITY, l = 0.f;  // m stays -inf until this lane sees a key

  for (int k0 = 0; k0 < wg_keys; k0 += KT) {
    __syncthreads();
    for (int c = tid; c < KT * D / 4; c += NT) {
      const int row = c / (D / 4);
      const int dc = c % (D / 4);
      const int key = k0 + row;
      float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < a.n_k) {
        kv = *(const float4*)(Kp + (int64_t)key * a.k_sr + 4 * dc);
        vv = *(const float4*)(Vp + (int64_t)key * a.v_sr + 4 * dc);
      }
      *(float4*)&Ks[row * RS + 4 * dc] = kv;
      *(float4*)&Vs[row * RS + 4 * dc] = vv;
    }
    __syncthreads();
    if (k0 + r >= lim) continue;  // none of this lane's keys in the tile is visible

    float s[KT / SPLIT];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < KT / SPLIT; ++j) {
      const int row = SPLIT * j + r;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *(const float4*)&Ks[row * RS + d];
        dot = fmaf(q[d], kv.x, dot);
        dot = fmaf(q[d + 1], kv.y, dot);
        dot = fmaf(q[d + 2], kv.z, dot);
        dot = fmaf(q[d + 3], kv.w, dot);
      }
      s[j] = (k0 + row < lim) ? dot * a.scale : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    // mt is finite: key k0 + r is visible
    const float m_new = fmaxf(m, mt);
    const float alpha = expf(m - m_new);  // exp(-inf) = 0 on this lane's first visible tile
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < KT / SPLIT; ++j) {
      const int row = SPLIT * j + r;
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 vv = *(const float4*)&Vs[row * RS + d];
        acc[d] = fmaf(p, vv.x, acc[d]);
        acc[d + 1] = fmaf(p, vv.y, acc[d + 1]);
        acc[d + 2] = fmaf(p, vv.z, acc[d + 2]);
        acc[d + 3] = fmaf(p, vv.w, acc[d + 3]);
      }
    }
  }

  // Merge the eight partial softmaxes of the row (lanes of a group are
  // adjacent).  Lane 0 of every group sees key 0, so the merged m is finite.
  static_assert(SPLIT == 8, "the group reductions span 8 lanes");
  const float mg = group8_max(m);
  const float w = (m == -INFINITY) ? 0.f : expf(m - mg);
  const float lg = group8_sum(l * w);
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = group8_sum(acc[d] * w);

  if (my_q < a.n_q && r == 0) {
    float* orow = Op + (int64_t)my_q * a.o_sr;
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      float4 v;
      v.x = acc[4 * j] / lg; v.y = acc[4 * j + 1] / lg; v.z = acc[4 * j + 2] / lg; v.w = acc[4 * j + 3] / lg;
      *(float4*)(orow + 4 * j) = v;
    }
  }
}

}  // namespace

hipError_t launch_attn_f32_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  const int nqt = (a.n_q + QB - 1) / QB;
  dim3 grid(a.B * a.h, nqt);
  void* args[] = {(void*)&a};
  return launch_kernel((const void*)attn_fwd_f32_d64_kernel, grid, dim3(NT), args, 0, s, ev.start,
                            ev.stop, 0);
}

}  // namespace mha
