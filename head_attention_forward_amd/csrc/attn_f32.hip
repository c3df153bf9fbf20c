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
//
// Launches too small to give every compute unit a workgroup that way (the
// single-head 64-query shape, for one) take a second kernel with a whole
// wave per query instead: lane j scores key j of the tile, the wave reduces
// the tile's maximum and sum across lanes, and lane d accumulates output
// column d -- about a tenth of the other kernel's vector instructions per
// wave, so the launch's one round of waves finishes sooner.
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

// Maximum and sum over the 64 lanes of a wave (butterfly over lane ^ 1 ..
// lane ^ 32; every lane ends with the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

constexpr int SQ = 4;  // waves (queries) per workgroup of the one-wave-per-query kernel

// One wave per query.  The workgroup's SQ waves take consecutive queries of
// one (batch, head) and share each 64-key K and V tile in LDS.  Per tile,
// lane j forms the score of key k0 + j (four partial sums over d, so that
// the products do not wait on each other), the wave takes the tile's
// maximum, rescales its running sum and accumulator (the streaming softmax
// of the other kernel, per tile instead of per lane), and lane d adds
// sum_j p_j V[k0 + j][d] with the weights p_j passed through LDS.
__global__ __launch_bounds__(SQ * 64) void attn_fwd_f32_d64_wave_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float Ks[KT * RS];
  __shared__ __attribute__((aligned(16))) float Vs[KT * D];
  __shared__ __attribute__((aligned(16))) float Ps[SQ][KT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x;
  const int b = bh / a.h;
  const int hh = bh - b * a.h;
  const int q0 = (int)blockIdx.y * SQ;
  const int my_q = q0 + wave;
  const bool active = my_q < a.n_q;  // wave-uniform
  const int qc = min(my_q, a.n_q - 1);

  const float* Qp = (const float*)a.Q + b * a.q_sb + hh * a.q_sh;
  const float* Kp = (const float*)a.K + b * a.k_sb + hh * a.k_sh;
  const float* Vp = (const float*)a.V + b * a.v_sb + hh * a.v_sh;
  float* Op = (float*)a.O + b * a.o_sb + hh * a.o_sh;

  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int wg_last = min(q0 + SQ, a.n_q) - 1;
  const int wg_keys = a.causal ? min(L, wg_last + 1) : L;
  const int lim = a.causal ? min(L, qc + 1) : L;

  // The query row in every lane (all lanes read the same 256 bytes).
  float q[D];
  {
    const float4* src = (const float4*)(Qp + (int64_t)qc * a.q_sr);
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      const float4 v = src[j];
      q[4 * j] = v.x; q[4 * j + 1] = v.y; q[4 * j + 2] = v.z; q[4 * j + 3] = v.w;
    }
  }

  float m = -INFINITY, l = 0.f, acc = 0.f;  // acc: output column `lane`
  for (int k0 = 0; k0 < wg_keys; k0 += KT) {
    __syncthreads();  // every wave is done with the previous tile
    for (int c = tid; c < KT * D / 4; c += SQ * 64) {
      const int row = c / (D / 4);
      const int dc = c % (D / 4);
      const int key = min(k0 + row, a.n_k - 1);  // rows past n_k: never visible
      *(float4*)&Ks[row * RS + 4 * dc] = *(const float4*)(Kp + (int64_t)key * a.k_sr + 4 * dc);
      *(float4*)&Vs[row * D + 4 * dc] = *(const float4*)(Vp + (int64_t)key * a.v_sr + 4 * dc);
    }
    __syncthreads();
    if (!active || k0 >= lim) continue;  // wave-uniform: no visible key in this tile

    float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
    const float* krow = &Ks[lane * RS];
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const float4 kv = *(const float4*)&krow[d];
      d0 = fmaf(q[d], kv.x, d0);
      d1 = fmaf(q[d + 1], kv.y, d1);
      d2 = fmaf(q[d + 2], kv.z, d2);
      d3 = fmaf(q[d + 3], kv.w, d3);
    }
    const bool vis = k0 + lane < lim;
    const float sc = vis ? ((d0 + d1) + (d2 + d3)) * a.scale : -INFINITY;
    const float m_new = fmaxf(m, wave_max(sc));  // finite: key k0 is visible
    const float alpha = expf(m - m_new);         // exp(-inf) = 0 on the first visible tile
    const float p = vis ? expf(sc - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
    m = m_new;
    Ps[wave][lane] = p;  // this wave's weights, read back by every lane below
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int j = 0; j < KT; j += 4) {
      const float4 pw = *(const float4*)&Ps[wave][j];
      a0 = fmaf(pw.x, Vs[j * D + lane], a0);
      a1 = fmaf(pw.y, Vs[(j + 1) * D + lane], a1);
      a2 = fmaf(pw.z, Vs[(j + 2) * D + lane], a2);
      a3 = fmaf(pw.w, Vs[(j + 3) * D + lane], a3);
    }
    acc = acc * alpha + ((a0 + a1) + (a2 + a3));
  }
  if (active) Op[(int64_t)my_q * a.o_sr + lane] = acc / l;
}

}  // namespace

hipError_t launch_attn_f32_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  void* args[] = {(void*)&a};
  const int nqt = (a.n_q + QB - 1) / QB;
  // Fewer 32-query workgroups than compute units: one wave per query.
  if ((int64_t)a.B * a.h * nqt < device_compute_units()) {
    dim3 grid(a.B * a.h, (a.n_q + SQ - 1) / SQ);
    return launch_kernel((const void*)attn_fwd_f32_d64_wave_kernel, grid, dim3(SQ * 64), args, 0, s,
                         ev.start, ev.stop, 0);
  }
  dim3 grid(a.B * a.h, nqt);
  return launch_kernel((const void*)attn_fwd_f32_d64_kernel, grid, dim3(NT), args, 0, s, ev.start,
                            ev.stop, 0);
}

}  // namespace mha
