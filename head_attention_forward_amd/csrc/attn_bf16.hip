// Fused scaled dot-product attention, forward, bf16 in / bf16 out, fp32
// accumulation, head size 64, for gfx950 (CDNA4).
//
// Computes, per (batch, head), O = softmax(Q K^T * scale + M) V without ever
// storing the n_q x n_k score matrix.  Definition: devpress.csdn.net
// "【深度学习】Transformer", section 2.1, equation (2.4); hex4c59.cc "读懂
// Attention Is All You Need", sections "六步算完一行注意力" and
// "把所有位置合并，就是那条核心公式".  Mask M (0 / -inf, added before the
// softmax): hex4c59.cc, section "掩码必须在 softmax 之前生效".
//
// The row softmax is evaluated in streaming form over key tiles: a running
// row maximum m, a running sum l of exp(s - m) and an accumulator of
// exp(s - m) v are rescaled by exp(m_old - m_new) whenever the maximum grows,
// and O = acc / l at the end.  This is an exact rewrite of the row softmax
// (the shift by the row maximum does not change the result; hex4c59.cc,
// section "用几十行代码核对刚才的数值").  Masked keys are never added: a
// partially visible tile sets their scores to -inf (weight exactly 0), a
// tile with no visible key is skipped, which is what -inf before the
// softmax means.
//
// Work decomposition
//   workgroup = NW waves = NW*32 consecutive queries of one (batch, head);
//   grid.x = batch*heads (fastest, so consecutive workgroups of one head
//   land on the same XCD when batch*heads is a multiple of 8 and share its
//   L2), grid.y = query tiles, heaviest causal tiles dispatched first.
//   Per wave, per 64-key tile:
//     S^T[64 keys x 32 queries] = K_tile . Q^T       (8 MFMA 32x32x16)
//     online softmax on S^T: each lane owns one query and 32 of its 64
//     scores; the other 32 sit in lane ^ 32 (one cross-lane max per tile,
//     one cross-lane sum at the end)
//     O^T[64 d x 32 queries] += V_tile^T . P^T         (8 MFMA 32x32x16)
//   Computing the transposed products keeps every accumulator element of a
//   lane on that lane's own query, so rescaling and the final division are
//   per-lane scalars, and P^T leaves the first MFMA already in the B-operand
//   layout of the second: the MFMA output rows of lane group g are keys
//   {8j + 4g + r}, and the V^T operand is read with the same key order.
//   K is staged in LDS as [key][d] (row stride 144 B), V transposed as
//   [d][key] (row stride 144 B); the next tile is prefetched into registers
//   while the current one is computed.
#include "kernels.h"

#include <math.h>

namespace mha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 64;        // head size (d_k = d_v)
constexpr int QW = 32;       // queries per wave
constexpr int KT = 64;       // keys per tile
constexpr int KLD = D + 8;   // LDS row stride of the K tile, elements
constexpr int VLD = KT + 8;  // LDS row stride of the V^T tile, elements

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ bf16x8 to_bf16x8(f32x16 v, int half) {
  f32x8 t;
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = v[8 * half + j];
  return __builtin_convertvector(t, bf16x8);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_d64_kernel(const AttnArgs a) {
  static_assert(NW == 2 || NW == 4, "tile loaders assume 128 or 256 threads");
  constexpr int NT = NW * 64;
  constexpr int KCH = (KT * D / 8) / NT;        // 16-byte K chunks per thread
  constexpr int VCH = (KT / 2) * (D / 8) / NT;  // (2 keys x 16 bytes) V chunks per thread

  __shared__ __attribute__((aligned(16))) __bf16 Ks[KT * KLD];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int g = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / a.h;
  const int hh = bh - b * a.h;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int q0 = qt * (NW * QW);
  const int qw0 = q0 + wave * QW;
  const int my_q = qw0 + col;

  const __bf16* Qp = (const __bf16*)a.Q + b * a.q_sb + hh * a.q_sh;
  const __bf16* Kp = (const __bf16*)a.K + b * a.k_sb + hh * a.k_sh;
  const __bf16* Vp = (const __bf16*)a.V + b * a.v_sb + hh * a.v_sh;
  __bf16* Op = (__bf16*)a.O + b * a.o_sb + hh * a.o_sh;

  // Visible keys: j < L for every query (padding), and j <= i when causal.
  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int wg_last = min(q0 + NW * QW, a.n_q) - 1;
  const int wv_last = min(qw0 + QW, a.n_q) - 1;
  const int wg_keys = a.causal ? min(L, wg_last + 1) : L;
  const int wv_keys = (wv_last < qw0) ? 0 : (a.causal ? min(L, wv_last + 1) : L);
  const int lim = a.causal ? min(L, my_q + 1) : L;  // >= 1 for every lane

  // Q^T as the B operand of S^T = K Q^T: lane (col, g) holds Q[q][16s+8g .. +7].
  bf16x8 qf[4];
  if (my_q < a.n_q) {
    const bf16x8* src = (const bf16x8*)(Qp + (int64_t)my_q * a.q_sr);
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = src[2 * s + g];
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = bf16x8{};
  }

  u32x4 kreg[KCH];
  u32x4 vreg[VCH][2];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + r * NT;
      const int key = k0 + (c >> 3);
      const int dc = c & 7;
      kreg[r] = key < a.n_k ? *(const u32x4*)(Kp + (int64_t)key * a.k_sr + dc * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int p = tid + r * NT;
      const int key = k0 + 2 * (p & 31);
      const int dc = p >> 5;
      vreg[r][0] = key < a.n_k ? *(const u32x4*)(Vp + (int64_t)key * a.v_sr + dc * 8) : u32x4{0, 0, 0, 0};
      vreg[r][1] = key + 1 < a.n_k ? *(const u32x4*)(Vp + (int64_t)(key + 1) * a.v_sr + dc * 8)
                                   : u32x4{0, 0, 0, 0};
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + r * NT;
      *(u32x4*)&Ks[(c >> 3) * KLD + (c & 7) * 8] = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int p = tid + r * NT;
      const int kp = p & 31;
      const int dc = p >> 5;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned x0 = vreg[r][0][j];  // V[2kp][8dc+2j], V[2kp][8dc+2j+1]
        const unsigned x1 = vreg[r][1][j];  // V[2kp+1][...]
        const unsigned even = (x0 & 0xffffu) | (x1 << 16);
        const unsigned odd = (x0 >> 16) | (x1 & 0xffff0000u);
        *(unsigned*)&Vt[(8 * dc + 2 * j) * VLD + 2 * kp] = even;
        *(unsigned*)&Vt[(8 * dc + 2 * j + 1) * VLD + 2 * kp] = odd;
      }
    }
  };

  const float c2 = a.scale * 1.4426950408889634f;  // scale * log2(e)
  float m = -INFINITY;  // running max of raw q.k for this lane's query
  float l = 0.f;        // this lane's share of the running row sum
  f32x16 o0 = {}, o1 = {};

  const int ntiles = (wg_keys + KT - 1) / KT;
  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * KT;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(k0 + KT);
    if (k0 >= wv_keys) continue;  // no visible key for any query of this wave

    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 ka = *(const bf16x8*)&Ks[col * KLD + 16 * ks + 8 * g];
      const bf16x8 kb = *(const bf16x8*)&Ks[(32 + col) * KLD + 16 * ks + 8 * g];
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[ks], s1, 0, 0, 0);
    }
    // s0[i] is the score of key k0 + 8(i/4) + 4g + i%4, s1[i] of that key + 32.
    if (k0 + KT > lim) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= lim) s0[i] = -INFINITY;
        if (key + 32 >= lim) s1[i] = -INFINITY;
      }
    }
    float mt = s0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s1[i]);
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m, mt);
    const float alpha = fast_exp2((m - m_new) * c2);  // 0 on the first visible tile
    m = m_new;
    const float mc = m_new * c2;
    l *= alpha;
    o0 *= alpha;
    o1 *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = fast_exp2(fmaf(s0[i], c2, -mc));
      s1[i] = fast_exp2(fmaf(s1[i], c2, -mc));
      l += s0[i] + s1[i];
    }
    // P^T blocks as B operands: p{kb}{hf} covers keys k0 + 32kb + 16hf + {4g+r, 8+4g+r}.
    const bf16x8 p00 = to_bf16x8(s0, 0), p01 = to_bf16x8(s0, 1);
    const bf16x8 p10 = to_bf16x8(s1, 0), p11 = to_bf16x8(s1, 1);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const __bf16* vrow = &Vt[(32 * db + col) * VLD + 4 * g];
      f32x16 acc = db == 0 ? o0 : o1;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x4 lo = *(const bf16x4*)(vrow + 16 * kk);
        const bf16x4 hi = *(const bf16x4*)(vrow + 16 * kk + 8);
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 pb = kk == 0 ? p00 : kk == 1 ? p01 : kk == 2 ? p10 : p11;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc, 0, 0, 0);
      }
      if (db == 0) o0 = acc; else o1 = acc;
    }
  }

  l += xor32(l);
  const float inv = 1.f / l;
  if (my_q < a.n_q) {
    __bf16* orow = Op + (int64_t)my_q * a.o_sr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 v0, v1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v0[r] = o0[4 * j + r] * inv;
        v1[r] = o1[4 * j + r] * inv;
      }
      // o_db[4j + r] is O[q][32db + 8j + 4g + r].
      *(bf16x4*)(orow + 8 * j + 4 * g) = __builtin_convertvector(v0, bf16x4);
      *(bf16x4*)(orow + 32 + 8 * j + 4 * g) = __builtin_convertvector(v1, bf16x4);
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16_d64(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = 4;
  const int nqt = (a.n_q + NW * QW - 1) / (NW * QW);
  dim3 grid(a.B * a.h, nqt);
  void* args[] = {(void*)&a};
  return hipLaunchKernel((const void*)attn_fwd_bf16_d64_kernel<NW>, grid, dim3(NW * 64), args, 0, s);
}

}  // namespace mha
