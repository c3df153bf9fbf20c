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
// The row softmax is evaluated in streaming form over key tiles: every lane
// keeps a reference value m for its query, a running sum l of
// exp(s - m) and an accumulator of exp(s - m) v; O = acc / l at the end.
// Any finite m gives the same quotient (shifting every score of a row by the
// same amount does not change its softmax; hex4c59.cc, section
// "用几十行代码核对刚才的数值" subtracts the row maximum for the same
// reason), so a row's m is moved only when a tile's maximum exceeds it by
// more than 2^8 in weight -- then that row's acc and l are rescaled by
// exp(m_old - m_new).  Every weight stays below 2^8 and most tiles need no
// rescale.  Each row decides for itself, so a row's arithmetic depends only
// on the keys it can see.  Masked keys contribute exactly 0: a partially
// visible tile sets their scores to -inf, a tile with no visible key is
// skipped.
//
// Work decomposition
//   workgroup = NW waves, wave w owns the 32 queries q0 + 32w .. +31;
//   grid.x = batch*heads (fastest: the workgroups of one head land on the
//   same XCD when batch*heads is a multiple of 8 and share its L2),
//   grid.y = query tiles, heaviest causal tiles dispatched first.
//   Per wave and 64-key tile:
//     S^T[64 keys x 32 queries] = K_tile . Q^T     (8 MFMA 32x32x16)
//     O^T[64 d x 32 queries]   += V_tile^T . P^T   (8 MFMA 32x32x16)
//   The transposed products keep every accumulator element of a lane on
//   that lane's own query (lane = query, lane ^ 32 holds the other half of
//   its keys), so the softmax bookkeeping is per-lane scalar work with one
//   cross-half max per tile (v_permlane32_swap), and P^T leaves the first
//   MFMA already in the B-operand layout of the second: the MFMA output rows
//   of lane group g are keys {8j + 4g + r}, and the V^T operand is gathered
//   in that key order by transposing LDS reads (ds_read_b64_tr_b16) of the
//   row-major V tile.
//   K and V tiles go from global memory straight into LDS
//   (global_load_lds_dwordx4, no register staging) through a ring of NS tile
//   buffers, NS-1 tiles ahead of the one being computed; 16-byte chunks are
//   XOR-swizzled so that both LDS read patterns are conflict-free.  Without
//   staging registers a wave needs <= 128 VGPRs, so four waves share each
//   SIMD and one wave's softmax overlaps another's matrix products.
#include "kernels.h"

#include <math.h>

namespace mha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int D = 64;
constexpr int KT = 64;
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ int k_off(int r, int chunk) { return r * D + ((chunk ^ ((r >> 1) & 7)) << 3); }
__device__ __forceinline__ int v_off(int r, int chunk) { return r * D + ((chunk ^ (((r >> 1) & 1) << 2)) << 3); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ i16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}
// 16-byte global -> LDS copy per lane (lane l writes lds_base + 16 l).  Issued
// as inline assembly so that the compiler does not wait for it before every
// LDS read; the kernel waits for it explicitly (vmcnt) before the barrier that
// publishes the tile.
__device__ __forceinline__ void dma16(const void* src, const void* lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) char*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(src)
               : "memory", "m0");
}
// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Four waves per SIMD (<= 128 VGPRs); LDS allows it for NW * NS <= 16.
template <int NW, int NS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void attn_fwd_bf16_d64_kernel(const AttnArgs a) {
  constexpr int BLK = KT * D * 2 / 1024;  // 1 KB blocks per tile and matrix
  constexpr int CHW = BLK / NW;           // load instructions per wave, tile and matrix
  constexpr int QT = NW * 32;
  static_assert(CHW * NW == BLK, "waves must split the tile evenly");

  __shared__ __attribute__((aligned(1024))) __bf16 Ks[NS][KT * D];
  __shared__ __attribute__((aligned(1024))) __bf16 Vs[NS][KT * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int g = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / a.h;
  const int hh = bh - b * a.h;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int q0 = qt * QT;

  const __bf16* Qp = (const __bf16*)a.Q + b * a.q_sb + hh * a.q_sh;
  const __bf16* Kp = (const __bf16*)a.K + b * a.k_sb + hh * a.k_sh;
  const __bf16* Vp = (const __bf16*)a.V + b * a.v_sb + hh * a.v_sh;
  __bf16* Op = (__bf16*)a.O + b * a.o_sb + hh * a.o_sh;

  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int wg_last = min(q0 + QT, a.n_q) - 1;
  const int wg_keys = a.causal ? min(L, wg_last + 1) : L;
  const int qw0 = q0 + 32 * wave;
  const int my_q = qw0 + col;
  const int lim = a.causal ? min(L, my_q + 1) : L;
  const int wv_last = min(qw0 + 32, a.n_q) - 1;
  const int wv_keys =
      __builtin_amdgcn_readfirstlane(wv_last < qw0 ? 0 : (a.causal ? min(L, wv_last + 1) : L));
  const int ntiles = __builtin_amdgcn_readfirstlane((wg_keys + KT - 1) / KT);


  // Direct loads: instruction r of this wave fills LDS block (wave*CHW + r)
  // (8 rows); lane l writes 16-byte chunk l of it, i.e. row q >> 3, stored
  // chunk q & 7 with q = block*64 + l, which holds the source chunk that
  // the swizzle maps there.
  int drow[CHW], kcol[CHW], vcol[CHW];
#pragma unroll
  for (int r = 0; r < CHW; ++r) {
    const int q = (wave * CHW + r) * 64 + lane;
    drow[r] = q >> 3;
    kcol[r] = ((q & 7) ^ ((drow[r] >> 1) & 7)) * 8;
    vcol[r] = ((q & 7) ^ (((drow[r] >> 1) & 1) << 2)) * 8;
  }
  auto issue = [&](int tile, int buf) {
#pragma unroll
    for (int r = 0; r < CHW; ++r) {
      const int key = min(tile * KT + drow[r], a.n_k - 1);
      dma16(Kp + (int64_t)key * a.k_sr + kcol[r], &Ks[buf][(wave * CHW + r) * 512]);
      dma16(Vp + (int64_t)key * a.v_sr + vcol[r], &Vs[buf][(wave * CHW + r) * 512]);
    }
  };

  const float c2 = a.scale * 1.4426950408889634f;
  float m = -INFINITY;
  float l = 0.f;
  f32x16 o0 = {}, o1 = {};
  const int tr_key = ((lane & 15) >> 2) + 4 * g;
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, s);
  bf16x8 qf[4];
  {
    const bf16x8* src = (const bf16x8*)(Qp + (int64_t)min(my_q, a.n_q - 1) * a.q_sr);
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = src[2 * s + g];
  }
  wait_vmcnt<0>();  // Q fragment and the first tiles have landed

  int buf = 0;
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * KT;
    wait_vmcnt<(NS - 2) * 2 * CHW>();
    __syncthreads();
    {
      int nb = buf + NS - 1;
      if (nb >= NS) nb -= NS;
      issue(t + NS - 1, nb);
    }
    if (k0 < wv_keys) {
      const __bf16* ks = Ks[buf];
      const __bf16* vs = Vs[buf];
      f32x16 s0 = {}, s1 = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 ka = *(const bf16x8*)&ks[k_off(col, 2 * kk + g)];
        const bf16x8 kb = *(const bf16x8*)&ks[k_off(32 + col, 2 * kk + g)];
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[kk], s1, 0, 0, 0);
      }
      if (k0 + KT > lim) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= lim) s0[i] = -INFINITY;
          if (key + 32 >= lim) s1[i] = -INFINITY;
        }
      }
      float mt = fmaxf(s0[0], s0[1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) mt = fmaxf(mt, fmaxf(s0[i], s0[i + 1]));
#pragma unroll
      for (int i = 0; i < 16; i += 2) mt = fmaxf(mt, fmaxf(s1[i], s1[i + 1]));
      mt = max_halves(mt);
      const bool grow = (mt - m) * c2 > kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? fmaxf(m, mt) : m;
        const float alpha = m_new == m ? 1.f : fast_exp2((m - m_new) * c2);
        m = m_new;
        l *= alpha;
        o0 *= alpha;
        o1 *= alpha;
      }
      const float mc = m * c2;
      bf16x8 p[4];
      const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int hf = 0; hf < 4; ++hf) {
        f32x8 w;
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = fast_exp2(fmaf(hf < 2 ? s0[8 * hf + r] : s1[8 * (hf - 2) + r], c2, -mc));
        const bf16x8 pb = __builtin_convertvector(w, bf16x8);
        p[hf] = pb;
#pragma unroll
        for (int r = 0; r < 8; r += 2)
          l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[r], pb[r + 1]}, one, l, false);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = 16 * kk + tr_key;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int d = 32 * db + tr_d;
          const i16x4 lo = tr_read(&vs[v_off(key, d >> 3) + (d & 7)]);
          const i16x4 hi = tr_read(&vs[v_off(key + 8, d >> 3) + (d & 7)]);
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          if (db == 0) o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kk], o0, 0, 0, 0);
          else o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kk], o1, 0, 0, 0);
        }
      }
    }
    buf = buf + 1 == NS ? 0 : buf + 1;
  }
  wait_vmcnt<0>();  // no load may still target LDS when the workgroup ends

  const float inv = 1.f / sum_halves(l);
  if (my_q < a.n_q) {
    __bf16* orow = Op + (int64_t)my_q * a.o_sr;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 v0, v1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v0[r] = o0[4 * i4 + r] * inv;
        v1[r] = o1[4 * i4 + r] * inv;
      }
      *(bf16x4*)(orow + 8 * i4 + 4 * g) = __builtin_convertvector(v0, bf16x4);
      *(bf16x4*)(orow + 32 + 8 * i4 + 4 * g) = __builtin_convertvector(v1, bf16x4);
    }
  }
}

template <int NW, int NS>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  constexpr int QT = NW * 32;
  dim3 grid(a.B * a.h, (a.n_q + QT - 1) / QT);
  void* args[] = {(void*)&a};
  return hipExtLaunchKernel((const void*)attn_fwd_bf16_d64_kernel<NW, NS>, grid, dim3(NW * 64), args,
                            0, s, ev.start, ev.stop, 0);
}

}  // namespace

hipError_t launch_attn_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  // Measured on MI355X: with many 128-query blocks (long sequences) 8-wave
  // workgroups with a 3-tile ring are fastest; otherwise 4-wave workgroups
  // with a 2-tile ring (more independent workgroups per compute unit).
  const long blocks = (long)a.B * a.h * ((a.n_q + 127) / 128);
  if (blocks >= 2048) return launch_cfg<8, 3>(a, s, ev);
  return launch_cfg<4, 2>(a, s, ev);
}

}  // namespace mha


