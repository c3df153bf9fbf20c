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
// reason), so a tile's weights are first taken with the row's current m,
// without computing the tile's maximum.  Only when a row's weights of the
// tile sum to more than 2^8 (some score exceeds m by that much, or m is
// still its initial sentinel on the row's first tile) does the row move m to the exact
// maximum of everything it has seen, rescale acc and l by exp(m_old - m_new)
// and take the tile's weights again.  Every weight stays at most 2^8, and
// after a row's first tile this almost never happens.  Each row decides for
// itself, so a row's arithmetic depends only
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
constexpr float kMaxTileSum = 256.0f;  // 2^8: bound on one lane's tile weight sum
constexpr float kNoMax = -1.0e30f;     // m before a row has seen any key

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
// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16-byte global -> LDS copy per lane from a wave-uniform 64-bit base plus a
// per-lane 32-bit byte offset (no vector address arithmetic); lane l writes
// LDS byte address lds + 16 l.
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff, unsigned lds) {
  // The base is wave-uniform; readfirstlane pins it to SGPRs for the saddr operand.
  const unsigned long long p = (unsigned long long)(size_t)sbase;
  // (readfirstlane returns int: widen through unsigned, never sign-extend.)
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)p);
  const unsigned long long sp = ((unsigned long long)hi << 32) | (unsigned long long)lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"((const void*)(size_t)sp)
               : "memory", "m0");
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p);
}

// WPE waves per SIMD (4: <= 128 VGPRs, 3: <= 168); LDS allows four for NW * NS <= 16.
template <int NW, int NS, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_fwd_bf16_d64_kernel(const AttnArgs a) {
  static_assert(NS == 2 || NS == 3, "ring depth");
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
  const int b = __builtin_amdgcn_readfirstlane(bh / a.h);  // wave-uniform: keep in SGPRs
  const int hh = bh - b * a.h;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int q0 = qt * QT;

  const __bf16* Qp = (const __bf16*)a.Q + b * a.q_sb + hh * a.q_sh;
  const char* Kp = (const char*)((const __bf16*)a.K + b * a.k_sb + hh * a.k_sh);
  const char* Vp = (const char*)((const __bf16*)a.V + b * a.v_sb + hh * a.v_sh);
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
  // the swizzle maps there.  Byte offsets from the tile's first row.
  auto chunk_of = [&](int r, int& row, int& kc, int& vc) {
    const int q = (wave * CHW + r) * 64 + lane;
    row = q >> 3;
    kc = ((q & 7) ^ ((row >> 1) & 7)) * 8;
    vc = ((q & 7) ^ (((row >> 1) & 1) << 2)) * 8;
  };
  unsigned koff[CHW], voff[CHW];
#pragma unroll
  for (int r = 0; r < CHW; ++r) {
    int row, kc, vc;
    chunk_of(r, row, kc, vc);
    koff[r] = (unsigned)(row * a.k_sr + kc) * 2u;
    voff[r] = (unsigned)(row * a.v_sr + vc) * 2u;
  }
  const unsigned ks_lds = lds_addr(&Ks[0][0]);
  const unsigned vs_lds = lds_addr(&Vs[0][0]);
  auto issue = [&](int tile, int buf) {
    const unsigned kd = ks_lds + (unsigned)(buf * KT * D + wave * CHW * 512) * 2u;
    const unsigned vd = vs_lds + (unsigned)(buf * KT * D + wave * CHW * 512) * 2u;
    const int k0 = tile * KT;
    if (k0 + KT <= a.n_k) {
      const char* kb = Kp + (int64_t)k0 * a.k_sr * 2;
      const char* vb = Vp + (int64_t)k0 * a.v_sr * 2;
#pragma unroll
      for (int r = 0; r < CHW; ++r) {
        dma16_s(kb, koff[r], kd + 1024u * r);
        dma16_s(vb, voff[r], vd + 1024u * r);
      }
    } else {  // ragged last tile: rows past n_k read the last row (never used)
#pragma unroll
      for (int r = 0; r < CHW; ++r) {
        int row, kc, vc;
        chunk_of(r, row, kc, vc);
        const int key = min(k0 + row, a.n_k - 1);
        dma16_s(Kp, (unsigned)(key * a.k_sr + kc) * 2u, kd + 1024u * r);
        dma16_s(Vp, (unsigned)(key * a.v_sr + vc) * 2u, vd + 1024u * r);
      }
    }
  };

  const float c2 = a.scale * 1.4426950408889634f;
  // m starts at a finite sentinel far below any score rather than -inf, so
  // that no weight is ever exp2(-inf + inf) = NaN: on a row's first tile
  // every visible weight overflows to +inf (which forces the exact-maximum
  // path) and masked ones are exp2(-inf) = 0.  (This file is compiled on the
  // assumption that no NaN occurs.)
  float m = kNoMax;
  float l = 0.f;
  f32x16 o0 = {}, o1 = {};

  // LDS read offsets (elements within one tile buffer).  K (A operand of
  // S^T = K Q^T): lane (col, g) reads key col (and col + 32, 2048 elements
  // further) at chunk 2kk + g.  V^T (A operand of O^T += V^T P^T): the
  // transposing read of 16-lane group (key block, d block); the key block of
  // step kk is 16kk rows further, the +8-key half 512 elements further.
  int kx[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kx[kk] = k_off(col, 2 * kk + g);
  const int tr_key = ((lane & 15) >> 2) + 4 * g;
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int vx[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = 32 * db + tr_d;
    vx[db] = v_off(tr_key, d >> 3) + (d & 7);
  }

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < ntiles) issue(s, s);
  bf16x8 qf[4];
  {
    const bf16x8* src = (const bf16x8*)(Qp + (int64_t)min(my_q, a.n_q - 1) * a.q_sr);
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = src[2 * s + g];
  }

  // The softmax bookkeeping runs per 32-key half tile: half h of a tile is
  // the scores sh (keys k0 + 32h + 8(i/4) + 4g + i%4 for sh[i]), and its
  // weights are the P.V operands p[2h], p[2h+1].  Working in halves lets the
  // vector ALU work on one half while the matrix unit multiplies the other.
  //
  // Weights for reference value m: 2^(s c2 - m c2), rounded to bf16; returns
  // this lane's sum of the rounded weights.
  auto weights = [&](const f32x16& sh, bf16x8& pa, bf16x8& pb) {
    const float mc = m * c2;
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float lt = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x8 w;
#pragma unroll
      for (int r = 0; r < 8; ++r) w[r] = fast_exp2(fmaf(sh[8 * hf + r], c2, -mc));
      const bf16x8 pw = __builtin_convertvector(w, bf16x8);
      if (hf == 0) pa = pw;
      else pb = pw;
#pragma unroll
      for (int r = 0; r < 8; r += 2)
        lt = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pw[r], pw[r + 1]}, one, lt, false);
    }
    return lt;
  };
  // The weights are first taken with the current m.  If some weight of a
  // row came out above 2^8 in total (or m is still the sentinel), that
  // row's m moves to the exact maximum of everything it has seen, its acc
  // and l are rescaled, and the half's weights are taken again.
  auto half = [&](const f32x16& sh, bf16x8& pa, bf16x8& pb) {
    float lt = weights(sh, pa, pb);
    unsigned need = lt > kMaxTileSum;  // lt is finite or +inf, never NaN
    {
      const auto r = __builtin_amdgcn_permlane32_swap(need, need, false, false);
      need = r[0] | r[1];  // both halves of a query row decide together
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      float mt = fmaxf(sh[0], sh[1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) mt = fmaxf(mt, fmaxf(sh[i], sh[i + 1]));
      mt = max_halves(mt);
      if (need) {
        const float m_new = fmaxf(m, mt);
        const float alpha = fast_exp2((m - m_new) * c2);  // 0 while m is the sentinel
        m = m_new;
        l *= alpha;
        o0 *= alpha;
        o1 *= alpha;
      }
      lt = weights(sh, pa, pb);
    }
    l += lt;
  };
  // O^T += V^T P^T over the 32 keys of half h (key blocks 2h, 2h+1).
  auto pv_half = [&](const __bf16* vs, int h, const bf16x8& pa, const bf16x8& pb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kk = 2 * h + j;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const i16x4 lo = tr_read(&vs[vx[db] + 16 * kk * D]);
        const i16x4 hi = tr_read(&vs[vx[db] + (16 * kk + 8) * D]);
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8& pk = j == 0 ? pa : pb;
        if (db == 0) o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk, o0, 0, 0, 0);
        else o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk, o1, 0, 0, 0);
      }
    }
  };

  auto step = [&](int t, const __bf16* ks, const __bf16* vs) {
    const int k0 = t * KT;
    if (k0 >= wv_keys) return;  // no visible key for any query of this wave
    // S^T = K Q^T, first-half chain leading so that its softmax can start
    // while the second half's products are still running.
    f32x16 s0 = {}, s1 = {};
    bf16x8 ka[4], kb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      ka[kk] = *(const bf16x8*)&ks[kx[kk]];
      kb[kk] = *(const bf16x8*)&ks[kx[kk] + 32 * D];
    }
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], s0, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[1], qf[1], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[0], qf[0], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2], qf[2], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[1], qf[1], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[3], qf[3], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[2], qf[2], s1, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[3], qf[3], s1, 0, 0, 0);
    if (k0 + KT > lim) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= lim) s0[i] = -INFINITY;
        if (key + 32 >= lim) s1[i] = -INFINITY;
      }
    }
    bf16x8 p[4];
    half(s0, p[0], p[1]);
    pv_half(vs, 0, p[0], p[1]);
    half(s1, p[2], p[3]);
    pv_half(vs, 1, p[2], p[3]);
  };

  // The ring index is a compile-time constant in each unrolled copy.
  for (int t0 = 0; t0 < ntiles; t0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int t = t0 + u;
      if (t < ntiles) {
        if (NS == 3 && t + 1 < ntiles) wait_vmcnt<2 * CHW>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (t + NS - 1 < ntiles) issue(t + NS - 1, (u + NS - 1) % NS);
        step(t, Ks[u], Vs[u]);
      }
    }
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

template <int NW, int NS, int WPE>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  constexpr int QT = NW * 32;
  dim3 grid(a.B * a.h, (a.n_q + QT - 1) / QT);
  void* args[] = {(void*)&a};
  return hipExtLaunchKernel((const void*)attn_fwd_bf16_d64_kernel<NW, NS, WPE>, grid, dim3(NW * 64),
                            args, 0, s, ev.start, ev.stop, 0);
}

}  // namespace

hipError_t launch_attn_bf16_d64_cfg(const AttnArgs& a, int cfg, hipStream_t s, LaunchEvents ev) {
  switch (cfg) {
    case 0: return launch_cfg<4, 2, 4>(a, s, ev);
    case 1: return launch_cfg<4, 2, 3>(a, s, ev);
    case 2: return launch_cfg<4, 3, 3>(a, s, ev);
    case 3: return launch_cfg<8, 2, 4>(a, s, ev);
    case 4: return launch_cfg<8, 3, 4>(a, s, ev);
    case 5: return launch_cfg<8, 3, 3>(a, s, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  // Measured on MI355X: with many 128-query blocks (long sequences) 8-wave
  // workgroups with a 2-tile ring and four waves per SIMD are fastest;
  // otherwise 4-wave workgroups with a 2-tile ring and three waves per SIMD.
  const long blocks = (long)a.B * a.h * ((a.n_q + 127) / 128);
  if (blocks >= 2048) return launch_attn_bf16_d64_cfg(a, 3, s, ev);
  return launch_attn_bf16_d64_cfg(a, 1, s, ev);
}

}  // namespace mha
