// Per-wave streaming attention of 32 queries of one (batch, head), shared
// by the attention kernels of libmha.  It computes, for the 32 queries a wave owns,
//   O = softmax(Q K^T * scale + M) V                  (M: 0 or -inf)
// (devpress.csdn.net "【深度学习】Transformer", section 2.1, equation
// (2.4); hex4c59.cc "读懂 Attention Is All You Need", sections
// "六步算完一行注意力" and "把所有位置合并，就是那条核心公式"; the mask is
// added before the softmax, hex4c59.cc, section "掩码必须在 softmax 之前生效").
//
// The row softmax is evaluated in streaming form over key tiles: every lane
// keeps a reference value m for its query, a running sum l of
// exp(s - m) and an accumulator of exp(s - m) v; O = acc / l at the end.
// Any finite m gives the same quotient (shifting every score of a row by the
// same amount does not change its softmax; hex4c59.cc, section
// "用几十行代码核对刚才的数值" subtracts the row maximum for the same
// reason), so a tile's weights are first taken with the row's current m,
// without computing the tile's maximum.  Only when a row's weights of a
// half tile sum to more than 2^8 (some score exceeds m by that much, or m is
// still its initial sentinel on the row's first tile) does the row move m to
// the exact maximum of everything it has seen, rescale acc and l by
// exp(m_old - m_new) and take the half's weights again.  Every weight stays
// at most 2^8, and after a row's first tile this almost never happens.  Each
// row decides for itself, so a row's arithmetic depends only on the keys it
// can see.  Masked keys contribute exactly 0: a partially visible tile sets
// their scores to -inf, a tile with no visible key is skipped.
//
// Layout of one wave's products (col = lane & 31, g = lane >> 5):
//   S^T[64 keys x 32 queries] = K_tile . Q^T      (8 MFMA 32x32x16)
//   O^T[64 d x 32 queries]   += V_tile^T . P^T    (8 MFMA 32x32x16)
// The transposed products keep every accumulator element of a lane on that
// lane's own query (lane = query, lane ^ 32 holds the other half of its
// keys), so the softmax bookkeeping is per-lane scalar work with one
// cross-half exchange (v_permlane32_swap), and P^T leaves the first MFMA
// already in the B-operand layout of the second: the MFMA output rows of
// lane group g are keys {8j + 4g + r}, and the V^T operand is gathered in
// that key order by transposing LDS reads (ds_read_b64_tr_b16).
//
// Files that include this header are compiled on the assumption that no
// NaN occurs (the arithmetic below never produces one).
#pragma once

#include <math.h>

#include "device.h"

namespace mha {
namespace dev {

constexpr int D = 64;                  // head size d_k = d_v
constexpr int KT = 64;                 // keys per tile
constexpr float kMaxTileSum = 256.0f;  // 2^8: bound on one lane's half-tile weight sum
constexpr float kNoMax = -1.0e30f;     // m before a row has seen any key

// K tile [64][64] bf16, 128-byte rows: chunk c of row r at chunk c ^ ((r >> 1) & 7).
__device__ __forceinline__ int k_off(int r, int chunk) { return r * D + ((chunk ^ ((r >> 1) & 7)) << 3); }
// V tile [64][64] bf16, 128-byte rows: chunk c of row r at chunk c ^ (((r >> 1) & 1) << 2).
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

// A lane's 64-wide row of transposed-product accumulators (a0: columns
// 8 i + 4 g + r at a0[4 i + r], i = 0..3; a1 the same 32 columns further),
// times c, rounded to bf16 and stored at `row`.  Lanes l and l + 32 hold the
// two halves of every 16-byte chunk of the row; one permlane32 swap per
// register gives each lane a whole chunk, so the row goes out in 16-byte
// stores.  Call with every lane active; `valid` predicates the stores (row
// must be a valid row address either way).
__device__ __forceinline__ void store_row_bf16(__bf16* row, int g, const f32x16& a0, const f32x16& a1,
                                               float c, bool valid) {
  u32x2 pk[8];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    f32x4 v0, v1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v0[r] = a0[4 * i4 + r] * c;
      v1[r] = a1[4 * i4 + r] * c;
    }
    pk[i4] = __builtin_bit_cast(u32x2, __builtin_convertvector(v0, bf16x4));
    pk[4 + i4] = __builtin_bit_cast(u32x2, __builtin_convertvector(v1, bf16x4));
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const auto sw = __builtin_amdgcn_permlane32_swap(pk[4 * blk + 2 * p][w], pk[4 * blk + 2 * p + 1][w],
                                                         false, false);
        out[w] = sw[0];
        out[2 + w] = sw[1];
      }
      if (valid) *(u32x4*)(row + 32 * blk + 16 * p + 8 * g) = out;
    }
}

// Streaming attention state of one wave: 32 queries of one (batch, head).
// Key tiles come from LDS in the k_off (K) and v_off (V) layouts.
struct WaveAttention {
  float c2;         // scale * log2(e)
  float m;          // reference value of this lane's query (raw q.k units)
  float l;          // this lane's share of the running sum of weights
  f32x16 o0, o1;    // O^T accumulators: d 0..31 and 32..63 of this lane's query
  bf16x8 qf[4];     // Q^T operand: Q[q][16s + 8g .. +7]
  int g;            // lane >> 5
  int kx[4];        // K operand offsets (elements) for key col, chunk 2kk + g
  int vx[2];        // V^T transposing-read offsets for d blocks 0 and 1

  __device__ __forceinline__ void init(int lane, float scale) {
    const int col = lane & 31;
    g = lane >> 5;
    c2 = scale * 1.4426950408889634f;
    // m starts at a finite sentinel far below any score rather than -inf, so
    // that no weight is ever exp2(-inf + inf) = NaN: on a row's first tile
    // every visible weight overflows to +inf (which forces the exact-maximum
    // path) and masked ones are exp2(-inf) = 0.
    m = kNoMax;
    l = 0.f;
    o0 = f32x16{};
    o1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kx[kk] = k_off(col, 2 * kk + g);
    // Transposing read: within each 16-lane group, lane s addresses key
    // (s / 4) (+4 for g = 1) and d 4 (s % 4) .. +3 of its 16-wide d block.
    const int tr_key = ((lane & 15) >> 2) + 4 * g;
    const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * db + tr_d;
      vx[db] = v_off(tr_key, d >> 3) + (d & 7);
    }
  }

  // Q row `row` (64 bf16, 16-byte aligned) into the Q^T operand.
  __device__ __forceinline__ void load_q(const __bf16* row) {
    const bf16x8* src = (const bf16x8*)row;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = src[2 * s + g];
  }

  // Q row `row` of a [rows][64] LDS buffer in the k_off layout.
  __device__ __forceinline__ void load_q_lds(const __bf16* qs, int row) {
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *(const bf16x8*)&qs[k_off(row, 2 * s + g)];
  }

  // Weights of one half tile for the current m: 2^(s c2 - m c2), rounded
  // to bf16; returns this lane's sum of the rounded weights.
  __device__ __forceinline__ float weights(const f32x16& sh, bf16x8& pa, bf16x8& pb) const {
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
  }

  // Softmax bookkeeping of one half tile (scores sh; weights into pa, pb).
  __device__ __forceinline__ void half(const f32x16& sh, bf16x8& pa, bf16x8& pb) {
    float lt = weights(sh, pa, pb);
    // One compare decides for the whole wave (its lane mask is the ballot;
    // lt is finite or +inf, never NaN); on the exact path both halves of a
    // query row decide together.
    if (__builtin_amdgcn_ballot_w64(lt > kMaxTileSum) != 0) {
      unsigned need = lt > kMaxTileSum;
      {
        const auto r = __builtin_amdgcn_permlane32_swap(need, need, false, false);
        need = r[0] | r[1];
      }
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
  }

  // O^T += V^T P^T over the 32 keys of half h (key blocks 2h, 2h+1).
  __device__ __forceinline__ void pv_half(const __bf16* vs, int h, const bf16x8& pa, const bf16x8& pb) {
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
  }

  // One 64-key tile starting at key k0 (ks, vs: the tile in LDS).  Keys at or
  // beyond `lim` are hidden from this lane's query; lim_min is the smallest
  // lim of the wave (wave-uniform).  The softmax runs per 32-key half, first
  // half leading, so that the vector ALU works on one half while the matrix
  // unit multiplies the other.
  __device__ __forceinline__ void tile(const __bf16* ks, const __bf16* vs, int k0, int lim, int lim_min) {
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
    // s0[i] is the score of key k0 + 8(i/4) + 4g + i%4, s1[i] of that key + 32.
    if (k0 + KT > lim_min) {
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
  }

  // ---- a tile held in registers ------------------------------------------
  // The operands of one 64-key tile, read out of LDS in one go, so that the
  // LDS slot can take the next tile's copy while this one is multiplied.
  struct TileRegs {
    bf16x8 k[8];  // K operand: key blocks 0..3 of the first 32 keys, then of the second
    bf16x8 v[8];  // V^T operand of key block kk (0..3) and d block db at 2 kk + db
  };
  __device__ __forceinline__ void read_tile(const __bf16* ks, const __bf16* vs, TileRegs& r) const {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      r.k[kk] = *(const bf16x8*)&ks[kx[kk]];
      r.k[4 + kk] = *(const bf16x8*)&ks[kx[kk] + 32 * D];
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const i16x4 lo = tr_read(&vs[vx[db] + 16 * kk * D]);
        const i16x4 hi = tr_read(&vs[vx[db] + (16 * kk + 8) * D]);
        r.v[2 * kk + db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  }
  // tile() on a tile held in registers (same products, same order).
  __device__ __forceinline__ void tile_regs(const TileRegs& r, int k0, int lim, int lim_min) {
    f32x16 s0 = {}, s1 = {};
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[0], qf[0], s0, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[1], qf[1], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[4], qf[0], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[2], qf[2], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[5], qf[1], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[3], qf[3], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[6], qf[2], s1, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[7], qf[3], s1, 0, 0, 0);
    if (k0 + KT > lim_min) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= lim) s0[i] = -INFINITY;
        if (key + 32 >= lim) s1[i] = -INFINITY;
      }
    }
    bf16x8 p[4];
    half(s0, p[0], p[1]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.v[2 * j], p[j], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.v[2 * j + 1], p[j], o1, 0, 0, 0);
    }
    half(s1, p[2], p[3]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.v[4 + 2 * j], p[2 + j], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.v[4 + 2 * j + 1], p[2 + j], o1, 0, 0, 0);
    }
  }

  // Fold in the state (m2, l2, p0, p1) of the same queries over another set
  // of keys: both parts are rescaled to the larger reference value, which is
  // the streaming softmax's own update.  A part that saw no key (m at the
  // sentinel, l and the accumulators 0) gets the factor 0, or 1 when
  // neither did.
  __device__ __forceinline__ void merge(float m2, float l2, const f32x16& p0, const f32x16& p1) {
    const float mn = fmaxf(m, m2);
    const float a1 = fast_exp2((m - mn) * c2);
    const float a2 = fast_exp2((m2 - mn) * c2);
    m = mn;
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o0[i] = o0[i] * a1 + p0[i] * a2;
      o1[i] = o1[i] * a1 + p1[i] * a2;
    }
  }

  // 1 / (row sum of weights); a cross-lane exchange: call with all lanes active.
  __device__ __forceinline__ float inv_sum() const { return 1.f / sum_halves(l); }

  // Natural log of the row's sum of exp(scale * s) over its visible keys,
  // from inv = inv_sum(): the weights are exp(scale (s - m)), so the sum is
  // exp(scale m) / inv.
  __device__ __forceinline__ float row_lse(float inv) const {
    return (m * c2 - __builtin_amdgcn_logf(inv)) * 0.6931471805599453f;
  }

  // O row of this lane's query = acc * inv, rounded to bf16 (lane g writes d
  // 8i + 4g .. +3 of both 32-wide halves).
  // Output row = acc / l rounded to bf16 (store_row_bf16).  Call with
  // every lane active; `valid` predicates the stores.
  __device__ __forceinline__ void store(__bf16* orow, float inv, bool valid) const {
    store_row_bf16(orow, g, o0, o1, inv, valid);
  }
};

}  // namespace dev
}  // namespace mha
