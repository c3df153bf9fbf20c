// Attention for few queries over many keys (the incremental-decoding shape:
// one new query per sequence against its cached keys and values), bf16 in /
// bf16 out, fp32 accumulation, head size 64, for gfx950.  Same definition as
// the main attention kernel, O = softmax(Q K^T * scale + M) V (devpress.csdn.net
// "【深度学习】Transformer", section 2.1, equation (2.4); the key-padding
// mask hides a sequence's keys past its length, hex4c59.cc "读懂 Attention
// Is All You Need", section "掩码必须在 softmax 之前生效"), and the same
// per-wave streaming softmax (wave_attention.h).
//
// With n_q <= 32 the main kernel has one busy wave per (batch, head), which
// walks every key tile alone.  Here the eight waves of a workgroup split the
// keys instead: wave w takes key tiles w, w + 8, w + 16, ... and streams
// them through its own 16 KB LDS slot (it issues, waits for and reads its own
// copies, so the loop has no workgroup barrier).  A wave reads its tile out
// of the slot into registers and issues the next tile's copy before it
// multiplies, so a copy is in flight while it computes.  Each wave ends with a partial state of the
// softmax over its keys -- a reference value m, a sum l and an accumulator --
// for the same 32 query rows; the eight are merged as one streaming step
// would merge them (common reference m* = max m_w; l and the accumulator
// scaled by exp(m_w - m*) and summed), which is the same softmax because the
// split only reorders the sum over keys.  (Measured on MI355X: 6% faster
// than four waves with two slots each.)
//
// Grid: batch * heads workgroups, longest sequences first (padded); a
// head's K/V rows are read once.  The
// shape is bandwidth-bound: per key 256 bytes of K and V against 4 * 64 *
// n_q flops.
#include "wave_attention.h"

namespace mha {
namespace {

using namespace dev;

constexpr int NW = 8;                 // waves per workgroup
constexpr int TILE_BYTES = KT * D * 2;  // one matrix of a tile (8 KB)
constexpr int SLOT = 2 * KT * D;      // elements of one ring slot (K then V)

__global__ __launch_bounds__(NW * 64) void attn_decode_bf16_d64_kernel(const AttnArgs a) {
  // Per wave: one slot of (K tile, V tile).  128 KB.
  __shared__ __attribute__((aligned(1024))) __bf16 ring[NW][SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;

  // Workgroups in dispatch order take the longest sequences first.  With
  // splits > 1, the `splits` consecutive workgroups of a (batch, head) share
  // its key tiles: workgroup sp, wave w takes tiles sp * NW + w + k * NW * splits.
  const int S = a.splits > 1 ? a.splits : 1;
  const int grp = __builtin_amdgcn_readfirstlane((int)blockIdx.x / S);
  const int sp = (int)blockIdx.x - grp * S;
  const int slot = __builtin_amdgcn_readfirstlane(grp / a.h);
  const int hh = grp - slot * a.h;
  const int b = __builtin_amdgcn_readfirstlane(a.padded ? (int)a.order[slot] : slot);
  const __bf16* Qp = wave_uniform((const __bf16*)a.Q + b * a.q_sb + hh * a.q_sh);
  const char* Kp = wave_uniform((const char*)((const __bf16*)a.K + b * a.k_sb + hh * a.k_sh));
  const char* Vp = wave_uniform((const char*)((const __bf16*)a.V + b * a.v_sb + hh * a.v_sh));
  __bf16* Op = wave_uniform((__bf16*)a.O + b * a.o_sb + hh * a.o_sh);

  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  L = __builtin_amdgcn_readfirstlane(L);
  const int ntiles = (L + KT - 1) / KT;
  const int my_q = col;  // n_q <= 32: the wave's rows are queries 0..31

  // Copies: instruction r (0..7) of a matrix fills LDS block r of the tile
  // (rows 8r .. 8r+7); lane l writes 16-byte chunk l of it: row q >> 3,
  // stored chunk q & 7 with q = 64 r + l, holding the source chunk that the
  // K (k_off) or V (v_off) swizzle maps there.  Byte offsets from row 0.
  auto chunk_of = [&](int r, int& row, int& kc, int& vc) {
    const int q = r * 64 + lane;
    row = q >> 3;
    kc = ((q & 7) ^ ((row >> 1) & 7)) * 8;
    vc = ((q & 7) ^ (((row >> 1) & 1) << 2)) * 8;
  };
  const unsigned ring_lds = lds_addr(&ring[wave][0]);
  auto issue = [&](int tile) {
    const unsigned kd = ring_lds;
    const unsigned vd = kd + (unsigned)TILE_BYTES;
    const int k0 = tile * KT;
    const char* kb = wave_uniform(Kp + (int64_t)k0 * a.k_sr * 2);  // the tile's first row (64-bit)
    const char* vb = wave_uniform(Vp + (int64_t)k0 * a.v_sr * 2);
    if (k0 + KT <= a.n_k) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        int row, kc, vc;
        chunk_of(r, row, kc, vc);
        dma16_s(kb, (unsigned)(row * a.k_sr + kc) * 2u, kd + 1024u * r);
        dma16_s(vb, (unsigned)(row * a.v_sr + vc) * 2u, vd + 1024u * r);
      }
    } else {  // ragged last tile: rows past n_k read the last row (never used)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        int row, kc, vc;
        chunk_of(r, row, kc, vc);
        const int rr = min(row, a.n_k - 1 - k0);  // offsets from the tile's own row
        dma16_s(kb, (unsigned)(rr * a.k_sr + kc) * 2u, kd + 1024u * r);
        dma16_s(vb, (unsigned)(rr * a.v_sr + vc) * 2u, vd + 1024u * r);
      }
    }
  };

  WaveAttention wa;
  wa.init(lane, a.scale);
  wa.load_q(Qp + (int64_t)min(my_q, a.n_q - 1) * a.q_sr);
  const int first = sp * NW + wave, stride = NW * S;
  if (first < ntiles) issue(first);
  for (int t = first; t < ntiles; t += stride) {
    wait_vmcnt<0>();
    const __bf16* ks = &ring[wave][0];
    // The tile moves into registers; once those reads have returned, the
    // slot takes the next tile's copy, which is in flight while this tile
    // is multiplied.
    WaveAttention::TileRegs r;
    wa.read_tile(ks, ks + KT * D, r);
    wait_lgkmcnt0();
    if (t + stride < ntiles) issue(t + stride);
    wa.tile_regs(r, t * KT, L, L);
  }
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with its ring

  // Merge: waves 1..NW-1 leave (m, l, O^T) in LDS, wave 0 folds them in.
  float* part = (float*)&ring[0][0];
  constexpr int PS = 64 * 34;  // floats per wave: m, l, 32 accumulator values per lane
  static_assert((NW - 1) * PS * 4 <= (int)sizeof(ring), "partial states fit in the ring");
  if (wave > 0) {
    float* p = part + (wave - 1) * PS;
    p[lane] = wa.m;
    p[64 + lane] = wa.l;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[128 + 64 * i + lane] = wa.o0[i];
      p[128 + 64 * (16 + i) + lane] = wa.o1[i];
    }
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    const float* p = part + (w - 1) * PS;
    const float m1 = p[lane], l1 = p[64 + lane];
    const float mm = fmaxf(wa.m, m1);
    // Partial states that saw no visible key keep the finite sentinel m and
    // l = 0, acc = 0: their factor underflows to 0.
    const float a0 = fast_exp2((wa.m - mm) * wa.c2), a1 = fast_exp2((m1 - mm) * wa.c2);
    wa.m = mm;
    wa.l = wa.l * a0 + l1 * a1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      wa.o0[i] = wa.o0[i] * a0 + p[128 + 64 * i + lane] * a1;
      wa.o1[i] = wa.o1[i] * a0 + p[128 + 64 * (16 + i) + lane] * a1;
    }
  }
  if (S > 1) {  // this workgroup's state, for the merge launch
    float* st = a.part + ((int64_t)(b * a.h + hh) * S + sp) * kDecodeStateFloats;
    st[lane] = wa.m;
    st[64 + lane] = wa.l;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[128 + 64 * i + lane] = wa.o0[i];
      st[128 + 64 * (16 + i) + lane] = wa.o1[i];
    }
    return;
  }
  const float inv = wa.inv_sum();
  wa.store(Op + (int64_t)min(my_q, a.n_q - 1) * a.o_sr, inv, my_q < a.n_q);
  if (a.lse != nullptr && my_q < a.n_q && wa.g == 0)
    a.lse[(int64_t)(b * a.h + hh) * a.n_q + my_q] = wa.row_lse(inv);
}

// One wave per (batch, head): folds the `splits` partial states in the same
// way the workgroup folded its waves' states, then normalises and stores.
__global__ __launch_bounds__(64) void attn_decode_merge_kernel(const AttnArgs a) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.h;
  const int hh = bh - b * a.h;
  const float* st = a.part + (int64_t)bh * a.splits * kDecodeStateFloats;
  WaveAttention wa;
  wa.init(lane, a.scale);
  wa.m = st[lane];
  wa.l = st[64 + lane];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    wa.o0[i] = st[128 + 64 * i + lane];
    wa.o1[i] = st[128 + 64 * (16 + i) + lane];
  }
  for (int s = 1; s < a.splits; ++s) {
    const float* p = st + (int64_t)s * kDecodeStateFloats;
    const float m1 = p[lane], l1 = p[64 + lane];
    const float mm = fmaxf(wa.m, m1);
    const float a0 = fast_exp2((wa.m - mm) * wa.c2), a1 = fast_exp2((m1 - mm) * wa.c2);
    wa.m = mm;
    wa.l = wa.l * a0 + l1 * a1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      wa.o0[i] = wa.o0[i] * a0 + p[128 + 64 * i + lane] * a1;
      wa.o1[i] = wa.o1[i] * a0 + p[128 + 64 * (16 + i) + lane] * a1;
    }
  }
  const int my_q = lane & 31;
  __bf16* Op = (__bf16*)a.O + b * a.o_sb + hh * a.o_sh;
  const float inv = wa.inv_sum();
  wa.store(Op + (int64_t)min(my_q, a.n_q - 1) * a.o_sr, inv, my_q < a.n_q);
  if (a.lse != nullptr && my_q < a.n_q && wa.g == 0)
    a.lse[(int64_t)bh * a.n_q + my_q] = wa.row_lse(inv);
}

}  // namespace

// More than two key tiles (a key range of at most 128 keeps the plain kernel,
// whose single-wave order the fused short-sequence kernel reproduces).
bool attn_decode_applies(const AttnArgs& a) {
  return a.n_q <= 32 && !a.causal && a.n_k > 2 * KT;
}

hipError_t launch_attn_decode_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  if (!attn_decode_applies(a) || a.splits > 1) return hipErrorInvalidValue;
  void* args[] = {(void*)&a};
  return launch_kernel((const void*)attn_decode_bf16_d64_kernel, dim3(a.B * a.h), dim3(NW * 64),
                            args, 0, s, ev.start, ev.stop, 0);
}

hipError_t launch_attn_decode_split_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev_part,
                                             LaunchEvents ev_merge) {
  if (!attn_decode_applies(a) || a.splits < 2 || a.part == nullptr) return hipErrorInvalidValue;
  void* args[] = {(void*)&a};
  hipError_t e = launch_kernel((const void*)attn_decode_bf16_d64_kernel, dim3(a.B * a.h * a.splits),
                                    dim3(NW * 64), args, 0, s, ev_part.start, ev_part.stop, 0);
  if (e != hipSuccess) return e;
  return launch_kernel((const void*)attn_decode_merge_kernel, dim3(a.B * a.h), dim3(64), args, 0, s,
                            ev_merge.start, ev_merge.stop, 0);
}

}  // namespace mha
