// Fused scaled dot-product attention, forward, bf16 in / bf16 out, fp32
// accumulation, head size 64, for gfx950.  The score matrix is never
// stored: each workgroup streams K/V tiles of one (batch, head) through LDS
// and every wave keeps the streaming softmax state of its 32 queries (the
// per-wave arithmetic, with its sources, is described in wave_attention.h).
//
// Work decomposition
//   workgroup = NW waves, wave w owns the 32 queries q0 + 32w .. +31;
//   grid.x = batch*heads (fastest: the workgroups of one head land on the
//   same XCD when batch*heads is a multiple of 8 and share its L2),
//   grid.y = query tiles, heaviest causal tiles dispatched first.
//   K and V tiles go from global memory straight into LDS
//   (global_load_lds_dwordx4, no register staging) through a ring of NS tile
//   buffers, NS-1 tiles ahead of the one being computed; 16-byte chunks are
//   XOR-swizzled so that both LDS read patterns are conflict-free.  A wave
//   skips the tiles none of its queries can see (causal).
//   Key split (KS = 2 or 4, for launches too small to give every SIMD
//   several waves): the workgroup holds KS groups of NW waves over the same
//   queries; group j takes the j-th of KS consecutive runs of the query
//   tile's key tiles, each group through its own ring slot of every stage.
//   At the end groups 1 .. KS-1 hand their softmax states (reference value,
//   sum, accumulators) to group 0 through LDS, which merges them (the
//   streaming softmax's own rescaling rule) and writes the output.  The
//   longest chain of dependent tiles a wave walks shrinks KS-fold and KS
//   times as many waves share each SIMD.
#include "wave_attention.h"

namespace mha {
namespace {

using namespace dev;

// WPE waves per SIMD (4: <= 128 VGPRs, 3: <= 168).  KS key groups of NW
// waves each (1, 2 or 4).  LDS: NS * KS * 16 KB per workgroup.
template <int NW, int NS, int WPE, int KS>
__global__ __launch_bounds__(NW * KS * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_fwd_bf16_d64_kernel(const AttnArgs a) {
  static_assert(NS == 2 || NS == 3, "ring depth");
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && NS == 2), "key split: two or four groups, two-slot ring");
  constexpr int BLK = KT * D * 2 / 1024;  // 1 KB blocks per tile and matrix
  constexpr int CHW = BLK / NW;           // load instructions per wave, tile and matrix
  constexpr int QT = NW * 32;
  static_assert(CHW * NW == BLK, "waves must split the tile evenly");
  // Merge buffers (the key split): groups 1 and 2 in the K ring, group 3 and
  // the reference values and sums in the V ring.
  static_assert(KS == 1 || (KS < 4 ? 1 : 2) * NW * 32 * 64 * 4 <= NS * KS * KT * D * 2, "merge: K ring");
  static_assert(KS < 4 || NW * 32 * 64 * 4 + 3 * NW * 2 * 64 * 4 <= NS * KS * KT * D * 2, "merge: V ring");

  // Ring slot s of group j: Ks[s][j], Vs[s][j].
  __shared__ __attribute__((aligned(1024))) __bf16 Ks[NS][KS][KT * D];
  __shared__ __attribute__((aligned(1024))) __bf16 Vs[NS][KS][KT * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = KS == 1 ? 0 : wave_all / NW;  // key group
  const int wave = wave_all - kg * NW;         // query block of the tile
  const int col = lane & 31;

  const int bh = blockIdx.x;
  const int b = __builtin_amdgcn_readfirstlane(bh / a.h);  // wave-uniform: keep in SGPRs
  const int hh = bh - b * a.h;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int q0 = qt * QT;

  const __bf16* Qp = wave_uniform((const __bf16*)a.Q + b * a.q_sb + hh * a.q_sh);
  const char* Kp = wave_uniform((const char*)((const __bf16*)a.K + b * a.k_sb + hh * a.k_sh));
  const char* Vp = wave_uniform((const char*)((const __bf16*)a.V + b * a.v_sb + hh * a.v_sh));
  __bf16* Op = wave_uniform((__bf16*)a.O + b * a.o_sb + hh * a.o_sh);

  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int wg_last = min(q0 + QT, a.n_q) - 1;
  const int wg_keys = a.causal ? min(L, wg_last + 1) : L;
  const int qw0 = q0 + 32 * wave;
  const int my_q = qw0 + col;
  const int lim = a.causal ? min(L, my_q + 1) : L;
  const int lim_min = __builtin_amdgcn_readfirstlane(a.causal ? min(L, qw0 + 1) : L);
  const int wv_last = min(qw0 + 32, a.n_q) - 1;
  const int wv_keys =
      __builtin_amdgcn_readfirstlane(wv_last < qw0 ? 0 : (a.causal ? min(L, wv_last + 1) : L));
  const int ntiles = __builtin_amdgcn_readfirstlane((wg_keys + KT - 1) / KT);
  // Group kg walks tiles first_tile .. first_tile + my_tiles - 1; both groups
  // step through n_steps iterations (one barrier each).
  const int n_steps = (ntiles + KS - 1) / KS;
  const int first_tile = kg * n_steps;
  const int my_tiles = __builtin_amdgcn_readfirstlane(max(0, min(n_steps, ntiles - first_tile)));

  // Direct loads: instruction r of this wave fills LDS block (wave*CHW + r)
  // (8 rows) of its group's tile; lane l writes 16-byte chunk l of it, i.e.
  // row q >> 3, stored chunk q & 7 with q = block*64 + l, which holds the
  // source chunk that the swizzle maps there.  Byte offsets from the tile's
  // first row.
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
  const unsigned ks_lds = lds_addr(&Ks[0][kg][0]);
  const unsigned vs_lds = lds_addr(&Vs[0][kg][0]);
  // Tiles are issued in order; kb/vb point at the group's next one
  // (wave-uniform, advanced with scalar adds).
  const int64_t kstep = (int64_t)KT * a.k_sr * 2, vstep = (int64_t)KT * a.v_sr * 2;
  const char* kb = Kp + first_tile * kstep;
  const char* vb = Vp + first_tile * vstep;
  auto issue = [&](int step, int buf) {
    const unsigned kd = ks_lds + (unsigned)(buf * KS * KT * D + wave * CHW * 512) * 2u;
    const unsigned vd = vs_lds + (unsigned)(buf * KS * KT * D + wave * CHW * 512) * 2u;
    const int k0 = (first_tile + step) * KT;
    if (k0 + KT <= a.n_k) {
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
        const int rr = min(row, a.n_k - 1 - k0);  // offsets from the tile's own row
        dma16_s(kb, (unsigned)(rr * a.k_sr + kc) * 2u, kd + 1024u * r);
        dma16_s(vb, (unsigned)(rr * a.v_sr + vc) * 2u, vd + 1024u * r);
      }
    }
    kb += kstep;
    vb += vstep;
  };

  WaveAttention wa;
  wa.init(lane, a.scale);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < my_tiles) issue(s, s);
  wa.load_q(Qp + (int64_t)min(my_q, a.n_q - 1) * a.q_sr);

  // The ring index is a compile-time constant in each unrolled copy.
  for (int t0 = 0; t0 < n_steps; t0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int t = t0 + u;
      if (t < n_steps) {
        if (NS == 3 && t + 1 < my_tiles) wait_vmcnt<2 * CHW>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (t + NS - 1 < my_tiles) issue(t + NS - 1, (u + NS - 1) % NS);
        const int k0 = (first_tile + t) * KT;
        if (t < my_tiles && k0 < wv_keys)  // else no visible key
          wa.tile(Ks[u][kg], Vs[u][kg], k0, lim, lim_min);
      }
    }
  }
  wait_vmcnt<0>();  // no load may still target LDS when the workgroup ends

  if constexpr (KS > 1) {
    // Groups 1 .. KS-1 hand their states to group 0 through the (now idle)
    // ring.  Group j's accumulators: 32 floats a lane, float i of lane l of
    // query block w at [w][i][l] in a 32 KB region (the K ring's halves,
    // then the V ring's first); m and l at [j - 1][w][0 or 1][l] after them.
    constexpr int ACC = NW * 32 * 64;  // floats of one group's accumulators
    auto acc_of = [&](int j) -> float* {
      return j <= 2 ? (float*)&Ks[0][0][0] + (j - 1) * ACC : (float*)&Vs[0][0][0] + (j - 3) * ACC;
    };
    float* ml_base = (float*)&Vs[0][0][0] + (KS == 4 ? ACC : 0);
    __syncthreads();  // every wave is done with the tiles
    if (kg > 0) {
      float* acc_x = acc_of(kg) + wave * 32 * 64 + lane;
      float* ml_x = ml_base + ((kg - 1) * NW + wave) * 2 * 64 + lane;
      ml_x[0] = wa.m;
      ml_x[64] = wa.l;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc_x[i * 64] = wa.o0[i];
        acc_x[(16 + i) * 64] = wa.o1[i];
      }
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int j = 1; j < KS; ++j) {
      const float* acc_x = acc_of(j) + wave * 32 * 64 + lane;
      const float* ml_x = ml_base + ((j - 1) * NW + wave) * 2 * 64 + lane;
      f32x16 p0, p1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p0[i] = acc_x[i * 64];
        p1[i] = acc_x[(16 + i) * 64];
      }
      wa.merge(ml_x[0], ml_x[64], p0, p1);
    }
  }

  const float inv = wa.inv_sum();
  wa.store(Op + (int64_t)min(my_q, a.n_q - 1) * a.o_sr, inv, my_q < a.n_q);
  if (a.lse != nullptr && my_q < a.n_q && wa.g == 0)
    a.lse[(int64_t)(b * a.h + hh) * a.n_q + my_q] = wa.row_lse(inv);
}

template <int NW, int NS, int WPE, int KS = 1>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  constexpr int QT = NW * 32;
  dim3 grid(a.B * a.h, (a.n_q + QT - 1) / QT);
  void* args[] = {(void*)&a};
  return launch_kernel((const void*)attn_fwd_bf16_d64_kernel<NW, NS, WPE, KS>, grid, dim3(NW * KS * 64),
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
    case 6: return launch_cfg<4, 2, 4, 2>(a, s, ev);
    case 7: return launch_cfg<4, 2, 4, 4>(a, s, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev) {
  // A few queries over many keys: split the keys over waves instead
  // (attn_decode_bf16.hip).
  if (attn_decode_applies(a)) return launch_attn_decode_bf16_d64(a, s, ev);
  // Unmasked attention with at least two 8-wave workgroups (256 queries)
  // per compute unit: each K/V tile copied into LDS serves twice the
  // queries.  Measured on MI355X, same box: 4 x 16 x 2048 78.2 -> 73.4 us,
  // 4 x 16 x 4096 284 -> 278 us, 1 x 16 x 8192 284 -> 268 us; with fewer
  // workgroups than that they lose up to 30% (1 x 8 x 4096, 2 x 16 x 1024),
  // and on causal shapes the uneven work per query tile favours the
  // smaller workgroups.
  const int64_t wg8 = (int64_t)a.B * a.h * ((a.n_q + 255) / 256);
  if (!a.causal && !a.padded && wg8 >= 2 * (int64_t)device_compute_units())
    return launch_attn_bf16_d64_cfg(a, 3, s, ev);
  // At most one 4-wave workgroup per compute unit over at least 1024 keys:
  // two key groups per workgroup (one wave per SIMD is too few to hide a
  // tile's latencies, and each wave's chain of tiles is halved).  Measured on
  // MI355X, same box, unmasked: 1 x 8 x 4096 58.0 -> 45.5 us, 1 x 4 x 8192
  // 107 -> 85 us, 1 x 16 x 2048 29.5 -> 24.9 us, 2 x 8 x 1024 15.8 -> 13.9
  // us; causal: 1 x 8 x 4096 52.0 -> 41.8 us, 2 x 16 x 1024 16.6 -> 15.2 us.
  // With two workgroups per compute unit (4 x 16 x 1024) it gains nothing,
  // and it loses where the key range is short (32 x 8 x 100: 6.7 -> 7.6 us;
  // 16 x 8 x 512 causal: 12.9 -> 15.1 us).
  // From 2048 keys on, four key groups (16 waves, all 128 KB of LDS ring):
  // 1 x 8 x 4096 49.4 -> 44.7 us, causal 42.1 -> 37.1 us, 1 x 4 x 8192
  // 90 -> 79 us, 1 x 16 x 2048 25.8 -> 25.1 us against two groups; at 1024
  // keys two groups stay ahead (2 x 8 x 1024 14.1 vs 14.7 us).
  const int64_t wg4 = (int64_t)a.B * a.h * ((a.n_q + 127) / 128);
  if (wg4 <= (int64_t)device_compute_units() && a.n_k >= 2048)
    return launch_attn_bf16_d64_cfg(a, 7, s, ev);
  if (wg4 <= (int64_t)device_compute_units() && a.n_k >= 1024)
    return launch_attn_bf16_d64_cfg(a, 6, s, ev);
  // Otherwise 4-wave workgroups (128 queries) with a 2-tile ring and four
  // waves per SIMD are fastest, for short and long sequences alike.
  return launch_attn_bf16_d64_cfg(a, 0, s, ev);
}

}  // namespace mha
