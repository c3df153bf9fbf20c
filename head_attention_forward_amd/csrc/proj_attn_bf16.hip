// Fused input projections and attention for short sequences, bf16 in /
// bf16 out, fp32 accumulation, head size 64, for gfx950.
//
// One workgroup per (batch b, head i) computes, for its head only,
//   Q_i = X_q,b W_i^Q,  K_i = X_kv,b W_i^K,  V_i = X_kv,b W_i^V
// (devpress.csdn.net "【深度学习】Transformer", section 2.1, equations
// (2.1)-(2.3) and section 2.2; hex4c59.cc "读懂 Attention Is All You Need",
// sections "Q、K、V 是三种计算角色" and "多头注意力让一次读取有多组投影":
// head i owns column block i of the stacked projections), keeps the three
// tiles in LDS and then computes head_i = softmax(Q_i K_i^T / sqrt(d_k) + M) V_i
// with the same per-wave attention as the standalone attention kernel
// (wave_attention.h), writing head_i into its column block of the
// concatenated output.  Q, K and V never travel through HBM.
//
// The projection is the same computation as the standalone projection GEMM
// (the same bf16 MFMA 32x32x16 products in the same k order with the weight
// fragment as first operand, rounded to bf16 the same way), so both paths
// produce identical intermediates and outputs.
//
// Limits: n_q, n_k <= 128 (one 128-row tile each), d_model a multiple of 64.
//
// Work decomposition (8 waves): the projection output [128 rows x 192
// columns] (Q | K | V, 64 columns each) is 4 x 6 MFMA tiles of 32 x 32;
// wave w computes row block w & 3 and column blocks 3 (w >> 2) .. +2.  The
// activation rows and the three 64-column weight slices stream in 64-wide k
// stages through an LDS ring (global_load_lds_dwordx4, NS stages, NS-1
// ahead).  Afterwards the ring is reused for the bf16 Q, K, V tiles, and
// waves 0-3 run the attention of queries 32w .. 32w+31 over them.
#include "wave_attention.h"

namespace mha {
namespace {

using namespace dev;

constexpr int ROWS = 128;  // rows of the projection tile (>= n_q, n_k)
constexpr int BKP = 64;    // k per stage

// Activation tile [128][64]: 128-byte rows; chunk c of row m at c ^ ((m >> 1) & 7).
__device__ __forceinline__ int x_pos(int m, int chunk) { return chunk ^ ((m >> 1) & 7); }
// Weight tile [64][64]: 128-byte rows; chunk c of row k at c ^ (((k >> 1) & 1) << 2).
__device__ __forceinline__ int w_pos(int k, int chunk) { return chunk ^ (((k >> 1) & 1) << 2); }

// One 32 x 32 projection tile (MFMA accumulators: lane (col, grp) holds row
// `row` and columns 8 q + 4 grp .. +3 of the block, q = 0..3) rounded to bf16
// and stored as 32 rows of a Q, K (k_off) or V (v_off) tile, columns
// 32 half .. +31.  Lanes l and l + 32 hold the two halves of each 16-byte
// chunk; one permlane32 swap per register gives each lane a whole chunk
// (lane l chunk q = 2p, lane l + 32 chunk q = 2p + 1), so the tile goes
// out in 16-byte LDS writes (LDS writes cost the same per instruction at
// 8 and 16 bytes).  Call with all lanes active.
__device__ __forceinline__ void store_tile_bf16(__bf16* dst, bool v_layout, int row, int half, int grp,
                                                const f32x16& acc) {
  u32x2 pk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = acc[4 * q + r];
    pk[q] = __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // Lanes 0-31 keep columns 16 p .. +3 and receive 16 p + 4 .. +7 from
    // lane + 32; lanes 32-63 receive 16 p + 8 .. +11 and keep 16 p + 12 .. +15.
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto r = __builtin_amdgcn_permlane32_swap(pk[2 * p][w], pk[2 * p + 1][w], false, false);
      out[w] = r[0];
      out[2 + w] = r[1];
    }
    const int chunk = 4 * half + 2 * p + grp;
    *(u32x4*)&dst[v_layout ? v_off(row, chunk) : k_off(row, chunk)] = out;
  }
}

// Waits until at most `later` stages issued after the current one are still
// in flight (LPS loads per stage and wave), i.e. the current stage landed.
template <int NS, int LPS>
__device__ __forceinline__ void wait_stage(int later) {
  if constexpr (NS >= 4) {
    if (later >= 2) { wait_vmcnt<2 * LPS>(); return; }
  }
  if constexpr (NS >= 3) {
    if (later >= 1) { wait_vmcnt<LPS>(); return; }
  }
  wait_vmcnt<0>();
}

template <bool CROSS, int NS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(NS == 1 ? 4 : 2, NS == 1 ? 4 : 2)))
void proj_attn_bf16_kernel(const ProjAttnArgs a) {
  constexpr int XT = ROWS * BKP;               // elements of one activation tile
  constexpr int WT = BKP * D;                  // elements of one weight tile
  constexpr int NX = CROSS ? 2 : 1;            // activation tiles per stage
  constexpr int STAGE = NX * XT + 3 * WT;      // elements per stage
  constexpr int XL = XT * 2 / 1024 / 8;        // 1 KB activation loads per wave and tile (2)
  constexpr int WL = 3 * WT * 2 / 1024 / 8;    // 1 KB weight loads per wave and stage (3)
  constexpr int LPS = NX * XL + WL;
  // The ring also holds the Q, K, V tiles after the projection.
  constexpr int RING = NS * STAGE > 3 * ROWS * D ? NS * STAGE : 3 * ROWS * D;

  __shared__ __attribute__((aligned(1024))) __bf16 ring[RING];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int grp = lane >> 5;

  // XCD-aware order: workgroups are dealt to the XCDs round-robin; unit
  // (b, head) = b*h + head is remapped so that each XCD owns a contiguous
  // run of units, i.e. whole batches: an activation row block is then read
  // into one XCD's L2 only.  When the run is made of whole batches, the
  // XCD's units are taken head by head (all of its batches for one head,
  // then the next head), so the workgroups resident together share few
  // heads' weight slices and their batches' rows, and later workgroups find
  // both in L2 (measured on the cross-attention block, whose XCD runs take
  // two rounds: 1.45x fewer bytes fetched from memory, same time).
  int bh;
  {
    const int T = a.B * a.h;
    const int bid = blockIdx.x;
    const int X = a.xcds > 0 ? a.xcds : 1;
    const int x = bid % X;
    const int per = T / X;
    const int rem = T - per * X;
    const int start = x * per + min(x, rem);
    const int len = per + (x < rem ? 1 : 0);
    const int j = bid / X;
    int u = start + j;
    if (len % a.h == 0 && start % a.h == 0) {
      const int nb = len / a.h;  // whole batches in this XCD's run
      u = start + (j % nb) * a.h + j / nb;
    }
    bh = __builtin_amdgcn_readfirstlane(u);
  }
  const int b = __builtin_amdgcn_readfirstlane(bh / a.h);
  const int hh = bh - b * a.h;
  const int dm = a.d_model;
  const int ldw = a.h * D;  // row stride of the stacked weights
  const int nsteps = dm / BKP;

  const char* xq = (const char*)a.Xq + (int64_t)b * a.n_q * dm * 2;
  const char* xkv = (const char*)a.Xkv + (int64_t)b * a.n_k * dm * 2;

  // DMA sources.  Activation load r of this wave fills block 2 wave + r of
  // a tile (rows 8 blk .. +7); weight load r fills block 3 wave + r of the
  // 24 weight blocks (block j: matrix j / 8, rows 8 (j % 8) .. +7).  Rows
  // past n read the last row (their results are never used).  Byte offsets
  // from the stage's scalar base.
  unsigned xq_off[XL], xkv_off[XL], w_off[WL];
  const char* w_src[WL];
#pragma unroll
  for (int r = 0; r < XL; ++r) {
    const int row = 8 * (XL * wave + r) + (lane >> 3);
    const int c = x_pos(row, lane & 7);
    xq_off[r] = (unsigned)(min(row, a.n_q - 1) * dm + 8 * c) * 2u;
    xkv_off[r] = (unsigned)(min(row, a.n_k - 1) * dm + 8 * c) * 2u;
  }
#pragma unroll
  for (int r = 0; r < WL; ++r) {
    const int j = WL * wave + r;
    const int row = 8 * (j & 7) + (lane >> 3);
    const int c = w_pos(row, lane & 7);
    const int mat = j >> 3;
    w_src[r] = (const char*)(mat == 0 ? a.Wq : (mat == 1 ? a.Wk : a.Wv));
    w_off[r] = (unsigned)(row * ldw + hh * D + 8 * c) * 2u;
  }
  const unsigned ring_lds = lds_addr(&ring[0]);
  auto issue = [&](int step, int buf) {
    const int k0 = step * BKP;
    const unsigned base = ring_lds + (unsigned)(buf * STAGE) * 2u;
#pragma unroll
    for (int r = 0; r < XL; ++r)
      dma16_s(xq + k0 * 2, xq_off[r], base + (unsigned)((XL * wave + r) * 1024));
    if constexpr (CROSS) {
#pragma unroll
      for (int r = 0; r < XL; ++r)
        dma16_s(xkv + k0 * 2, xkv_off[r], base + (unsigned)(XT * 2 + (XL * wave + r) * 1024));
    }
#pragma unroll
    for (int r = 0; r < WL; ++r)
      dma16_s(w_src[r] + (int64_t)k0 * ldw * 2, w_off[r],
              base + (unsigned)(NX * XT * 2 + (WL * wave + r) * 1024));
  };

  // This wave's three 32 x 32 output tiles: rows 32 rb .. +31, column
  // blocks cb0 .. cb0 + 2 of (Q0 Q1 K0 K1 V0 V1).
  const int rb = wave & 3;
  const int cb0 = 3 * (wave >> 2);
  f32x16 acc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) acc[c] = f32x16{};
  const int xrow = 32 * rb + col;
  const int tr_k = (lane & 15) >> 2;
  const int tr_n = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  auto compute = [&](const __bf16* st, const int ks_lo, const int ks_hi) {
    const __bf16* xs_q = st;
    const __bf16* xs_kv = CROSS ? st + XT : st;
#pragma unroll
    for (int ks = ks_lo; ks < ks_hi; ++ks) {
      const int xo = xrow * BKP + 8 * x_pos(xrow, 2 * ks + grp);
      const bf16x8 fq = *(const bf16x8*)&xs_q[xo];
      const bf16x8 fkv = CROSS ? *(const bf16x8*)&xs_kv[xo] : fq;
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const int cb = cb0 + c;  // wave-uniform
        const __bf16* ws = st + NX * XT + (cb >> 1) * WT;
        const int k = 16 * ks + 8 * grp + tr_k;
        const int n = 32 * (cb & 1) + tr_n;
        const i16x4 lo = tr_read(&ws[k * D + 8 * w_pos(k, n >> 3) + (n & 7)]);
        const i16x4 hi = tr_read(&ws[(k + 4) * D + 8 * w_pos(k + 4, n >> 3) + (n & 7)]);
        const bf16x8 wf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, cb < 2 ? fq : fkv, acc[c], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nsteps) issue(s, s);
  // The copies of a stage are issued by half of the waves (0-3) before the
  // stage's products and by the other half (4-7, the second wave of each
  // SIMD) halfway through them, so that the address unit drains one half's
  // copies while the other half multiplies.
  for (int t = 0; t < nsteps; ++t) {
    if constexpr (NS == 1) {
      // One stage buffer (two workgroups per compute unit): copy, wait,
      // multiply; the other workgroup's copies overlap this one's products.
      issue(t, 0);
      wait_vmcnt<0>();
      __syncthreads();
      compute(&ring[0], 0, BKP / 16);
      __syncthreads();  // every wave is done with the buffer before the next copy
    } else {
      wait_stage<NS, LPS>(min(NS - 2, nsteps - 1 - t));
      __syncthreads();
      const bool more = t + NS - 1 < nsteps;
      const __bf16* st = &ring[(t % NS) * STAGE];
      if (more && wave < 4) issue(t + NS - 1, (t + NS - 1) % NS);
      compute(st, 0, BKP / 32);
      if (more && wave >= 4) issue(t + NS - 1, (t + NS - 1) % NS);
      compute(st, BKP / 32, BKP / 16);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with the ring

  // Q, K, V tiles (bf16, rounded as the projection GEMM rounds) into the
  // ring: Q and K in the k_off layout, V in the v_off layout.
  __bf16* Qs = &ring[0];
  __bf16* Ks = &ring[ROWS * D];
  __bf16* Vs = &ring[2 * ROWS * D];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int cb = cb0 + c;
    const int mat = cb >> 1;
    store_tile_bf16(mat == 0 ? Qs : (mat == 1 ? Ks : Vs), mat == 2, xrow, cb & 1, grp, acc[c]);
  }
  __syncthreads();

  if (wave >= 4) return;  // n_q <= 128: four query blocks
  const int qw0 = 32 * wave;
  if (qw0 >= a.n_q) return;
  const int my_q = qw0 + col;
  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int lim = a.causal ? min(L, my_q + 1) : L;
  const int lim_min = __builtin_amdgcn_readfirstlane(a.causal ? min(L, qw0 + 1) : L);
  const int wv_last = min(qw0 + 32, a.n_q) - 1;
  const int wv_keys = __builtin_amdgcn_readfirstlane(a.causal ? min(L, wv_last + 1) : L);
  WaveAttention wa;
  wa.init(lane, a.scale);
  wa.load_q_lds(Qs, min(my_q, a.n_q - 1));
#pragma unroll
  for (int t = 0; t < ROWS / KT; ++t)
    if (t * KT < wv_keys) wa.tile(Ks + t * KT * D, Vs + t * KT * D, t * KT, lim, lim_min);
  const float inv = wa.inv_sum();
  wa.store((__bf16*)a.O + ((int64_t)b * a.n_q + min(my_q, a.n_q - 1)) * ldw + hh * D, inv, my_q < a.n_q);
}

// Two heads per workgroup, for launches with more (batch, head) units than
// compute units (a unit per workgroup would give two workgroups per unit
// with one stage buffer each).  Workgroup (b, pair p) computes Q_i = X_q,b
// W^Q_i, K_i = X_kv,b W^K_i and V_i = X_kv,b W^V_i for heads i = 2p, 2p + 1:
// the activation tiles of a k stage are copied into LDS once for both heads
// (per unit 40 KB instead of 56 KB a stage in cross-attention), and each
// wave computes a 64 x 96 block of the [128 x 384] result (two row blocks,
// three column blocks), which reads fewer LDS bytes per product than a
// 32 x 96 block.  Per output element: the same products in the same k order
// as the one-head kernel and the projection GEMM, the same bf16 rounding.
// Then waves 0-3 attend head 2p and waves 4-7 head 2p + 1.  Two 80 KB stages
// (all of LDS for cross-attention), one stage in flight during the products
// of the other.  In cross-attention, X_q row blocks past n_q are not copied:
// the query rows they give are never read (self-attention copies every row,
// clamped, since the same rows give K and V, whose rows past n_k must stay
// finite for the masked products).
template <bool CROSS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void proj_attn2_bf16_kernel(const ProjAttnArgs a) {
  constexpr int NS = 2;
  constexpr int XT = ROWS * BKP;               // elements of one activation tile
  constexpr int WT = BKP * D;                  // elements of one weight tile
  constexpr int NX = CROSS ? 2 : 1;            // activation tiles per stage
  constexpr int NWT = 6;                       // weight tiles per stage: (Q, K, V) x 2 heads
  constexpr int STAGE = NX * XT + NWT * WT;    // elements per stage
  constexpr int XL = XT * 2 / 1024 / 8;        // 1 KB activation loads per wave and tile (2)
  constexpr int WL = NWT * WT * 2 / 1024 / 8;  // 1 KB weight loads per wave and stage (6)
  // The ring also holds both heads' Q, K, V tiles after the projection.
  constexpr int RING = NS * STAGE > 6 * ROWS * D ? NS * STAGE : 6 * ROWS * D;

  __shared__ __attribute__((aligned(1024))) __bf16 ring[RING];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int grp = lane >> 5;
  const int pairs = a.h >> 1;

  // XCD-aware order: workgroups are dealt to the XCDs round-robin.  When
  // the units divide evenly, XCD x owns a block of batches and a block of
  // head pairs (two head-pair blocks when they divide: each XCD then reads
  // a quarter of the activations and half of the weights into its L2,
  // instead of an eighth and all of them), else a contiguous run of units.
  int u;
  {
    const int T = a.B * pairs;
    const int bid = blockIdx.x;
    const int X = a.xcds > 0 ? a.xcds : 1;
    u = bid;
    if (T % X == 0) {
      const int x = bid % X;
      const int j = bid / X;
      const int g = (X % 2 == 0 && pairs % 2 == 0 && a.B % (X / 2) == 0) ? 2 : (a.B % X == 0 ? 1 : 0);
      if (g > 0) {
        const int nb = a.B / (X / g);  // batches per XCD
        const int np = pairs / g;      // head pairs per XCD
        u = ((x / g) * nb + j / np) * pairs + (x % g) * np + j % np;
      } else {
        u = x * (T / X) + j;
      }
    }
    u = __builtin_amdgcn_readfirstlane(u);
  }
  const int b = __builtin_amdgcn_readfirstlane(u / pairs);
  const int hp = u - b * pairs;
  const int dm = a.d_model;
  const int ldw = a.h * D;  // row stride of the stacked weights
  const int nsteps = dm / BKP;

  const char* xq = (const char*)a.Xq + (int64_t)b * a.n_q * dm * 2;
  const char* xkv = (const char*)a.Xkv + (int64_t)b * a.n_k * dm * 2;

  // DMA sources.  Activation load r of this wave fills block XL wave + r of
  // a tile (rows 8 blk .. +7; in cross-attention X_q blocks at or past n_q
  // are skipped); weight load r fills block WL wave + r of the 48 weight
  // blocks (block j: tile j / 8 = (head, matrix) = ((j / 8) / 3, (j / 8) % 3),
  // rows 8 (j % 8) .. +7).
  unsigned xq_off[XL], xkv_off[XL], w_off[WL];
  const char* w_src[WL];
#pragma unroll
  for (int r = 0; r < XL; ++r) {
    const int row = 8 * (XL * wave + r) + (lane >> 3);
    const int c = x_pos(row, lane & 7);
    xq_off[r] = (unsigned)(min(row, a.n_q - 1) * dm + 8 * c) * 2u;
    xkv_off[r] = (unsigned)(min(row, a.n_k - 1) * dm + 8 * c) * 2u;
  }
#pragma unroll
  for (int r = 0; r < WL; ++r) {
    const int j = WL * wave + r;
    const int row = 8 * (j & 7) + (lane >> 3);
    const int c = w_pos(row, lane & 7);
    const int t = j >> 3;
    const int mat = t % 3;
    w_src[r] = (const char*)(mat == 0 ? a.Wq : (mat == 1 ? a.Wk : a.Wv));
    w_off[r] = (unsigned)(row * ldw + (2 * hp + t / 3) * D + 8 * c) * 2u;
  }
  const unsigned ring_lds = lds_addr(&ring[0]);
  auto issue = [&](int step, int buf) {
    const int k0 = step * BKP;
    const unsigned base = ring_lds + (unsigned)(buf * STAGE) * 2u;
#pragma unroll
    for (int r = 0; r < XL; ++r)
      if (!CROSS || 8 * (XL * wave + r) < a.n_q)
        dma16_s(xq + k0 * 2, xq_off[r], base + (unsigned)((XL * wave + r) * 1024));
    if constexpr (CROSS) {
#pragma unroll
      for (int r = 0; r < XL; ++r)
        dma16_s(xkv + k0 * 2, xkv_off[r], base + (unsigned)(XT * 2 + (XL * wave + r) * 1024));
    }
#pragma unroll
    for (int r = 0; r < WL; ++r)
      dma16_s(w_src[r] + (int64_t)k0 * ldw * 2, w_off[r],
              base + (unsigned)(NX * XT * 2 + (WL * wave + r) * 1024));
  };

  // This wave's six 32 x 32 output tiles: row blocks 2 rh, 2 rh + 1 and
  // column blocks 3 cg .. 3 cg + 2 of the twelve (Q0 Q1 K0 K1 V0 V1 of head
  // 2p, then the same six of head 2p + 1).  Column block cb reads weight
  // tile cb / 2.
  // The first two column blocks of a wave are both Q blocks (cg even) or
  // both K/V blocks (cg odd); the third is always a K/V block.  So the
  // products take activation fragments fa (X_q or X_kv, a wave-uniform
  // choice of tile) and fb (X_kv): the loop is straight-line code, with no
  // branch between the LDS reads and the products.
  const int rh = wave & 1;
  const int cg = wave >> 1;
  const bool q_first = (cg & 1) == 0;
  f32x16 acc[2][3];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int c = 0; c < 3; ++c) acc[rr][c] = f32x16{};
  const int tr_k = (lane & 15) >> 2;
  const int tr_n = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  auto compute = [&](const __bf16* st, const int ks_lo, const int ks_hi) {
    const __bf16* xs_kv = CROSS ? st + XT : st;
    const __bf16* xs_a = (CROSS && q_first) ? st : xs_kv;
#pragma unroll
    for (int ks = ks_lo; ks < ks_hi; ++ks) {
      bf16x8 fa[2], fb[2], wf[3];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int xrow = 64 * rh + 32 * rr + col;
        const int xo = xrow * BKP + 8 * x_pos(xrow, 2 * ks + grp);
        fa[rr] = *(const bf16x8*)&xs_a[xo];
        fb[rr] = *(const bf16x8*)&xs_kv[xo];
      }
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const int cb = 3 * cg + c;  // wave-uniform
        const __bf16* ws = st + NX * XT + (cb >> 1) * WT;
        const int k = 16 * ks + 8 * grp + tr_k;
        const int n = 32 * (cb & 1) + tr_n;
        const i16x4 lo = tr_read(&ws[k * D + 8 * w_pos(k, n >> 3) + (n & 7)]);
        const i16x4 hi = tr_read(&ws[(k + 4) * D + 8 * w_pos(k + 4, n >> 3) + (n & 7)]);
        wf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          acc[rr][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[c], c < 2 ? fa[rr] : fb[rr], acc[rr][c], 0, 0, 0);
    }
  };

  issue(0, 0);
  // Stage t + 1 is copied while stage t is multiplied: waves 0-3 issue its
  // copies before the products, waves 4-7 halfway through them, so that the
  // address unit drains one half's copies while the other half multiplies.
  for (int t = 0; t < nsteps; ++t) {
    wait_vmcnt<0>();  // this wave's copies of stage t have landed
    __syncthreads();  // ... and every wave's; stage t - 1's buffer is free
    const bool more = t + 1 < nsteps;
    const __bf16* st = &ring[(t & 1) * STAGE];
    if (more && wave < 4) issue(t + 1, (t + 1) & 1);
    compute(st, 0, BKP / 32);
    if (more && wave >= 4) issue(t + 1, (t + 1) & 1);
    compute(st, BKP / 32, BKP / 16);
  }
  __syncthreads();  // every wave is done with the ring

  // Q, K, V tiles of both heads (bf16, rounded as the projection GEMM
  // rounds) into the ring: head j's Q, K, V at tiles 3 j, 3 j + 1, 3 j + 2,
  // Q and K in the k_off layout, V in the v_off layout.
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int cb = 3 * cg + c;
    const int mat = (cb % 6) >> 1;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
      store_tile_bf16(&ring[(cb >> 1) * ROWS * D], mat == 2, 64 * rh + 32 * rr + col, cb & 1, grp, acc[rr][c]);
  }
  __syncthreads();

  // n_q <= 128: four query blocks per head.
  const int head = wave >> 2;
  const int qw0 = 32 * (wave & 3);
  if (qw0 >= a.n_q) return;
  const __bf16* Qs = &ring[3 * head * ROWS * D];
  const __bf16* Ks = Qs + ROWS * D;
  const __bf16* Vs = Ks + ROWS * D;
  const int my_q = qw0 + col;
  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int lim = a.causal ? min(L, my_q + 1) : L;
  const int lim_min = __builtin_amdgcn_readfirstlane(a.causal ? min(L, qw0 + 1) : L);
  const int wv_last = min(qw0 + 32, a.n_q) - 1;
  const int wv_keys = __builtin_amdgcn_readfirstlane(a.causal ? min(L, wv_last + 1) : L);
  WaveAttention wa;
  wa.init(lane, a.scale);
  wa.load_q_lds(Qs, min(my_q, a.n_q - 1));
#pragma unroll
  for (int t = 0; t < ROWS / KT; ++t)
    if (t * KT < wv_keys) wa.tile(Ks + t * KT * D, Vs + t * KT * D, t * KT, lim, lim_min);
  const float inv = wa.inv_sum();
  wa.store((__bf16*)a.O + ((int64_t)b * a.n_q + min(my_q, a.n_q - 1)) * ldw + (2 * hp + head) * D, inv,
           my_q < a.n_q);
}

template <bool CROSS>
hipError_t launch2(const ProjAttnArgs& a0, hipStream_t s, LaunchEvents ev) {
  ProjAttnArgs a = a0;
  a.xcds = device_xcds();
  void* args[] = {(void*)&a};
  return launch_kernel((const void*)proj_attn2_bf16_kernel<CROSS>, dim3(a.B * (a.h / 2)), dim3(512),
                       args, 0, s, ev.start, ev.stop, 0);
}

template <bool CROSS, int NS>
hipError_t launch(const ProjAttnArgs& a0, hipStream_t s, LaunchEvents ev) {
  ProjAttnArgs a = a0;
  a.xcds = device_xcds();
  void* args[] = {(void*)&a};
  return launch_kernel((const void*)proj_attn_bf16_kernel<CROSS, NS>, dim3(a.B * a.h), dim3(512),
                            args, 0, s, ev.start, ev.stop, 0);
}

}  // namespace

bool proj_attn_supported(int n_q, int n_k, int d_model) {
  return n_q <= ROWS && n_k <= ROWS && d_model % BKP == 0;
}

hipError_t launch_proj_attn_bf16(const ProjAttnArgs& a, hipStream_t s, LaunchEvents ev) {
  if (!proj_attn_supported(a.n_q, a.n_k, a.d_model)) return hipErrorInvalidValue;
  const bool self = a.Xq == a.Xkv && a.n_q == a.n_k;
  // More (batch, head) units than compute units: with an even head count,
  // two heads per workgroup (proj_attn2_bf16_kernel: the cross-attention
  // block's fused kernel 38.4 -> 32.0 us); with an odd one, one head per
  // workgroup and one stage buffer, so that two workgroups share a unit and
  // one's copies overlap the other's products (that block, 512 workgroups:
  // 49 -> 39 us against the deep ring).  Otherwise one workgroup per unit
  // with a deep ring: four 40 KB stages (all 160 KB of LDS) for
  // self-attention, measured 3% faster than three; two 56 KB stages for
  // cross-attention.
  if ((int64_t)a.B * a.h > device_compute_units()) {
    if (a.h % 2 == 0) return self ? launch2<false>(a, s, ev) : launch2<true>(a, s, ev);
    return self ? launch<false, 1>(a, s, ev) : launch<true, 1>(a, s, ev);
  }
  return self ? launch<false, 4>(a, s, ev) : launch<true, 2>(a, s, ev);
}

}  // namespace mha
