// Projection GEMM for the multi-head block, bf16 in / bf16 out, fp32
// accumulation, for gfx950.
//
//   C[M][N] = A[M][K] . [W_0 | W_1 | W_2]          (W_s row-major [K][width_s])
//
// Used for the input projections Q = X W^Q, K = X W^K, V = X W^V
// (devpress.csdn.net "【深度学习】Transformer", section 2.1, equations
// (2.1)-(2.3); hex4c59.cc "读懂 Attention Is All You Need", section
// "Q、K、V 是三种计算角色") -- all three stacked into one launch for
// self-attention -- and for the output projection Concat . W^O
// (devpress.csdn.net section 2.2).  The epilogue scatters each column
// segment per head (head i = column block i, as in the pages' head split),
// so the projection writes Q, K, V directly in the [B][h][n][d] layout the
// attention kernel streams, and the output projection writes Y row-major.
//
// Tiling: WM x WN waves (2 x 2 or 2 x 4); a BM x BN output tile, each wave a
// (BM/WM) x (BN/WN) block of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16).
// K advances 64 per stage.  Stages go from global memory straight into LDS
// (global_load_lds_dwordx4: no register staging) through a ring of NS
// buffers, NS-1 stages ahead of the one being multiplied, one barrier per
// stage.  Both tiles keep their global row-major layout in LDS, with 16-byte
// chunks XOR-swizzled so that the operand reads are free of bank conflicts:
// the activation operand (8 consecutive k of one row per lane) is one
// 16-byte read, the weight operand (8 consecutive k of one column) two
// transposing reads (ds_read_b64_tr_b16).
//
// The products are computed transposed, C^T = W^T A^T: the weight fragment
// is the MFMA's first operand.  A lane then holds, for one output row, four
// runs of 4 consecutive columns, which it stores as 8-byte vectors.
//
// Tile order: workgroups are dealt to the XCDs round-robin (8 on MI355X; the
// launchers read the count from the device); the linear
// workgroup id is remapped so that each XCD owns a contiguous band of the
// row-major tile order (whole rows of tiles), i.e. each XCD's L2 streams its
// own band of activation rows and the (small) weight matrix, instead of
// every XCD reading every activation row.
#include "device.h"

namespace mha {
namespace {

using namespace dev;

constexpr int BK = 64;

// A tile [BM][64]: 128-byte rows; chunk c of row m sits at chunk c ^ ((m >> 1) & 7).
__device__ __forceinline__ int a_pos(int m, int chunk) { return chunk ^ ((m >> 1) & 7); }
// W tile [64][BN]: BN = 128 -> 256-byte rows, chunk c of row k at c ^ ((k & 3) << 2);
// BN = 64 -> 128-byte rows, chunk c of row k at c ^ (((k >> 1) & 1) << 2).
template <int BN>
__device__ __forceinline__ int b_pos(int k, int chunk) {
  if constexpr (BN >= 128) return chunk ^ ((k & 3) << 2);
  else return chunk ^ (((k >> 1) & 1) << 2);
}

// Waits until at most `later` stages issued after the current one are still
// in flight (LPS loads per stage and wave), i.e. the current stage landed.
template <int LPS, int NS>
__device__ __forceinline__ void wait_stage(int later) {
  if constexpr (NS >= 4) {
    if (later >= 2) { wait_vmcnt<2 * LPS>(); return; }
  }
  if constexpr (NS >= 3) {
    if (later >= 1) { wait_vmcnt<LPS>(); return; }
  }
  wait_vmcnt<0>();
}

// Segment of column n and its fields, selected without indexing the argument
// array dynamically (which would spill it to memory).
__device__ __forceinline__ int seg_of(const GemmArgs& g, int n) {
  return (g.nseg > 1 && n >= g.col_start[1]) + (g.nseg > 2 && n >= g.col_start[2]);
}
template <typename T>
__device__ __forceinline__ T seg_field(const GemmArgs& g, int s, T GemmSeg::*f) {
  return s == 0 ? g.seg[0].*f : (s == 1 ? g.seg[1].*f : g.seg[2].*f);
}
__device__ __forceinline__ const void* seg_ptr(const GemmArgs& g, int s) {
  return seg_field(g, s, &GemmSeg::W);
}
__device__ __forceinline__ int seg_start(const GemmArgs& g, int s) {
  return s == 0 ? g.col_start[0] : (s == 1 ? g.col_start[1] : g.col_start[2]);
}

// One output tile (or one k range of one tile, split-K) of the GEMM g;
// bid is the workgroup's index within the GEMM's own grid.
template <int BM, int BN, int NS, int WM, int WN>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const int bid_in) {
  static_assert(BM == 64 || BM == 128 || BM == 256, "tile rows");
  static_assert(BN == 64 || BN == 128 || BN == 256, "tile columns");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  constexpr int NWAVE = WM * WN;
  constexpr int MB = BM / WM / 32;     // 32-row MFMA tiles per wave
  constexpr int NB = BN / WN / 32;     // 32-column MFMA tiles per wave
  static_assert(MB >= 1 && NB >= 1, "wave tile of at least 32 x 32");
  constexpr int AL = BM * BK * 2 / 1024 / NWAVE;   // 1 KB A loads per wave and stage
  constexpr int BL = BK * BN * 2 / 1024 / NWAVE;   // 1 KB W loads per wave and stage
  static_assert(AL >= 1 && BL >= 1, "every wave loads part of each tile");
  constexpr int LPS = AL + BL;
  constexpr int BROW = BN / 8;                 // 16-byte chunks per W row

  __shared__ __attribute__((aligned(1024))) __bf16 As[NS][BM * BK];
  __shared__ __attribute__((aligned(1024))) __bf16 Bs[NS][BK * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int grp = lane >> 5;
  const int wm = wave / WN;
  const int wn = wave % WN;

  const int N = g.col_start[g.nseg];
  const int MT = (g.M + BM - 1) / BM;
  const int NT = (N + BN - 1) / BN;
  // XCD-aware tile order (see the file comment).  Split-K launches are 1-D
  // over (tile, split) with the split fastest: workgroups are dealt to the
  // XCDs round-robin, so with 8 splits each XCD owns one k range of both
  // operands for every tile, a slice its L2 holds.
  int tile, split = 0;
  if (g.splits > 1) {
    tile = bid_in / g.splits;
    split = bid_in - tile * g.splits;
  } else {
    const int T = MT * NT;
    const int bid = bid_in;
    const int X = g.xcds > 0 ? g.xcds : 1;
    const int x = bid % X;
    const int per = T / X;
    const int rem = T - per * X;
    tile = x * per + min(x, rem) + bid / X;
  }
  const int m0 = (tile / NT) * BM;
  const int n0 = (tile % NT) * BN;
  // Split-K (g.splits > 1): the workgroup of split z takes k stages
  // [s_first, s_first + nsteps) of the total and writes fp32 partial sums.
  const int total_steps = (g.K + BK - 1) / BK;
  int s_first = 0, nsteps = total_steps;
  if (g.splits > 1) {
    const int per = (total_steps + g.splits - 1) / g.splits;
    s_first = min(split * per, total_steps);
    nsteps = min(per, total_steps - s_first);
  }
  const bool ktail = (g.K % BK) != 0;  // the last stage reaches past K

  // The tile's columns lie in one segment (segment starts are multiples of BN).
  const int sg = seg_of(g, n0);
  const int wwidth = seg_field(g, sg, &GemmSeg::width);
  const int ldw_s = seg_field(g, sg, &GemmSeg::ldw);
  const int wstride = ldw_s > 0 ? ldw_s : wwidth;  // row stride of the segment's weight
  const int ncol0 = n0 - seg_start(g, sg);  // first tile column within the segment
  const char* a_tile = (const char*)g.A + (int64_t)m0 * g.K * 2;
  const char* w_seg = (const char*)seg_ptr(g, sg);

  // DMA sources.  A load r of this wave fills LDS block (wave*AL + r): rows
  // 8 blk .. +7, lane l -> row 8 blk + l/8, stored chunk l%8, which holds the
  // source chunk the swizzle maps there.  Rows past M read the last row
  // (never stored).  W load r fills LDS block (wave*BL + r): 1024 / (2 BN)
  // rows of BN columns; columns past the segment read its last chunk (never
  // stored).  Offsets are bytes from the stage's scalar base.
  unsigned a_voff[AL], w_voff[BL];
  int a_kc[AL], w_row[BL], w_col[BL];
#pragma unroll
  for (int r = 0; r < AL; ++r) {
    const int row = 8 * (wave * AL + r) + (lane >> 3);
    a_kc[r] = 8 * a_pos(row, lane & 7);
    a_voff[r] = (unsigned)((min(m0 + row, g.M - 1) - m0) * g.K + a_kc[r]) * 2u;
  }
#pragma unroll
  for (int r = 0; r < BL; ++r) {
    const int row = (wave * BL + r) * (1024 / (2 * BN)) + lane / BROW;
    w_row[r] = row;
    w_col[r] = min(ncol0 + 8 * b_pos<BN>(row, lane % BROW), wwidth - 8);
    w_voff[r] = (unsigned)(row * wstride + w_col[r]) * 2u;
  }
  // LDS byte addresses of the two rings (wave-uniform, computed once).
  const unsigned as_lds = lds_addr(&As[0][0]);
  const unsigned bs_lds = lds_addr(&Bs[0][0]);
  auto issue = [&](int step, int buf) {
    const int k0 = (s_first + step) * BK;
    const unsigned a_dst = as_lds + (unsigned)(buf * BM * BK + wave * AL * 512) * 2u;
    const unsigned b_dst = bs_lds + (unsigned)(buf * BK * BN + wave * BL * 512) * 2u;
    if (!ktail || k0 + BK <= g.K) {
      const char* ab = a_tile + k0 * 2;
      const char* wb = w_seg + (int64_t)k0 * wstride * 2;
#pragma unroll
      for (int r = 0; r < AL; ++r) dma16_s(ab, a_voff[r], a_dst + 1024u * r);
#pragma unroll
      for (int r = 0; r < BL; ++r) dma16_s(wb, w_voff[r], b_dst + 1024u * r);
    } else {  // last stage of a K that is not a multiple of 64: clamp per lane
#pragma unroll
      for (int r = 0; r < AL; ++r) {
        const unsigned o = a_voff[r] + 2u * (unsigned)(min(k0 + a_kc[r], g.K - 8) - a_kc[r]);
        dma16_s(a_tile, o, a_dst + 1024u * r);
      }
      const char* wb = w_seg + (int64_t)k0 * wstride * 2;  // the stage's first weight row
#pragma unroll
      for (int r = 0; r < BL; ++r) {
        const unsigned o = (unsigned)((min(k0 + w_row[r], g.K - 1) - k0) * wstride + w_col[r]) * 2u;
        dma16_s(wb, o, b_dst + 1024u * r);
      }
    }
  };

  // The last stage of a K that is not a multiple of 64 loaded clamped
  // addresses past K; once it has landed, every lane clears the 16-byte
  // chunks it loaded there, so those k contribute exact zeros.
  auto zero_past_k = [&](int step, int buf) {
    const int k0 = (s_first + step) * BK;
#pragma unroll
    for (int r = 0; r < AL; ++r)
      if (k0 + a_kc[r] >= g.K) *(u32x4*)&As[buf][(wave * AL + r) * 512 + 8 * lane] = u32x4{};
#pragma unroll
    for (int r = 0; r < BL; ++r)
      if (k0 + w_row[r] >= g.K) *(u32x4*)&Bs[buf][(wave * BL + r) * 512 + 8 * lane] = u32x4{};
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  // LDS read offsets (elements within a stage), fixed across stages.
  // Activation operand: row wm*BM/2 + 32i + col, chunk 2ks + grp.  Weight
  // operand (transposing read): within each 16-lane group, lane s addresses
  // row (s / 4) and columns 4 (s % 4) .. +3.
  int x_off[MB][BK / 16];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = wm * (BM / WM) + 32 * i + col;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) x_off[i][ks] = row * BK + 8 * a_pos(row, 2 * ks + grp);
  }
  const int tr_k = (lane & 15) >> 2;
  const int tr_n = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int w_off[NB][BK / 16][2];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = wn * (BN / WN) + 32 * j + tr_n;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int k = 16 * ks + 8 * grp + tr_k;
      w_off[j][ks][0] = k * BN + 8 * b_pos<BN>(k, n >> 3) + (n & 7);
      w_off[j][ks][1] = (k + 4) * BN + 8 * b_pos<BN>(k + 4, n >> 3) + (n & 7);
    }
  }

  auto compute = [&](const __bf16* as, const __bf16* bs) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 xf[MB], wf[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) xf[i] = *(const bf16x8*)&as[x_off[i][ks]];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const i16x4 lo = tr_read(&bs[w_off[j][ks][0]]);
        const i16x4 hi = tr_read(&bs[w_off[j][ks][1]]);
        wf[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nsteps) issue(s, s);

  // The ring index is a compile-time constant in each unrolled copy, so every
  // LDS address is a per-lane offset plus an immediate.
  for (int t0 = 0; t0 < nsteps; t0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int t = t0 + u;
      if (t < nsteps) {
        wait_stage<LPS, NS>(min(NS - 2, nsteps - 1 - t));
        if (ktail && s_first + t == total_steps - 1) zero_past_k(t, u);
        __syncthreads();
        if (t + NS - 1 < nsteps) issue(t + NS - 1, (u + NS - 1) % NS);
        compute(As[u], Bs[u]);
      }
    }
  }

  // acc[i][j][e] = C[m][n], m = m0 + wm*BM/2 + 32i + col,
  //                         n = n0 + wn*BN/2 + 32j + 8(e/4) + 4grp + e%4.
  if (g.splits > 1) {  // fp32 partial sums of this k range: partial[z][m][n]
    float* part = g.partial + (int64_t)split * g.M * N;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int nb = n0 + wn * (BN / WN) + 32 * j;
      if (nb >= N) continue;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = m0 + wm * (BM / WM) + 32 * i + col;
        if (m >= g.M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (nb + 8 * q >= N) continue;
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
          *(f32x4*)(part + (int64_t)m * N + nb + 8 * q + 4 * grp) = v;
        }
      }
    }
    return;
  }
  // A 32-column block lies in one segment and one head (segment widths and
  // head widths are multiples of 32 unless there is a single segment with a
  // single head), so its destination is fixed per block; N is a multiple of 8.
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int nb = n0 + wn * (BN / WN) + 32 * j;  // wave-uniform
    if (nb >= N) continue;
    const int s = seg_of(g, nb);
    const int rows = seg_field(g, s, &GemmSeg::rows);
    const int hd = seg_field(g, s, &GemmSeg::hd);
    const int heads = seg_field(g, s, &GemmSeg::heads);
    const int c = nb - seg_start(g, s);
    const int head = heads == 1 ? 0 : c / hd;
    __bf16* base = (__bf16*)seg_field(g, s, &GemmSeg::dst) + (int64_t)head * rows * hd + (c - head * hd);
    const int64_t bstride = (int64_t)heads * rows * hd;
    // Bias of this lane's columns nb + 8q + 4grp .. +3 (zero without one).
    // The four loads are issued together (columns clamped into the row; a
    // block past N is never stored), so their latencies overlap.
    f32x4 bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bq[q] = f32x4{};
    if (g.bias != nullptr) {
      bf16x4 braw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        braw[q] = *(const bf16x4*)((const __bf16*)g.bias + min(nb + 8 * q + 4 * grp, N - 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) bq[q] = __builtin_convertvector(braw[q], f32x4);
    }
    // Lanes l and l + 32 hold the two halves (4 columns each) of every
    // 16-byte chunk of row m; one permlane32 swap per register gives each
    // lane a whole chunk (lane l chunk 2p, lane l + 32 chunk 2p + 1), so the
    // row goes out in 16-byte stores -- half the store instructions of
    // 8-byte ones, measured 13% faster on the decoder block's projection.
    // The swaps run with every lane active; only the stores are predicated.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + wm * (BM / WM) + 32 * i + col;
      const int mc = min(m, g.M - 1);
      const int bb = mc / rows;
      const int pos = mc - bb * rows;
      __bf16* dst = base + bb * bstride + (int64_t)pos * hd;
      u32x2 pk[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][j][4 * q + r] + bq[q][r];
          if (g.relu) v[r] = fmaxf(v[r], 0.f);
        }
        pk[q] = __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const auto sw = __builtin_amdgcn_permlane32_swap(pk[2 * p][w], pk[2 * p + 1][w], false, false);
          out[w] = sw[0];
          out[2 + w] = sw[1];
        }
        const int cc = 16 * p + 8 * grp;  // this lane's chunk: columns nb + cc .. +7
        if (m < g.M && nb + cc < N) *(u32x4*)(dst + cc) = out;
      }
    }
  }
}

template <int BM, int BN, int NS, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(const GemmArgs g) {
  gemm_tile<BM, BN, NS, WM, WN>(g, (int)blockIdx.x);
}

template <int BM, int BN, int NS, int WM = 2, int WN = 2>
hipError_t launch_tile(const GemmArgs& g0, hipStream_t s, LaunchEvents ev) {
  GemmArgs g = g0;
  g.xcds = device_xcds();
  const int N = g.col_start[g.nseg];
  const int tiles = ((N + BN - 1) / BN) * ((g.M + BM - 1) / BM);
  void* args[] = {(void*)&g};
  return launch_kernel((const void*)gemm_bf16_kernel<BM, BN, NS, WM, WN>,
                            dim3(tiles * (g.splits > 1 ? g.splits : 1)), dim3(64 * WM * WN), args, 0, s,
                            ev.start, ev.stop, 0);
}

// Sum of the split-K partials, rounded once to bf16 and written to the
// segments (plain row-major outputs).  One thread per 8 columns.
__device__ __forceinline__ void splitk_reduce(const GemmArgs& g, const int bid) {
  const int N = g.col_start[g.nseg];
  const int chunks = N / 8;
  const int64_t idx = (int64_t)bid * 256 + threadIdx.x;
  if (idx >= (int64_t)g.M * chunks) return;
  const int m = (int)(idx / chunks);
  const int n = (int)(idx - (int64_t)m * chunks) * 8;
  f32x4 a = {}, b = {};
  for (int z = 0; z < g.splits; ++z) {
    const float* p = g.partial + ((int64_t)z * g.M + m) * N + n;
    a += *(const f32x4*)p;
    b += *(const f32x4*)(p + 4);
  }
  f32x8 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = a[r];
    v[4 + r] = b[r];
  }
  const int sg = seg_of(g, n);
  const int width = seg_field(g, sg, &GemmSeg::width);
  __bf16* dst = (__bf16*)seg_field(g, sg, &GemmSeg::dst) + (int64_t)m * width + (n - seg_start(g, sg));
  *(bf16x8*)dst = __builtin_convertvector(v, bf16x8);
}

__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const GemmArgs g) {
  splitk_reduce(g, (int)blockIdx.x);
}

// Independent jobs of one launch (GemmGroup): job j owns workgroups
// [start[j], start[j] + count[j]); starts are multiples of 8, so that the
// XCD a workgroup lands on is the one the job's own tile order assumes.
// Workgroups between jobs (padding) return at once.
__global__ __launch_bounds__(256) void gemm_group_kernel(const GemmGroup gg) {
  const int b = (int)blockIdx.x;
  int j = -1;
#pragma unroll
  for (int i = 0; i < kMaxGroupJobs; ++i)
    if (i < gg.n && b >= gg.start[i] && b < gg.start[i] + gg.count[i]) j = i;
  j = __builtin_amdgcn_readfirstlane(j);
  if (j < 0) return;
  const GemmArgs& g = j == 0 ? gg.job[0] : (j == 1 ? gg.job[1] : gg.job[2]);
  const int rb = b - (j == 0 ? gg.start[0] : (j == 1 ? gg.start[1] : gg.start[2]));
  const int red = j == 0 ? gg.reduce[0] : (j == 1 ? gg.reduce[1] : gg.reduce[2]);
  if (red) splitk_reduce(g, rb);
  else gemm_tile<64, 64, 3, 2, 2>(g, rb);
}

// Every segment must start on a multiple of the tile width (a tile's columns
// lie in one segment) and N must be a multiple of 8.
bool tiles_fit(const GemmArgs& g, int bn) {
  for (int s = 0; s < g.nseg; ++s)
    if (g.col_start[s] % bn != 0) return false;
  return g.col_start[g.nseg] % 8 == 0 && g.K % 8 == 0;
}

}  // namespace

hipError_t launch_gemm_bf16_cfg(const GemmArgs& g, int cfg, hipStream_t s, LaunchEvents ev) {
  static const int kBN[] = {128, 128, 128, 128, 128, 64, 64, 64, 64, 128, 128, 128, 64, 256, 128};
  if (cfg < 0 || cfg > 14 || !tiles_fit(g, kBN[cfg])) return hipErrorInvalidValue;
  switch (cfg) {
    case 0: return launch_tile<128, 128, 2>(g, s, ev);
    case 1: return launch_tile<128, 128, 3>(g, s, ev);
    case 2: return launch_tile<64, 128, 2>(g, s, ev);
    case 3: return launch_tile<64, 128, 3>(g, s, ev);
    case 4: return launch_tile<64, 128, 4>(g, s, ev);
    case 5: return launch_tile<128, 64, 3>(g, s, ev);
    case 6: return launch_tile<64, 64, 3>(g, s, ev);
    case 7: return launch_tile<64, 64, 4>(g, s, ev);
    case 8: return launch_tile<128, 64, 4>(g, s, ev);
    case 9: return launch_tile<128, 128, 2, 2, 4>(g, s, ev);
    case 10: return launch_tile<128, 128, 3, 2, 4>(g, s, ev);
    case 11: return launch_tile<64, 128, 2, 2, 4>(g, s, ev);
    case 13: return launch_tile<256, 256, 2, 4, 4>(g, s, ev);
    case 14: return launch_tile<256, 128, 3, 4, 2>(g, s, ev);
    default: return launch_tile<128, 64, 2, 4, 2>(g, s, ev);
  }
}

hipError_t launch_gemm_bf16_group(GemmGroup gg, hipStream_t s, LaunchEvents ev) {
  if (gg.n < 1 || gg.n > kMaxGroupJobs) return hipErrorInvalidValue;
  const int X = device_xcds();  // each job starts on a multiple of it: its own XCD-aware order
  int next = 0;
  for (int j = 0; j < gg.n; ++j) {
    const GemmArgs& g = gg.job[j];
    const int N = g.col_start[g.nseg];
    int64_t cnt;
    if (gg.reduce[j]) {
      if (g.splits < 2 || g.partial == nullptr || N % 8 != 0) return hipErrorInvalidValue;
      cnt = ((int64_t)g.M * (N / 8) + 255) / 256;
    } else {
      if (!tiles_fit(g, 64)) return hipErrorInvalidValue;
      if (g.splits > 1) {
        if (g.partial == nullptr || g.bias != nullptr || g.relu) return hipErrorInvalidValue;
        for (int sg = 0; sg < g.nseg; ++sg)
          if (g.seg[sg].heads != 1 || g.seg[sg].width % 8 != 0) return hipErrorInvalidValue;
      }
      cnt = (int64_t)((N + 63) / 64) * ((g.M + 63) / 64) * (g.splits > 1 ? g.splits : 1);
    }
    gg.start[j] = next;
    gg.count[j] = (int)cnt;
    gg.job[j].xcds = X;
    const int64_t end = ((int64_t)next + cnt + X - 1) / X * X;
    if (end > (int64_t)1 << 30) return hipErrorInvalidValue;
    next = (int)end;
  }
  void* args[] = {(void*)&gg};
  return launch_kernel((const void*)gemm_group_kernel, dim3(next), dim3(256), args, 0, s, ev.start,
                            ev.stop, 0);
}

hipError_t launch_gemm_bf16_splitk(const GemmArgs& g, hipStream_t s, LaunchEvents ev_gemm,
                                   LaunchEvents ev_reduce) {
  // 64 x 64 tiles, 3-stage ring: the split-K shapes are small outputs.
  if (g.splits < 2 || g.partial == nullptr || g.bias != nullptr || g.relu || !tiles_fit(g, 64))
    return hipErrorInvalidValue;
  for (int sg = 0; sg < g.nseg; ++sg)
    if (g.seg[sg].heads != 1 || g.seg[sg].width % 8 != 0) return hipErrorInvalidValue;
  hipError_t e = launch_tile<64, 64, 3>(g, s, ev_gemm);
  if (e != hipSuccess) return e;
  const int N = g.col_start[g.nseg];
  const int64_t threads = (int64_t)g.M * (N / 8);
  void* args[] = {(void*)&g};
  return launch_kernel((const void*)gemm_splitk_reduce_kernel, dim3((unsigned)((threads + 255) / 256)),
                            dim3(256), args, 0, s, ev_reduce.start, ev_reduce.stop, 0);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, LaunchEvents ev) {
  // Measured on MI355X over the block's projection shapes and the FFN's:
  // 128 x 128 tiles with 8 waves (more waves issuing the stage copies) once
  // there are enough tiles to occupy the compute units (2-stage ring, two
  // workgroups per unit, from about 1.5 tiles per unit on), otherwise 64 x 64
  // tiles with 4 waves for parallelism.  Larger tiles (256 x 128) were
  // slower on every shape measured.
  const int N = g.col_start[g.nseg];
  // 256 x 256 tiles with 16 waves (64 x 64 per wave: half the bytes brought
  // into LDS per flop of 128 x 128, and 1 KB of LDS reads per MFMA) when they fill the compute
  // units: their last round occupies at least three quarters of the 256
  // (decoder QKV projection, 8192 x 1536, K = 512: 26.3 vs 30.3 us; with
  // half the units idle, 128 tiles, they are 1.3x slower).
  if (tiles_fit(g, 256)) {
    const long t256 = (long)((N + 255) / 256) * ((g.M + 255) / 256);
    if (t256 % 256 == 0 || t256 % 256 >= 192) return launch_gemm_bf16_cfg(g, 13, s, ev);
  }
  if (!tiles_fit(g, 128)) return launch_gemm_bf16_cfg(g, 6, s, ev);
  // 256 x 128 tiles (4 x 2 waves of 64 x 64, three stages) for wide outputs
  // with at least 150 of them (measured: encoder QKV projection 3200 x 1536
  // 18.9 -> 15.0 us, cross-attention K/V 4096 x 2048 27.7 -> 26.3, FFN first
  // GEMM 3200 x 2048 17.2 -> 16.6; narrower outputs, 512 columns, were
  // 1.3-1.6x slower on them).
  if (N >= 1536 && (long)((N + 127) / 128) * ((g.M + 255) / 256) >= 150)
    return launch_gemm_bf16_cfg(g, 14, s, ev);
  const long t128 = (long)((N + 127) / 128) * ((g.M + 127) / 128);
  if (t128 >= 400) return launch_gemm_bf16_cfg(g, 9, s, ev);
  if (t128 >= 150) return launch_gemm_bf16_cfg(g, 10, s, ev);
  return launch_gemm_bf16_cfg(g, 6, s, ev);
}

}  // namespace mha
