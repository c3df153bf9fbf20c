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
// Tiling: 256 threads = 2 x 2 waves; a BM x 128 output tile, each wave a
// (BM/2) x 64 block of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16).  K
// advances 64 per step through two LDS buffers (one barrier per step); the
// global loads of step t+2 are in flight while step t is multiplied.  Both
// tiles stay in their global row-major layout in LDS: the A operand (8
// consecutive k of one row per lane) is one 16-byte read, the weight operand
// (8 consecutive k of one column) is two transposing reads
// (ds_read_b64_tr_b16).  Rows are XOR-swizzled in 16-byte chunks so that
// both read patterns are free of bank conflicts.
#include "kernels.h"

namespace mha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BK = 64;
constexpr int BN = 128;

// A tile [BM][BK]: 128-byte rows; chunk c of row m sits at chunk c ^ ((m >> 1) & 7).
__device__ __forceinline__ int a_off(int m, int chunk) {
  return m * BK + ((chunk ^ ((m >> 1) & 7)) << 3);
}
// W tile [BK][BN]: 256-byte rows; chunk c of row k sits at chunk c ^ ((k & 3) << 2).
__device__ __forceinline__ int b_off(int k, int chunk) {
  return k * BN + ((chunk ^ ((k & 3) << 2)) << 3);
}

__device__ __forceinline__ i16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

template <int BM>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const GemmArgs g) {
  constexpr int MB = BM / 64;                  // 32-row MFMA tiles per wave
  constexpr int NB = 2;                        // 32-column MFMA tiles per wave
  constexpr int ACH = BM * BK / 8 / 256;       // 16-byte A chunks per thread per step
  constexpr int BCH = BK * BN / 8 / 256;       // 16-byte W chunks per thread per step

  __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BK * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 31;
  const int grp = lane >> 5;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int N = g.col_start[g.nseg];
  const __bf16* A = (const __bf16*)g.A;

  // Per-thread source rows/columns, fixed across K steps.  Loads are
  // unconditional (straight-line code keeps two steps of loads in flight):
  // rows past M and columns past N are clamped to the last one (their
  // results are never stored); k past K is zeroed when the chunk is stored.
  const __bf16* a_src[ACH];
  int a_row[ACH], a_chunk[ACH];
#pragma unroll
  for (int r = 0; r < ACH; ++r) {
    const int c = tid + r * 256;
    a_row[r] = c >> 3;
    a_chunk[r] = c & 7;
    const int m = min(m0 + a_row[r], g.M - 1);
    a_src[r] = A + (int64_t)m * g.K + a_chunk[r] * 8;
  }
  const __bf16* b_src[BCH];
  int b_stride[BCH], b_row[BCH], b_chunk[BCH];
#pragma unroll
  for (int r = 0; r < BCH; ++r) {
    const int c = tid + r * 256;
    b_row[r] = c >> 4;      // k within the step
    b_chunk[r] = c & 15;    // 8-column chunk within the tile
    const int n = min(n0 + b_chunk[r] * 8, N - 8);
    int s = 0;
    while (s + 1 < g.nseg && n >= g.col_start[s + 1]) ++s;
    b_src[r] = (const __bf16*)g.seg[s].W + (n - g.col_start[s]);
    b_stride[r] = g.seg[s].width;
  }

  u32x4 areg[ACH], breg[BCH];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const int k = min(k0 + a_chunk[r] * 8, g.K - 8) - a_chunk[r] * 8;
      areg[r] = *(const u32x4*)(a_src[r] + k);
    }
#pragma unroll
    for (int r = 0; r < BCH; ++r) {
      const int k = min(k0 + b_row[r], g.K - 1);
      breg[r] = *(const u32x4*)(b_src[r] + (int64_t)k * b_stride[r]);
    }
  };
  auto store_step = [&](int buf, int k0) {
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const bool ok = k0 + a_chunk[r] * 8 < g.K;
      *(u32x4*)&As[buf][a_off(a_row[r], a_chunk[r])] = ok ? areg[r] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < BCH; ++r) {
      const bool ok = k0 + b_row[r] < g.K;
      *(u32x4*)&Bs[buf][b_off(b_row[r], b_chunk[r])] = ok ? breg[r] : u32x4{0, 0, 0, 0};
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  // Weight-operand source lane pattern of the transposing read: within each
  // 16-lane group, lane s addresses row (s / 4) and columns 4 (s % 4) .. +3.
  const int tr_k = (lane & 15) >> 2;
  const int tr_n = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  const int steps = (g.K + BK - 1) / BK;
  load_step(0);
  store_step(0, 0);
  load_step(BK);
  for (int t = 0; t < steps; ++t) {
    const int buf = t & 1;
    __syncthreads();
    store_step(buf ^ 1, (t + 1) * BK);
    load_step((t + 2) * BK);
    // Keep the loads here: sinking them toward their use (next step) would
    // leave no compute to hide their latency.
    __builtin_amdgcn_sched_barrier(0);
    const __bf16* as = As[buf];
    const __bf16* bs = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[MB], bfr[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *(const bf16x8*)&as[a_off(wm * (BM / 2) + 32 * i + col, 2 * ks + grp)];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int k = 16 * ks + 8 * grp + tr_k;
        const int n = wn * 64 + 32 * j + tr_n;
        const i16x4 lo = tr_read(&bs[b_off(k, n >> 3) + (n & 7)]);
        const i16x4 hi = tr_read(&bs[b_off(k + 4, n >> 3) + (n & 7)]);
        bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // acc[i][j][e] = C[m0 + wm*BM/2 + 32i + 8(e/4) + 4grp + e%4][n0 + wn*64 + 32j + col]
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = n0 + wn * 64 + 32 * j + col;
    if (n >= N) continue;
    int s = 0;
    while (s + 1 < g.nseg && n >= g.col_start[s + 1]) ++s;
    const GemmSeg& sg = g.seg[s];
    const int c = n - g.col_start[s];
    const int head = c / sg.hd;
    const int dd = c - head * sg.hd;
    __bf16* dst = (__bf16*)sg.dst + (int64_t)head * sg.rows * sg.hd + dd;
    const int64_t batch_stride = (int64_t)sg.heads * sg.rows * sg.hd;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      // Rows of this lane: mb + {0,1,2,3, 8..11, 16..19, 24..27}, mb = first row.
      const int mb = m0 + wm * (BM / 2) + 32 * i + 4 * grp;
      int bb = mb / sg.rows;
      int pos = mb - bb * sg.rows;
      int m = mb;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int next = mb + 8 * (e >> 2) + (e & 3);
        while (m < next) {  // advance (bb, pos) to row `next`
          ++m;
          if (++pos == sg.rows) { pos = 0; ++bb; }
        }
        if (m < g.M) dst[bb * batch_stride + (int64_t)pos * sg.hd] = (__bf16)acc[i][j][e];
      }
    }
  }
}

template <int BM>
hipError_t launch_tile(const GemmArgs& g, hipStream_t s, LaunchEvents ev) {
  const int N = g.col_start[g.nseg];
  dim3 grid((N + BN - 1) / BN, (g.M + BM - 1) / BM);
  void* args[] = {(void*)&g};
  return hipExtLaunchKernel((const void*)gemm_bf16_kernel<BM>, grid, dim3(256), args, 0, s,
                            ev.start, ev.stop, 0);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, LaunchEvents ev) {
  const int N = g.col_start[g.nseg];
  // 128-row tiles when they still give every compute unit two workgroups,
  // otherwise 64-row tiles for more parallelism.
  const long big = (long)((N + BN - 1) / BN) * ((g.M + 127) / 128);
  if (big >= 512) return launch_tile<128>(g, s, ev);
  return launch_tile<64>(g, s, ev);
}

}  // namespace mha
