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
// Tiling: 256 threads = 2 x 2 waves, each wave owns a (BM/2) x (BN/2) block of
// 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16).  K advances 32 at a time;
// the A tile is staged in LDS as [m][k] and the weight tile transposed to
// [n][k], so both MFMA operands are single 16-byte LDS reads (the operands
// want 8 consecutive k per lane).  The next K tile is prefetched into
// registers while the current one is multiplied.
#include "kernels.h"

namespace mha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 32;
constexpr int LDK = BK + 8;  // LDS row stride (elements) of both tiles: 80 bytes

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const GemmArgs g) {
  constexpr int MB = BM / 64;                 // 32x32 tiles per wave along m
  constexpr int NB = BN / 64;                 // ... along n
  constexpr int ACH = BM * BK / 8 / 256;      // 16-byte A chunks per thread
  constexpr int BTOT = (BK / 2) * (BN / 8);   // (2 rows x 16 bytes) W chunks per tile
  constexpr int BCH = (BTOT + 255) / 256;      // ... per thread
  static_assert(ACH >= 1 && ACH * 256 == BM * BK / 8, "A tile must split evenly over 256 threads");

  __shared__ __attribute__((aligned(16))) __bf16 As[BM * LDK];
  __shared__ __attribute__((aligned(16))) __bf16 Bt[BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int grp = lane >> 5;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int N = g.col_start[g.nseg];
  const __bf16* A = (const __bf16*)g.A;

  u32x4 areg[ACH];
  u32x4 breg[BCH][2];

  // Weight chunk (k row pair kp, column chunk nc): the segment holding
  // column n0 + 8nc.  Widths are multiples of 8, so a chunk never straddles.
  auto w_ptr = [&](int n, int k) -> const __bf16* {
    int s = 0;
    while (s + 1 < g.nseg && n >= g.col_start[s + 1]) ++s;
    const GemmSeg& sg = g.seg[s];
    return (const __bf16*)sg.W + (int64_t)k * sg.width + (n - g.col_start[s]);
  };

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const int c = tid + r * 256;
      const int row = m0 + c / (BK / 8);
      const int k = k0 + (c % (BK / 8)) * 8;
      areg[r] = (row < g.M && k < g.K) ? *(const u32x4*)(A + (int64_t)row * g.K + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < BCH; ++r) {
      const int p = tid + r * 256;
      const int kp = p % (BK / 2);
      const int nc = p / (BK / 2);
      const int n = n0 + nc * 8;
      const int k = k0 + 2 * kp;
      if (p < BTOT && n < N) {
        breg[r][0] = k < g.K ? *(const u32x4*)w_ptr(n, k) : u32x4{0, 0, 0, 0};
        breg[r][1] = k + 1 < g.K ? *(const u32x4*)w_ptr(n, k + 1) : u32x4{0, 0, 0, 0};
      } else {
        breg[r][0] = u32x4{0, 0, 0, 0};
        breg[r][1] = u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const int c = tid + r * 256;
      *(u32x4*)&As[(c / (BK / 8)) * LDK + (c % (BK / 8)) * 8] = areg[r];
    }
#pragma unroll
    for (int r = 0; r < BCH; ++r) {
      const int p = tid + r * 256;
      const int kp = p % (BK / 2);
      const int nc = p / (BK / 2);
      if (p >= BTOT) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned x0 = breg[r][0][j];  // W[k][n+2j], W[k][n+2j+1]
        const unsigned x1 = breg[r][1][j];  // W[k+1][...]
        *(unsigned*)&Bt[(8 * nc + 2 * j) * LDK + 2 * kp] = (x0 & 0xffffu) | (x1 << 16);
        *(unsigned*)&Bt[(8 * nc + 2 * j + 1) * LDK + 2 * kp] = (x0 >> 16) | (x1 & 0xffff0000u);
      }
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  const int ktiles = (g.K + BK - 1) / BK;
  load_tile(0);
  for (int t = 0; t < ktiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ktiles) load_tile((t + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[MB], bfr[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *(const bf16x8*)&As[(wm * (BM / 2) + 32 * i + col) * LDK + 16 * ks + 8 * grp];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bfr[j] = *(const bf16x8*)&Bt[(wn * (BN / 2) + 32 * j + col) * LDK + 16 * ks + 8 * grp];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // acc[i][j][e] = C[m0 + wm*BM/2 + 32i + 8(e/4) + 4grp + e%4][n0 + wn*BN/2 + 32j + col]
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = n0 + wn * (BN / 2) + 32 * j + col;
    if (n >= N) continue;
    int s = 0;
    while (s + 1 < g.nseg && n >= g.col_start[s + 1]) ++s;
    const GemmSeg& sg = g.seg[s];
    const int c = n - g.col_start[s];
    const int head = c / sg.hd;
    const int dd = c - head * sg.hd;
    __bf16* dst = (__bf16*)sg.dst;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * (BM / 2) + 32 * i + 8 * (e >> 2) + 4 * grp + (e & 3);
        if (m >= g.M) continue;
        const int bb = m / sg.rows;
        const int pos = m - bb * sg.rows;
        const int64_t off = ((int64_t)(bb * sg.heads + head) * sg.rows + pos) * sg.hd + dd;
        dst[off] = (__bf16)acc[i][j][e];
      }
    }
  }
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs& g, hipStream_t s) {
  const int N = g.col_start[g.nseg];
  dim3 grid((N + BN - 1) / BN, (g.M + BM - 1) / BM);
  void* args[] = {(void*)&g};
  return hipLaunchKernel((const void*)gemm_bf16_kernel<BM, BN>, grid, dim3(256), args, 0, s);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  const int N = g.col_start[g.nseg];
  // Prefer big tiles; fall back to 64x64 when big tiles would leave most of
  // the 256 compute units idle.
  const long big = (long)((N + 127) / 128) * ((g.M + 127) / 128);
  if (big >= 256) return launch_tile<128, 128>(g, s);
  return launch_tile<64, 64>(g, s);
}

}  // namespace mha
