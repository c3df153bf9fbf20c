// Internal interface between the C-ABI layer (mha_api.hip) and the kernels.
// Not installed; the public interface is include/mha.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mha.h"

namespace mha {

// Per-batch key lengths travel inside the kernel arguments, which hold at
// most this many; the C-ABI layer splits a padded call over more batches
// into launches of at most kLaunchBatch batches each.
constexpr int kLaunchBatch = 256;

// Strides are in elements; the innermost (feature) dimension is contiguous.
struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int64_t q_sb, q_sh, q_sr;   // batch, head, row strides of Q
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t o_sb, o_sh, o_sr;
  int B, h, n_q, n_k;
  float scale;        // multiplies q.k
  int causal;         // key j hidden from query i when j > i
  int padded;         // key j hidden in batch b when j >= key_len[b]
  // Optional (bf16 kernels): row log-sum-exp, lse[(b*h + head)*n_q + i] =
  // ln(sum over visible keys j of exp(scale * q_i . k_j)); null: not written.
  float* lse;
  // Few-query kernel only: the key tiles of each (batch, head) are dealt to
  // `splits` workgroups, each writing its partial softmax state to `part`
  // (splits > 1; a second launch merges them).
  int splits;
  float* part;
  int32_t key_len[kLaunchBatch];
  // Batches by decreasing key length (padded only; the few-query kernel
  // takes the longest sequences first, so the last workgroups to start are
  // short ones).
  uint8_t order[kLaunchBatch];
};

// Attention backward: dQ, dK, dV of O = softmax(Q K^T * scale + M) V from
// the upstream gradient dO and the forward's row log-sum-exp.  Every tensor
// is head-major [B][h][n][64] bf16; Dw and Lw are fp32 workspace [B][h][n_q]
// that receive -rowsum(dO * O) and -lse / scale.
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;
  void* dQ;
  void* dK;
  void* dV;
  float* Dw;
  float* Lw;
  // batch, head, row strides (elements) of O, dQ, dK, dV; Q, K, V, dO are
  // head-major and dense
  int64_t o_sb, o_sh, o_sr;
  int64_t dq_sb, dq_sh, dq_sr;
  int64_t dk_sb, dk_sh, dk_sr;
  int64_t dv_sb, dv_sh, dv_sr;
  int B, h, n_q, n_k;
  float scale;
  int causal;
  int padded;
  int32_t key_len[kLaunchBatch];
};

// One column segment of a projection GEMM: columns [0, width) of weight W
// (row stride ldw, or width) and the per-head scatter of the result:
//   out element (row m, column c) -> dst[((b*heads + c/hd)*rows + pos)*hd + c%hd]
// with b = m / rows, pos = m % rows, hd = head width.  A plain row-major
// [M][width] output is heads = 1, hd = width, rows = M.
struct GemmSeg {
  const void* W;
  void* dst;
  int width;
  int hd;
  int heads;
  int rows;
  int ldw;   // row stride of W in elements (0: width); a multiple of 8
};

struct GemmArgs {
  const void* A;      // [M][K] row-major
  int M, K;
  int nseg;
  GemmSeg seg[3];
  int col_start[4];   // prefix sums of segment widths; col_start[nseg] = N
  // Epilogue (single-segment GEMMs only): bias[N] (bf16, may be null) is
  // added to every row before rounding, then max(0, .) when relu != 0.
  const void* bias;
  int relu;
  // Split-K (launch_gemm_bf16_splitk only): the k stages are shared out over
  // `splits` workgroups per tile, each writing fp32 partial sums
  // partial[z][M][N]; a second kernel adds them and rounds once.
  int splits;
  float* partial;
  // XCDs of the device (set by the launchers): the tile order gives each
  // XCD's workgroups a contiguous band of tile rows.
  int xcds;
};

// Residual + LayerNorm over rows of d features (bf16):
//   Y[m] = gamma * norm(X[m] + F[m]) + beta,  norm(u) = (u - mean) / sqrt(var + eps)
constexpr int kLnMaxWidth = 4096;
struct LnArgs {
  const void* X;      // [M][d]
  const void* F;      // [M][d]
  const void* gamma;  // [d]
  const void* beta;   // [d]
  void* Y;            // [M][d]; may be X or F
  int M, d;
  float eps;
};

// Scaled token embedding plus sinusoidal positional encoding:
//   out[b][p] = E[tokens[b][p]] * sqrt(d) + PE(pos0 + p)
struct EmbedArgs {
  const int32_t* tokens;  // [B][n] (device)
  const void* E;          // [vocab][d]
  void* out;              // [B][n][d]
  int B, n, vocab, d, pos0;
};

// Fused input projections + attention for short sequences (n_q, n_k <= 128,
// d_model a multiple of 64, head size 64): one workgroup per (batch, head)
// computes that head's Q, K, V tiles and its attention output.
struct ProjAttnArgs {
  const void* Xq;     // [B][n_q][d_model]
  const void* Xkv;    // [B][n_k][d_model] (may equal Xq)
  const void* Wq;     // [d_model][h*64]
  const void* Wk;
  const void* Wv;
  void* O;            // concatenated heads [B][n_q][h*64]
  int B, h, n_q, n_k, d_model;
  float scale;
  int causal;
  int padded;
  int xcds;           // XCDs of the device (set by the launcher)
  int32_t key_len[kLaunchBatch];
};

// Launch-time events: when `start`/`stop` are non-null they are recorded at
// the start and at the end of this kernel's execution (hipExtLaunchKernel).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

#ifdef MHA_FAULT_INJECTION
// Test builds only (fault_injection.hip): true while armed launches remain.
bool fault_injection_fires();
#endif

// Every kernel launch of the library goes through here (same arguments as
// hipExtLaunchKernel).  A build with MHA_FAULT_INJECTION defined can make
// launches fail here, without reaching the runtime, to test how a launch
// error travels back to the caller; the normal build has no such path.
inline hipError_t launch_kernel(const void* f, dim3 grid, dim3 block, void** args, size_t shared,
                                hipStream_t stream, hipEvent_t start, hipEvent_t stop, int flags) {
#ifdef MHA_FAULT_INJECTION
  if (fault_injection_fires()) return hipErrorLaunchFailure;
#endif
  return hipExtLaunchKernel(f, grid, block, args, shared, stream, start, stop, flags);
}

// Few queries (n_q <= 32, no causal mask) over more than 128 keys: the keys
// of each (batch, head) are split over the workgroup's waves.
bool attn_decode_applies(const AttnArgs& a);
hipError_t launch_attn_decode_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev);
// Split form (a.splits > 1, a.part holding decode_part_floats(a) floats):
// the partial launch, then the merge launch.
constexpr int kDecodeStateFloats = 34 * 64;  // one workgroup's state: m, l, 32 accumulators per lane
inline int64_t decode_part_floats(const AttnArgs& a) {
  return (int64_t)a.B * a.h * a.splits * kDecodeStateFloats;
}
hipError_t launch_attn_decode_split_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev_part,
                                             LaunchEvents ev_merge);
// Compute units and XCDs of the current device (read once per device).
int device_compute_units();
int device_xcds();
hipError_t launch_attn_bf16_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev = {});
// One fixed attention configuration (index into the instantiated set); for sweeps.
hipError_t launch_attn_bf16_d64_cfg(const AttnArgs& a, int cfg, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_attn_f32_d64(const AttnArgs& a, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_gemm_bf16_splitk(const GemmArgs& g, hipStream_t s, LaunchEvents ev_gemm = {},
                                   LaunchEvents ev_reduce = {});
// Up to three independent jobs in one launch, each a GEMM in 64 x 64 tiles
// (plain, or split-K writing its fp32 partials) or, reduce[j] != 0, the
// reduction of a split-K GEMM that an earlier launch finished.  The jobs
// must not depend on each other (they run concurrently).  start and count
// are filled in by the launcher.
constexpr int kMaxGroupJobs = 3;
struct GemmGroup {
  GemmArgs job[kMaxGroupJobs];
  int reduce[kMaxGroupJobs];
  int start[kMaxGroupJobs];
  int count[kMaxGroupJobs];
  int n;
};
hipError_t launch_gemm_bf16_group(GemmGroup gg, hipStream_t s, LaunchEvents ev = {});
// Backward: the dQ kernel (also writes Dw), then the dK/dV kernel (reads Dw).
hipError_t launch_attn_bwd_dq(const BwdArgs& a, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_attn_bwd_dkdv(const BwdArgs& a, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_add_layernorm_bf16(const LnArgs& a, hipStream_t s, LaunchEvents ev = {});
// dst_i[c][r] = src_i[r][c] for up to eight dense bf16 [R_i][C_i] matrices
// in one launch (R_i, C_i multiples of 8).
constexpr int kMaxTransposeBatch = 8;
struct TransposeBatch {
  const void* src[kMaxTransposeBatch];
  void* dst[kMaxTransposeBatch];
  int R[kMaxTransposeBatch];
  int C[kMaxTransposeBatch];
  int n;
};
hipError_t launch_transpose_bf16(const TransposeBatch& tb, hipStream_t s, LaunchEvents ev = {});
// f32 != 0: E and out are fp32, else bf16.
hipError_t launch_embed_positional(const EmbedArgs& a, int f32, hipStream_t s, LaunchEvents ev = {});
bool proj_attn_supported(int n_q, int n_k, int d_model);
hipError_t launch_proj_attn_bf16(const ProjAttnArgs& a, hipStream_t s, LaunchEvents ev = {});
// The argument checks of sdpa_backward (everything but the workspace), host only.
int check_backward_args(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* lse, const void* dQ, const void* dK, const void* dV, int B,
                        int h, int n_q, int n_k, int d_k, int d_v, float scale, int mask_kind,
                        const int32_t* key_lengths, int dtype);
// One fixed tile configuration (index into the instantiated set); for sweeps.
hipError_t launch_gemm_bf16_cfg(const GemmArgs& g, int cfg, hipStream_t s, LaunchEvents ev = {});

}  // namespace mha
