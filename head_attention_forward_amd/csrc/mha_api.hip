// C-ABI entry points of libmha (declared in include/mha.h).
//
// Every argument check happens here, on the host, before any HIP call; the
// kernels assume the shapes these checks admit.  The entry points only fill
// argument structs and enqueue launches on the caller's stream.
#include <math.h>
#include <string.h>

#include "kernels.h"

namespace mha {
namespace {

constexpr int64_t kIndexLimit = (int64_t)1 << 31;  // row/column counts stay int32
// GEMM operand widths (d_model, h*d_k, h*d_v, d_ff): a stage's per-lane byte
// offsets (up to 128 rows of a row-major operand) stay within 32 bits.
constexpr int64_t kMaxWidth = (int64_t)1 << 20;
constexpr size_t kAlign = 256;

size_t elt_size(int dtype) { return dtype == MHA_DTYPE_F32 ? 4 : 2; }

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_mask(int mask_kind, int B, int n_q, int n_k, const int32_t* key_lengths) {
  if (mask_kind < 0 || mask_kind > MHA_MASK_CAUSAL_KEY_PADDING) return MHA_ERR_MASK;
  if ((mask_kind & MHA_MASK_CAUSAL) && n_q != n_k) return MHA_ERR_MASK;
  if (mask_kind & MHA_MASK_KEY_PADDING) {
    if (key_lengths == nullptr) return MHA_ERR_KEYLEN;
    if (B > MHA_MAX_PADDED_BATCH) return MHA_ERR_UNSUPPORTED;
    for (int b = 0; b < B; ++b)
      if (key_lengths[b] < 1 || key_lengths[b] > n_k) return MHA_ERR_KEYLEN;
  }
  return MHA_OK;
}

int check_attn_dims(int B, int h, int n_q, int n_k, int d_k, int d_v) {
  if (B <= 0 || h <= 0 || n_q <= 0 || n_k <= 0 || d_k <= 0 || d_v <= 0) return MHA_ERR_DIM;
  if ((int64_t)B * h >= kIndexLimit) return MHA_ERR_DIM;
  if ((int64_t)B * n_q >= kIndexLimit || (int64_t)B * n_k >= kIndexLimit) return MHA_ERR_DIM;
  if ((int64_t)h * d_k >= kIndexLimit || (int64_t)h * d_v >= kIndexLimit) return MHA_ERR_DIM;
  if (n_q > 65535 * 128) return MHA_ERR_DIM;  // query tiles index grid.y
  if (d_k != 64 || d_v != 64) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

void fill_mask(AttnArgs& a, int mask_kind) {
  a.causal = (mask_kind & MHA_MASK_CAUSAL) ? 1 : 0;
  a.padded = (mask_kind & MHA_MASK_KEY_PADDING) ? 1 : 0;
}


struct Workspace {
  void* Q;
  void* K;
  void* V;
  void* O;
  size_t bytes;
};

Workspace carve(void* base, int B, int n_q, int n_k, int h, int d_k, int d_v, int dtype) {
  const size_t e = elt_size(dtype);
  const size_t q = round_up(e * B * (size_t)h * n_q * d_k);
  const size_t k = round_up(e * B * (size_t)h * n_k * d_k);
  const size_t v = round_up(e * B * (size_t)h * n_k * d_v);
  const size_t o = round_up(e * B * (size_t)n_q * h * d_v);
  char* p = (char*)base;
  return Workspace{p, p + q, p + q + k, p + q + k + v, q + k + v + o};
}

// Sizes, dtype and workspace of the block (shared by mha_forward and the stages).
int check_block(const void* ws, size_t ws_bytes, int B, int n_q, int n_k, int h, int d_k,
                int d_v, int dtype) {
  int st = check_attn_dims(B, h, n_q, n_k, d_k, d_v);
  if (st != MHA_OK) return st;
  if (dtype != MHA_DTYPE_BF16) return MHA_ERR_UNSUPPORTED;
  if (ws == nullptr) return MHA_ERR_WORKSPACE;
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return MHA_ERR_WORKSPACE;
  if (ws_bytes < carve(nullptr, B, n_q, n_k, h, d_k, d_v, dtype).bytes) return MHA_ERR_WORKSPACE;
  return MHA_OK;
}

// The projections additionally need d_model rows in whole 16-byte chunks.
int check_mha(const void* ws, size_t ws_bytes, int B, int n_q, int n_k, int d_model, int h,
              int d_k, int d_v, int dtype) {
  if (d_model <= 0 || d_model > kMaxWidth) return MHA_ERR_DIM;
  int st = check_block(ws, ws_bytes, B, n_q, n_k, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  if ((int64_t)h * d_k > kMaxWidth || (int64_t)h * d_v > kMaxWidth) return MHA_ERR_DIM;
  if (d_model % 8 != 0) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MHA_OK : MHA_ERR_HIP; }

// Hands out (start, stop) event pairs to successive launches of a timed call;
// a null timer hands out none.
struct Timer {
  hipEvent_t* ev = nullptr;
  int cap = 0;
  int used = 0;  // launches so far
  LaunchEvents next() {
    LaunchEvents le;
    if (ev != nullptr && 2 * used + 1 < cap) {
      le.start = ev[2 * used];
      le.stop = ev[2 * used + 1];
    }
    ++used;
    return le;
  }
};

LaunchEvents next_events(Timer* t) { return t ? t->next() : LaunchEvents{}; }

// The key lengths of batches [b0, b0 + a.B) into a launch's arguments
// (a.B <= kLaunchBatch), with the batches ordered by decreasing length.
void fill_lengths(AttnArgs& a, const int32_t* key_lengths, int b0) {
  const int32_t* kl = key_lengths + b0;
  for (int b = 0; b < a.B; ++b) {
    a.key_len[b] = kl[b];
    a.order[b] = (uint8_t)b;
  }
  // stable insertion sort by decreasing length
  for (int i = 1; i < a.B; ++i) {
    const uint8_t v = a.order[i];
    int j = i;
    while (j > 0 && kl[a.order[j - 1]] < kl[v]) {
      a.order[j] = a.order[j - 1];
      --j;
    }
    a.order[j] = v;
  }
}

template <typename T>
T* advance(T* p, int64_t elems, size_t elt) {
  return p == nullptr ? p : (T*)((char*)p + elems * (int64_t)elt);
}

// Batches per launch: all of them, unless the key lengths ride along.
int launch_batch(int B, int padded) { return padded ? kLaunchBatch : B; }

// One attention launch per chunk of at most kLaunchBatch batches when the
// key lengths ride along (a padded call), else one launch.  `a` describes
// the whole call; each chunk gets its own base pointers and lengths.
hipError_t launch_attention(const AttnArgs& a, const int32_t* key_lengths, int f32, hipStream_t s,
                            Timer* tm) {
  const size_t e = f32 ? 4 : 2;
  const int step = launch_batch(a.B, a.padded);
  for (int b0 = 0; b0 < a.B; b0 += step) {
    AttnArgs c = a;
    c.B = a.B - b0 < step ? a.B - b0 : step;
    c.Q = advance(a.Q, b0 * a.q_sb, e);
    c.K = advance(a.K, b0 * a.k_sb, e);
    c.V = advance(a.V, b0 * a.v_sb, e);
    c.O = advance(a.O, b0 * a.o_sb, e);
    c.lse = advance(a.lse, (int64_t)b0 * a.h * a.n_q, sizeof(float));
    if (c.padded) fill_lengths(c, key_lengths, b0);
    const LaunchEvents le = next_events(tm);
    const hipError_t err = f32 ? launch_attn_f32_d64(c, s, le) : launch_attn_bf16_d64(c, s, le);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// The backward's two launches per chunk (the dQ kernel writes the chunk's
// row terms, the dK/dV kernel of the same chunk reads them).
hipError_t launch_backward(const BwdArgs& a, const int32_t* key_lengths, hipStream_t s, Timer* tm) {
  const int step = launch_batch(a.B, a.padded);
  for (int b0 = 0; b0 < a.B; b0 += step) {
    BwdArgs c = a;
    c.B = a.B - b0 < step ? a.B - b0 : step;
    const int64_t q_rows = (int64_t)b0 * a.h * a.n_q, k_rows = (int64_t)b0 * a.h * a.n_k;
    c.Q = advance(a.Q, q_rows * 64, 2);   // dense head-major, head size 64
    c.dO = advance(a.dO, q_rows * 64, 2);
    c.K = advance(a.K, k_rows * 64, 2);
    c.V = advance(a.V, k_rows * 64, 2);
    c.O = advance(a.O, b0 * a.o_sb, 2);
    c.dQ = advance(a.dQ, b0 * a.dq_sb, 2);
    c.dK = advance(a.dK, b0 * a.dk_sb, 2);
    c.dV = advance(a.dV, b0 * a.dv_sb, 2);
    c.lse = advance(a.lse, q_rows, sizeof(float));
    c.Dw = advance(a.Dw, q_rows, sizeof(float));
    c.Lw = advance(a.Lw, q_rows, sizeof(float));
    if (c.padded)
      for (int b = 0; b < c.B; ++b) c.key_len[b] = key_lengths[b0 + b];
    hipError_t err = launch_attn_bwd_dq(c, s, next_events(tm));
    if (err != hipSuccess) return err;
    err = launch_attn_bwd_dkdv(c, s, next_events(tm));
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Few-query attention: workgroups per (batch, head) so that B * h of them
// fill the compute units (key tiles dealt out by eights per workgroup; at
// most kMaxDecodeSplits).  1 when the plain few-query launch already fills
// the chip, when the split does not apply, or for padded calls of more than
// one launch's batches.
constexpr int kMaxDecodeSplits = 8;
int decode_splits(int B, int h, int n_q, int n_k, int mask_kind) {
  if (n_q > 32 || (mask_kind & MHA_MASK_CAUSAL) || n_k <= 128 || B > kLaunchBatch) return 1;
  const int64_t bh = (int64_t)B * h;
  const int cus = device_compute_units();
  if (bh >= cus) return 1;
  int s = (int)((cus + bh - 1) / bh);
  const int tiles = (n_k + 63) / 64;
  const int by_tiles = (tiles + 7) / 8;  // each workgroup's eight waves want at least a tile each
  if (s > by_tiles) s = by_tiles;
  if (s > kMaxDecodeSplits) s = kMaxDecodeSplits;
  return s < 1 ? 1 : s;
}

// The fused projection + attention kernel, one launch per chunk likewise.
hipError_t launch_fused(const ProjAttnArgs& a, const int32_t* key_lengths, hipStream_t s, Timer* tm) {
  const int step = launch_batch(a.B, a.padded);
  for (int b0 = 0; b0 < a.B; b0 += step) {
    ProjAttnArgs c = a;
    c.B = a.B - b0 < step ? a.B - b0 : step;
    c.Xq = advance(a.Xq, (int64_t)b0 * a.n_q * a.d_model, 2);
    c.Xkv = advance(a.Xkv, (int64_t)b0 * a.n_k * a.d_model, 2);
    c.O = advance(a.O, (int64_t)b0 * a.n_q * a.h * 64, 2);
    if (c.padded)
      for (int b = 0; b < c.B; ++b) c.key_len[b] = key_lengths[b0 + b];
    const hipError_t err = launch_proj_attn_bf16(c, s, next_events(tm));
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Short sequences (both <= 128 rows) with d_model a multiple of 64 take the
// fused projection + attention kernel, then the output projection.
bool use_fused(int n_q, int n_k, int d_model) { return proj_attn_supported(n_q, n_k, d_model); }

// Launches an mha_forward call makes: fused path 2; otherwise one stacked
// projection for self-attention (two for cross-attention), then attention
// and the output projection.
int mha_launch_count(const void* X_q, const void* X_kv, int n_q, int n_k, int d_model) {
  if (use_fused(n_q, n_k, d_model)) return 2;
  return (X_q == X_kv && n_q == n_k) ? 3 : 4;
}

// Head-major layout [B][h][n][d] of the workspace Q, K, V.
void set_head_major(int64_t& sb, int64_t& sh, int64_t& sr, int h, int n, int d) {
  sr = d;
  sh = (int64_t)n * d;
  sb = (int64_t)h * n * d;
}

int do_project_in(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                  const void* Wv, int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                  const Workspace& w, hipStream_t stream, Timer* tm) {
  const GemmSeg sq{Wq, w.Q, h * d_k, d_k, h, n_q};
  const GemmSeg sk{Wk, w.K, h * d_k, d_k, h, n_k};
  const GemmSeg sv{Wv, w.V, h * d_v, d_v, h, n_k};
  if (X_q == X_kv && n_q == n_k) {
    // Self-attention: one launch over the stacked [W^Q | W^K | W^V].
    GemmArgs g{};
    g.A = X_q;
    g.M = B * n_q;
    g.K = d_model;
    g.nseg = 3;
    g.seg[0] = sq;
    g.seg[1] = sk;
    g.seg[2] = sv;
    g.col_start[0] = 0;
    g.col_start[1] = h * d_k;
    g.col_start[2] = 2 * h * d_k;
    g.col_start[3] = 2 * h * d_k + h * d_v;
    return launch_status(launch_gemm_bf16(g, stream, next_events(tm)));
  }
  GemmArgs gq{};
  gq.A = X_q;
  gq.M = B * n_q;
  gq.K = d_model;
  gq.nseg = 1;
  gq.seg[0] = sq;
  gq.col_start[0] = 0;
  gq.col_start[1] = h * d_k;
  int st = launch_status(launch_gemm_bf16(gq, stream, next_events(tm)));
  if (st != MHA_OK) return st;
  GemmArgs gkv{};
  gkv.A = X_kv;
  gkv.M = B * n_k;
  gkv.K = d_model;
  gkv.nseg = 2;
  gkv.seg[0] = sk;
  gkv.seg[1] = sv;
  gkv.col_start[0] = 0;
  gkv.col_start[1] = h * d_k;
  gkv.col_start[2] = h * d_k + h * d_v;
  return launch_status(launch_gemm_bf16(gkv, stream, next_events(tm)));
}

int do_attend(int B, int n_q, int n_k, int h, int d_k, int d_v, int mask_kind,
              const int32_t* key_lengths, const Workspace& w, hipStream_t stream, Timer* tm,
              float* lse = nullptr) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.Q = w.Q;
  a.K = w.K;
  a.V = w.V;
  a.O = w.O;
  set_head_major(a.q_sb, a.q_sh, a.q_sr, h, n_q, d_k);
  set_head_major(a.k_sb, a.k_sh, a.k_sr, h, n_k, d_k);
  set_head_major(a.v_sb, a.v_sh, a.v_sr, h, n_k, d_v);
  // Concatenated heads: [B][n_q][h*d_v], head i at columns [i*d_v, (i+1)*d_v).
  a.o_sr = (int64_t)h * d_v;
  a.o_sh = d_v;
  a.o_sb = (int64_t)n_q * h * d_v;
  a.B = B;
  a.h = h;
  a.n_q = n_q;
  a.n_k = n_k;
  a.scale = 1.0f / sqrtf((float)d_k);
  a.lse = lse;
  fill_mask(a, mask_kind);
  return launch_status(launch_attention(a, key_lengths, 0, stream, tm));
}

int do_project_out(const void* Wo, void* Y, int B, int n_q, int d_model, int h, int d_v,
                   const Workspace& w, hipStream_t stream, Timer* tm) {
  GemmArgs g{};
  g.A = w.O;
  g.M = B * n_q;
  g.K = h * d_v;
  g.nseg = 1;
  g.seg[0] = GemmSeg{Wo, Y, d_model, d_model, 1, B * n_q};
  g.col_start[0] = 0;
  g.col_start[1] = d_model;
  return launch_status(launch_gemm_bf16(g, stream, next_events(tm)));
}

// Plain row-major GEMM Y[M][N] = A[M][K] . W[K][N] (+ bias, ReLU).
int do_linear(const void* A, const void* W, const void* bias, int relu, void* Y, int M, int K,
              int N, hipStream_t stream, Timer* tm) {
  GemmArgs g{};
  g.A = A;
  g.M = M;
  g.K = K;
  g.nseg = 1;
  g.seg[0] = GemmSeg{W, Y, N, N, 1, M};
  g.col_start[0] = 0;
  g.col_start[1] = N;
  g.bias = bias;
  g.relu = relu;
  return launch_status(launch_gemm_bf16(g, stream, next_events(tm)));
}

int do_add_layernorm(const void* X, const void* F, const void* gamma, const void* beta, void* Y,
                     int M, int d, float eps, hipStream_t stream, Timer* tm) {
  LnArgs a{X, F, gamma, beta, Y, M, d, eps};
  return launch_status(launch_add_layernorm_bf16(a, stream, next_events(tm)));
}

int check_ln(int M, int d, float eps, int dtype) {
  if (M <= 0 || d <= 0 || (int64_t)M * d >= ((int64_t)1 << 40)) return MHA_ERR_DIM;
  if (!(isfinite(eps) && eps >= 0.f)) return MHA_ERR_SCALE;
  if (dtype != MHA_DTYPE_BF16) return MHA_ERR_UNSUPPORTED;
  if (d % 8 != 0 || d > kLnMaxWidth) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

// Rows and widths of the feed-forward GEMMs: whole 16-byte chunks.
int check_ffn(int M, int d_model, int d_ff, int dtype) {
  if (M <= 0 || d_model <= 0 || d_ff <= 0) return MHA_ERR_DIM;
  if (M >= kIndexLimit || d_model > kMaxWidth || d_ff > kMaxWidth) return MHA_ERR_DIM;
  if (dtype != MHA_DTYPE_BF16) return MHA_ERR_UNSUPPORTED;
  if (d_model % 8 != 0 || d_ff % 8 != 0) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

size_t ffn_ws(int M, int d_ff) { return round_up((size_t)2 * M * d_ff); }

int do_ffn(const void* X, const void* W1, const void* b1, const void* W2, const void* b2, void* Y,
           int M, int d_model, int d_ff, void* H, hipStream_t stream, Timer* tm) {
  int st = do_linear(X, W1, b1, 1, H, M, d_model, d_ff, stream, tm);
  if (st != MHA_OK) return st;
  return do_linear(H, W2, b2, 0, Y, M, d_ff, d_model, stream, tm);
}

// Encoder-layer workspace: the block's workspace, then the sublayer output
// S [M][d_model] (attention output, later the FFN output), x1 [M][d_model]
// and the FFN hidden layer H [M][d_ff].
struct LayerWorkspace {
  Workspace blk;
  void* S;
  void* x1;
  void* H;
  size_t bytes;
};

LayerWorkspace carve_layer(void* base, int B, int n, int d_model, int h, int d_k, int d_v,
                           int d_ff) {
  LayerWorkspace w;
  w.blk = carve(base, B, n, n, h, d_k, d_v, MHA_DTYPE_BF16);
  const size_t M = (size_t)B * n;
  const size_t act = round_up(2 * M * d_model);
  char* p = (char*)base + w.blk.bytes;
  w.S = p;
  w.x1 = p + act;
  w.H = p + 2 * act;
  w.bytes = w.blk.bytes + 2 * act + ffn_ws((int)M, d_ff);
  return w;
}

int layer_launch_count(int n, int d_model) {
  return (use_fused(n, n, d_model) ? 2 : 3) + 4;
}

// ---- training: the block's forward with its saved state, and its backward

// Forward state kept for the backward: the block workspace (Q, K, V
// head-major, O concatenated) and the row log-sum-exp [B][h][n_q].
struct TrainWs {
  Workspace blk;
  float* lse;
  size_t bytes;
};

TrainWs carve_train(void* base, int B, int n_q, int n_k, int h, int d_k, int d_v) {
  TrainWs t;
  t.blk = carve(base, B, n_q, n_k, h, d_k, d_v, MHA_DTYPE_BF16);
  t.lse = (float*)((char*)base + t.blk.bytes);
  t.bytes = t.blk.bytes + round_up((size_t)4 * B * h * n_q);
  return t;
}

// Backward scratch.  Self-attention (shared input): dQ | dK | dV side by side
// in one [M][3hd] buffer and [W^Q | W^K | W^V]^T stacked as one [3hd][d_model]
// matrix, so dX is one GEMM; cross-attention: dQ [M_q][hd] and dK | dV
// [M_k][2hd], with their transposed weights.
struct BwdWs {
  void* WoT;    // [h d_v][d_model]
  void* dO;     // [B][h][n_q][d_v]
  void* OcT;    // [h d_v][M_q]
  void* dQKV;   // self: [M][3hd]; cross: dQ [M_q][hd]
  void* dKV;    // cross: [M_k][2hd]
  float* rows;  // sdpa_backward row terms (two arrays)
  void* WT;     // self: [3hd][d_model]; cross: W^Q^T [hd][d_model]
  void* WkvT;   // cross: [2hd][d_model]
  void* XqT;    // [d_model][M_q]
  void* XkvT;   // cross: [d_model][M_k]
  float* partial;   // split-K partial sums of dW^O
  float* partial1;  // ... of dW^Q (with dW^K, dW^V for self-attention)
  float* partial2;  // cross-attention: ... of dW^K | dW^V
  size_t rows_each;
  size_t bytes;
};

// Split-K factor of a weight-gradient GEMM (small output, depth K = rows):
// one k range per XCD (the GEMM deals the splits to the 8 XCDs, so each L2
// holds one slice of both operands).
int wgrad_splits(int, int, int) { return 8; }

BwdWs carve_bwd(void* base, bool self_attn, int B, int n_q, int n_k, int d_model, int h, int d) {
  BwdWs w{};
  const size_t hd = (size_t)h * d, Mq = (size_t)B * n_q, Mk = (size_t)B * n_k, dm = d_model;
  char* p = (char*)base;
  auto take = [&](size_t bytes) {
    char* r = p;
    p += round_up(bytes);
    return (void*)r;
  };
  w.WoT = take(2 * hd * dm);
  w.dO = take(2 * Mq * hd);
  w.OcT = take(2 * hd * Mq);
  w.rows_each = round_up((size_t)4 * B * h * n_q);
  // Partial sums of the weight-gradient GEMMs, one region each: a reduction
  // runs in the same launch as a later split-K GEMM.
  w.partial = (float*)take(4 * (size_t)wgrad_splits((int)hd, d_model, (int)Mq) * hd * dm);
  if (self_attn) {
    w.partial1 = (float*)take(4 * (size_t)wgrad_splits(d_model, 3 * (int)hd, (int)Mq) * dm * 3 * hd);
  } else {
    w.partial1 = (float*)take(4 * (size_t)wgrad_splits(d_model, (int)hd, (int)Mq) * dm * hd);
    w.partial2 = (float*)take(4 * (size_t)wgrad_splits(d_model, 2 * (int)hd, (int)Mk) * dm * 2 * hd);
  }
  if (self_attn) {
    w.dQKV = take(2 * Mq * 3 * hd);
    w.rows = (float*)take(2 * w.rows_each);
    w.WT = take(2 * 3 * hd * dm);
    w.XqT = take(2 * dm * Mq);
  } else {
    w.dQKV = take(2 * Mq * hd);
    w.dKV = take(2 * Mk * 2 * hd);
    w.rows = (float*)take(2 * w.rows_each);
    w.WT = take(2 * hd * dm);
    w.WkvT = take(2 * 2 * hd * dm);
    w.XqT = take(2 * dm * Mq);
    w.XkvT = take(2 * dm * Mk);
  }
  w.bytes = (size_t)(p - (char*)base);
  return w;
}

// C = A . [segments], A [M][K] row-major; each segment a row-major weight
// (row stride ldw) written as a plain row-major [M][width] matrix.
// partial != null: split-K (a weight gradient: small output, K = rows).
GemmArgs rm_args(const void* A, int M, int K, int nseg, const void* const* W, void* const* dst,
                 const int* width, int ldw, float* partial = nullptr) {
  GemmArgs g{};
  g.A = A;
  g.M = M;
  g.K = K;
  g.nseg = nseg;
  int c = 0;
  for (int s = 0; s < nseg; ++s) {
    g.seg[s] = GemmSeg{W[s], dst[s], width[s], width[s], 1, M, ldw};
    g.col_start[s] = c;
    c += width[s];
  }
  g.col_start[nseg] = c;
  if (partial != nullptr) {
    g.splits = wgrad_splits(M, c, K);
    g.partial = partial;
  }
  return g;
}

int do_gemm_rm(const void* A, int M, int K, int nseg, const void* const* W, void* const* dst,
               const int* width, int ldw, hipStream_t stream, Timer* tm, float* partial = nullptr) {
  const GemmArgs g = rm_args(A, M, K, nseg, W, dst, width, ldw, partial);
  if (partial != nullptr) {
    const LaunchEvents e1 = next_events(tm);
    const LaunchEvents e2 = next_events(tm);
    return launch_status(launch_gemm_bf16_splitk(g, stream, e1, e2));
  }
  return launch_status(launch_gemm_bf16(g, stream, next_events(tm)));
}

// One batched transpose launch.
struct Transposes {
  TransposeBatch tb{};
  void add(const void* src, void* dst, int R, int C) {
    tb.src[tb.n] = src;
    tb.dst[tb.n] = dst;
    tb.R[tb.n] = R;
    tb.C[tb.n] = C;
    ++tb.n;
  }
  int launch(hipStream_t stream, Timer* tm) const {
    return launch_status(launch_transpose_bf16(tb, stream, next_events(tm)));
  }
};

// One grouped launch of independent GEMM / reduction jobs.
struct Group {
  GemmGroup gg{};
  Group& add(const GemmArgs& g, int red) {
    if (gg.n < kMaxGroupJobs) {
      gg.job[gg.n] = g;
      gg.reduce[gg.n] = red;
    }
    ++gg.n;  // past kMaxGroupJobs jobs the launcher rejects the group
    return *this;
  }
  Group& gemm(const GemmArgs& g) { return add(g, 0); }
  Group& reduce(const GemmArgs& g) { return add(g, 1); }
  int launch(hipStream_t stream, Timer* tm) const {
    return launch_status(launch_gemm_bf16_group(gg, stream, next_events(tm)));
  }
};

int mha_bwd_launch_count(bool self_attn) { return self_attn ? 6 : 7; }

}  // namespace
}  // namespace mha

using namespace mha;

namespace mha {
int check_backward_args(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* lse, const void* dQ, const void* dK, const void* dV, int B,
                        int h, int n_q, int n_k, int d_k, int d_v, float scale, int mask_kind,
                        const int32_t* key_lengths, int dtype) {
  if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV) return MHA_ERR_NULL;
  int st = check_attn_dims(B, h, n_q, n_k, d_k, d_v);
  if (st != MHA_OK) return st;
  if (!(isfinite(scale) && scale > 0.f)) return MHA_ERR_SCALE;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  if (dtype != MHA_DTYPE_BF16) return MHA_ERR_UNSUPPORTED;
  const void* p16[] = {Q, K, V, O, dO, dQ, dK, dV};
  for (const void* p : p16)
    if (!aligned16(p)) return MHA_ERR_UNSUPPORTED;
  if ((uintptr_t)lse & 3u) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}
}  // namespace mha

extern "C" {

const char* mha_status_str(int status) {
  switch (status) {
    case MHA_OK: return "ok";
    case MHA_ERR_NULL: return "a required pointer is NULL";
    case MHA_ERR_DIM: return "invalid size (non-positive or too large to index)";
    case MHA_ERR_MASK: return "unknown mask kind, or causal mask with n_q != n_k";
    case MHA_ERR_KEYLEN: return "key_lengths missing or a length outside [1, n_k]";
    case MHA_ERR_UNSUPPORTED: return "unsupported head size, dtype, alignment or batch limit";
    case MHA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MHA_ERR_HIP: return "HIP launch failed";
    case MHA_ERR_SCALE: return "scale must be finite and > 0";
    case MHA_ERR_EVENTS: return "timing events missing or fewer than two per launch";
    default: return "unknown status";
  }
}

int mha_forward_launches(int n_q, int n_k, int d_model, int self_attention) {
  if (n_q <= 0 || n_k <= 0 || d_model <= 0) return MHA_ERR_DIM;
  if (use_fused(n_q, n_k, d_model)) return 2;
  return (self_attention && n_q == n_k) ? 3 : 4;
}

size_t mha_workspace_bytes(int B, int n_q, int n_k, int h, int d_k, int d_v, int dtype) {
  if (B <= 0 || n_q <= 0 || n_k <= 0 || h <= 0 || d_k <= 0 || d_v <= 0) return 0;
  if (dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F32) return 0;
  return carve(nullptr, B, n_q, n_k, h, d_k, d_v, dtype).bytes;
}

static int sdpa_impl(const void* Q, const void* K, const void* V, void* O, int B, int h, int n_q,
                     int n_k, int d_k, int d_v, float scale, int mask_kind,
                     const int32_t* key_lengths, int dtype, hipStream_t stream, Timer* tm) {
  if (!Q || !K || !V || !O) return MHA_ERR_NULL;
  int st = check_attn_dims(B, h, n_q, n_k, d_k, d_v);
  if (st != MHA_OK) return st;
  if (!(isfinite(scale) && scale > 0.f)) return MHA_ERR_SCALE;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  if (dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F32) return MHA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return MHA_ERR_UNSUPPORTED;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  set_head_major(a.q_sb, a.q_sh, a.q_sr, h, n_q, d_k);
  set_head_major(a.k_sb, a.k_sh, a.k_sr, h, n_k, d_k);
  set_head_major(a.v_sb, a.v_sh, a.v_sr, h, n_k, d_v);
  set_head_major(a.o_sb, a.o_sh, a.o_sr, h, n_q, d_v);
  a.B = B;
  a.h = h;
  a.n_q = n_q;
  a.n_k = n_k;
  a.scale = scale;
  fill_mask(a, mask_kind);
  return launch_status(launch_attention(a, key_lengths, dtype == MHA_DTYPE_F32, stream, tm));
}

int sdpa_forward(const void* Q, const void* K, const void* V, void* O, int B, int h, int n_q,
                 int n_k, int d_k, int d_v, float scale, int mask_kind,
                 const int32_t* key_lengths, int dtype, hipStream_t stream) {
  return sdpa_impl(Q, K, V, O, B, h, n_q, n_k, d_k, d_v, scale, mask_kind, key_lengths, dtype,
                   stream, nullptr);
}

int sdpa_forward_timed(const void* Q, const void* K, const void* V, void* O, int B, int h,
                       int n_q, int n_k, int d_k, int d_v, float scale, int mask_kind,
                       const int32_t* key_lengths, int dtype, hipStream_t stream,
                       hipEvent_t* events, int capacity, int* n_launches) {
  if (events == nullptr || capacity < 2) return MHA_ERR_EVENTS;
  for (int i = 0; i < 2; ++i)
    if (events[i] == nullptr) return MHA_ERR_EVENTS;
  Timer tm{events, capacity, 0};
  const int st = sdpa_impl(Q, K, V, O, B, h, n_q, n_k, d_k, d_v, scale, mask_kind, key_lengths,
                           dtype, stream, &tm);
  if (n_launches) *n_launches = tm.used;
  return st;
}

int mha_project_in(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                   const void* Wv, int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                   int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!X_q || !X_kv || !Wq || !Wk || !Wv) return MHA_ERR_NULL;
  int st = check_mha(workspace, workspace_bytes, B, n_q, n_k, d_model, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  if (!aligned16(X_q) || !aligned16(X_kv) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv))
    return MHA_ERR_UNSUPPORTED;
  const Workspace w = carve(workspace, B, n_q, n_k, h, d_k, d_v, dtype);
  return do_project_in(X_q, X_kv, Wq, Wk, Wv, B, n_q, n_k, d_model, h, d_k, d_v, w, stream,
                       nullptr);
}

int mha_attend(int B, int n_q, int n_k, int h, int d_k, int d_v, int mask_kind,
               const int32_t* key_lengths, int dtype, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  int st = check_block(workspace, workspace_bytes, B, n_q, n_k, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  const Workspace w = carve(workspace, B, n_q, n_k, h, d_k, d_v, dtype);
  return do_attend(B, n_q, n_k, h, d_k, d_v, mask_kind, key_lengths, w, stream, nullptr);
}

int mha_project_out(const void* Wo, void* Y, int B, int n_q, int n_k, int d_model, int h,
                    int d_k, int d_v, int dtype, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  if (!Wo || !Y) return MHA_ERR_NULL;
  int st = check_mha(workspace, workspace_bytes, B, n_q, n_k, d_model, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  if (!aligned16(Wo) || !aligned16(Y)) return MHA_ERR_UNSUPPORTED;
  const Workspace w = carve(workspace, B, n_q, n_k, h, d_k, d_v, dtype);
  return do_project_out(Wo, Y, B, n_q, d_model, h, d_v, w, stream, nullptr);
}

static int mha_impl(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                    const void* Wv, const void* Wo, void* Y, int B, int n_q, int n_k, int d_model,
                    int h, int d_k, int d_v, int mask_kind, const int32_t* key_lengths, int dtype,
                    void* workspace, size_t workspace_bytes, hipStream_t stream, Timer* tm) {
  if (!X_q || !X_kv || !Wq || !Wk || !Wv || !Wo || !Y) return MHA_ERR_NULL;
  int st = check_mha(workspace, workspace_bytes, B, n_q, n_k, d_model, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  if (!aligned16(X_q) || !aligned16(X_kv) || !aligned16(Wq) || !aligned16(Wk) ||
      !aligned16(Wv) || !aligned16(Wo) || !aligned16(Y))
    return MHA_ERR_UNSUPPORTED;
  const Workspace w = carve(workspace, B, n_q, n_k, h, d_k, d_v, dtype);
  if (use_fused(n_q, n_k, d_model)) {
    ProjAttnArgs pa;
    memset(&pa, 0, sizeof(pa));
    pa.Xq = X_q;
    pa.Xkv = X_kv;
    pa.Wq = Wq;
    pa.Wk = Wk;
    pa.Wv = Wv;
    pa.O = w.O;
    pa.B = B;
    pa.h = h;
    pa.n_q = n_q;
    pa.n_k = n_k;
    pa.d_model = d_model;
    pa.scale = 1.0f / sqrtf((float)d_k);
    pa.causal = (mask_kind & MHA_MASK_CAUSAL) ? 1 : 0;
    pa.padded = (mask_kind & MHA_MASK_KEY_PADDING) ? 1 : 0;
    st = launch_status(launch_fused(pa, key_lengths, stream, tm));
  } else {
    st = do_project_in(X_q, X_kv, Wq, Wk, Wv, B, n_q, n_k, d_model, h, d_k, d_v, w, stream, tm);
    if (st != MHA_OK) return st;
    st = do_attend(B, n_q, n_k, h, d_k, d_v, mask_kind, key_lengths, w, stream, tm);
  }
  if (st != MHA_OK) return st;
  return do_project_out(Wo, Y, B, n_q, d_model, h, d_v, w, stream, tm);
}

int mha_forward(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                const void* Wv, const void* Wo, void* Y, int B, int n_q, int n_k, int d_model,
                int h, int d_k, int d_v, int mask_kind, const int32_t* key_lengths, int dtype,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mha_impl(X_q, X_kv, Wq, Wk, Wv, Wo, Y, B, n_q, n_k, d_model, h, d_k, d_v, mask_kind,
                  key_lengths, dtype, workspace, workspace_bytes, stream, nullptr);
}

int mha_forward_timed(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                      const void* Wv, const void* Wo, void* Y, int B, int n_q, int n_k,
                      int d_model, int h, int d_k, int d_v, int mask_kind,
                      const int32_t* key_lengths, int dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                      int capacity, int* n_launches) {
  const int need = 2 * mha_launch_count(X_q, X_kv, n_q, n_k, d_model);
  if (events == nullptr || capacity < need) return MHA_ERR_EVENTS;
  for (int i = 0; i < need; ++i)
    if (events[i] == nullptr) return MHA_ERR_EVENTS;
  Timer tm{events, capacity, 0};
  const int st = mha_impl(X_q, X_kv, Wq, Wk, Wv, Wo, Y, B, n_q, n_k, d_model, h, d_k, d_v,
                          mask_kind, key_lengths, dtype, workspace, workspace_bytes, stream, &tm);
  if (n_launches) *n_launches = tm.used;
  return st;
}

int add_layernorm_forward(const void* X, const void* F, const void* gamma, const void* beta,
                          void* Y, int M, int d, float eps, int dtype, hipStream_t stream) {
  if (!X || !F || !gamma || !beta || !Y) return MHA_ERR_NULL;
  const int st = check_ln(M, d, eps, dtype);
  if (st != MHA_OK) return st;
  if (!aligned16(X) || !aligned16(F) || !aligned16(gamma) || !aligned16(beta) || !aligned16(Y))
    return MHA_ERR_UNSUPPORTED;
  return do_add_layernorm(X, F, gamma, beta, Y, M, d, eps, stream, nullptr);
}

size_t ffn_workspace_bytes(int M, int d_model, int d_ff, int dtype) {
  if (check_ffn(M, d_model, d_ff, dtype) != MHA_OK) return 0;
  return ffn_ws(M, d_ff);
}

int ffn_forward(const void* X, const void* W1, const void* b1, const void* W2, const void* b2,
                void* Y, int M, int d_model, int d_ff, int dtype, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (!X || !W1 || !b1 || !W2 || !b2 || !Y) return MHA_ERR_NULL;
  int st = check_ffn(M, d_model, d_ff, dtype);
  if (st != MHA_OK) return st;
  if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0 ||
      workspace_bytes < ffn_ws(M, d_ff))
    return MHA_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(W1) || !aligned16(b1) || !aligned16(W2) || !aligned16(b2) ||
      !aligned16(Y))
    return MHA_ERR_UNSUPPORTED;
  return do_ffn(X, W1, b1, W2, b2, Y, M, d_model, d_ff, workspace, stream, nullptr);
}

size_t encoder_layer_workspace_bytes(int B, int n, int d_model, int h, int d_k, int d_v, int d_ff,
                                     int dtype) {
  if (B <= 0 || n <= 0 || d_model <= 0 || h <= 0 || d_k <= 0 || d_v <= 0 || d_ff <= 0) return 0;
  if (dtype != MHA_DTYPE_BF16) return 0;
  if ((int64_t)B * n >= kIndexLimit) return 0;
  return carve_layer(nullptr, B, n, d_model, h, d_k, d_v, d_ff).bytes;
}

int encoder_layer_launches(int n, int d_model) {
  if (n <= 0 || d_model <= 0) return MHA_ERR_DIM;
  return layer_launch_count(n, d_model);
}

static int layer_impl(const void* X, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                      const void* g1, const void* be1, const void* W1, const void* b1,
                      const void* W2, const void* b2, const void* g2, const void* be2, void* Y,
                      int B, int n, int d_model, int h, int d_k, int d_v, int d_ff, float eps,
                      int mask_kind, const int32_t* key_lengths, int dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, Timer* tm) {
  if (!X || !Wq || !Wk || !Wv || !Wo || !g1 || !be1 || !W1 || !b1 || !W2 || !b2 || !g2 || !be2 ||
      !Y)
    return MHA_ERR_NULL;
  int st = check_attn_dims(B, h, n, n, d_k, d_v);
  if (st != MHA_OK) return st;
  st = check_ffn(B * n, d_model, d_ff, dtype);
  if (st != MHA_OK) return st;
  st = check_ln(B * n, d_model, eps, dtype);
  if (st != MHA_OK) return st;
  st = check_mask(mask_kind, B, n, n, key_lengths);
  if (st != MHA_OK) return st;
  if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0 ||
      workspace_bytes < carve_layer(nullptr, B, n, d_model, h, d_k, d_v, d_ff).bytes)
    return MHA_ERR_WORKSPACE;
  const void* ptrs[] = {X, Wq, Wk, Wv, Wo, g1, be1, W1, b1, W2, b2, g2, be2, Y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MHA_ERR_UNSUPPORTED;
  const LayerWorkspace w = carve_layer(workspace, B, n, d_model, h, d_k, d_v, d_ff);
  const int M = B * n;
  // Sublayer 1: S = MultiHead(X, X, X); x1 = LayerNorm1(X + S).
  st = mha_impl(X, X, Wq, Wk, Wv, Wo, w.S, B, n, n, d_model, h, d_k, d_v, mask_kind, key_lengths,
                dtype, workspace, w.blk.bytes, stream, tm);
  if (st != MHA_OK) return st;
  st = do_add_layernorm(X, w.S, g1, be1, w.x1, M, d_model, eps, stream, tm);
  if (st != MHA_OK) return st;
  // Sublayer 2: S = FFN(x1); Y = LayerNorm2(x1 + S).
  st = do_ffn(w.x1, W1, b1, W2, b2, w.S, M, d_model, d_ff, w.H, stream, tm);
  if (st != MHA_OK) return st;
  return do_add_layernorm(w.x1, w.S, g2, be2, Y, M, d_model, eps, stream, tm);
}

int encoder_layer_forward(const void* X, const void* Wq, const void* Wk, const void* Wv,
                          const void* Wo, const void* ln1_gamma, const void* ln1_beta,
                          const void* W1, const void* b1, const void* W2, const void* b2,
                          const void* ln2_gamma, const void* ln2_beta, void* Y, int B, int n,
                          int d_model, int h, int d_k, int d_v, int d_ff, float eps,
                          int mask_kind, const int32_t* key_lengths, int dtype, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return layer_impl(X, Wq, Wk, Wv, Wo, ln1_gamma, ln1_beta, W1, b1, W2, b2, ln2_gamma, ln2_beta, Y,
                    B, n, d_model, h, d_k, d_v, d_ff, eps, mask_kind, key_lengths, dtype,
                    workspace, workspace_bytes, stream, nullptr);
}

int encoder_layer_forward_timed(const void* X, const void* Wq, const void* Wk, const void* Wv,
                                const void* Wo, const void* ln1_gamma, const void* ln1_beta,
                                const void* W1, const void* b1, const void* W2, const void* b2,
                                const void* ln2_gamma, const void* ln2_beta, void* Y, int B,
                                int n, int d_model, int h, int d_k, int d_v, int d_ff, float eps,
                                int mask_kind, const int32_t* key_lengths, int dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* events, int capacity, int* n_launches) {
  if (n <= 0 || d_model <= 0) return MHA_ERR_DIM;
  const int need = 2 * layer_launch_count(n, d_model);
  if (events == nullptr || capacity < need) return MHA_ERR_EVENTS;
  for (int i = 0; i < need; ++i)
    if (events[i] == nullptr) return MHA_ERR_EVENTS;
  Timer tm{events, capacity, 0};
  const int st = layer_impl(X, Wq, Wk, Wv, Wo, ln1_gamma, ln1_beta, W1, b1, W2, b2, ln2_gamma,
                            ln2_beta, Y, B, n, d_model, h, d_k, d_v, d_ff, eps, mask_kind,
                            key_lengths, dtype, workspace, workspace_bytes, stream, &tm);
  if (n_launches) *n_launches = tm.used;
  return st;
}

static int embed_impl(const int32_t* tokens, const void* E, void* out, int B, int n, int vocab,
                      int d_model, int pos0, int dtype, hipStream_t stream, Timer* tm) {
  if (!tokens || !E || !out) return MHA_ERR_NULL;
  if (B <= 0 || n <= 0 || vocab <= 0 || d_model <= 0 || pos0 < 0) return MHA_ERR_DIM;
  if ((int64_t)pos0 + n > ((int64_t)1 << 31) - 1) return MHA_ERR_DIM;
  if ((int64_t)B * n >= kIndexLimit || d_model > kMaxWidth) return MHA_ERR_DIM;
  if (B > 65535 * 8) return MHA_ERR_DIM;
  if (dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F32) return MHA_ERR_UNSUPPORTED;
  if (d_model % 8 != 0) return MHA_ERR_UNSUPPORTED;
  if (((uintptr_t)tokens & 3u) != 0 || !aligned16(E) || !aligned16(out)) return MHA_ERR_UNSUPPORTED;
  EmbedArgs a{tokens, E, out, B, n, vocab, d_model, pos0};
  return launch_status(launch_embed_positional(a, dtype == MHA_DTYPE_F32, stream, next_events(tm)));
}

int embed_positional_forward(const int32_t* tokens, const void* E, void* out, int B, int n,
                             int vocab, int d_model, int pos0, int dtype, hipStream_t stream) {
  return embed_impl(tokens, E, out, B, n, vocab, d_model, pos0, dtype, stream, nullptr);
}

int embed_positional_forward_timed(const int32_t* tokens, const void* E, void* out, int B, int n,
                                   int vocab, int d_model, int pos0, int dtype, hipStream_t stream,
                                   hipEvent_t* events, int capacity, int* n_launches) {
  if (events == nullptr || capacity < 2 || events[0] == nullptr || events[1] == nullptr)
    return MHA_ERR_EVENTS;
  Timer tm{events, capacity, 0};
  const int st = embed_impl(tokens, E, out, B, n, vocab, d_model, pos0, dtype, stream, &tm);
  if (n_launches) *n_launches = tm.used;
  return st;
}

size_t sdpa_decode_workspace_bytes(int B, int h, int n_q, int n_k) {
  if (B <= 0 || h <= 0 || n_q <= 0 || n_k <= 0) return 0;
  const int S = decode_splits(B, h, n_q, n_k, 0);
  const int64_t floats = S > 1 ? (int64_t)B * h * S * kDecodeStateFloats : 0;
  return round_up((size_t)(floats * 4 > 0 ? floats * 4 : 1));
}

int sdpa_decode_launches(int B, int h, int n_q, int n_k, int mask_kind) {
  if (B <= 0 || h <= 0 || n_q <= 0 || n_k <= 0) return MHA_ERR_DIM;
  const int step = (mask_kind & MHA_MASK_KEY_PADDING) ? kLaunchBatch : B;
  return decode_splits(B, h, n_q, n_k, mask_kind) > 1 ? 2 : (B + step - 1) / step;
}

static int decode_impl(const void* Q, const void* K, const void* V, void* O, int B, int h, int n_q,
                       int n_k, int d_k, int d_v, float scale, int mask_kind,
                       const int32_t* key_lengths, int dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, Timer* tm) {
  // The checks of sdpa_forward first (no HIP call before them) ...
  if (!Q || !K || !V || !O) return MHA_ERR_NULL;
  int st = check_attn_dims(B, h, n_q, n_k, d_k, d_v);
  if (st != MHA_OK) return st;
  if (!(isfinite(scale) && scale > 0.f)) return MHA_ERR_SCALE;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  if (dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F32) return MHA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return MHA_ERR_UNSUPPORTED;
  // ... then the split, which reads the device's compute-unit count.
  const int S = dtype == MHA_DTYPE_BF16 ? decode_splits(B, h, n_q, n_k, mask_kind) : 1;
  if (S == 1)  // the plain launch fills the chip (or the split does not apply)
    return sdpa_impl(Q, K, V, O, B, h, n_q, n_k, d_k, d_v, scale, mask_kind, key_lengths, dtype,
                     stream, tm);
  const size_t need = (size_t)B * h * S * kDecodeStateFloats * 4;
  if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0 || workspace_bytes < need)
    return MHA_ERR_WORKSPACE;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  set_head_major(a.q_sb, a.q_sh, a.q_sr, h, n_q, d_k);
  set_head_major(a.k_sb, a.k_sh, a.k_sr, h, n_k, d_k);
  set_head_major(a.v_sb, a.v_sh, a.v_sr, h, n_k, d_v);
  set_head_major(a.o_sb, a.o_sh, a.o_sr, h, n_q, d_v);
  a.B = B;
  a.h = h;
  a.n_q = n_q;
  a.n_k = n_k;
  a.scale = scale;
  a.splits = S;
  a.part = (float*)workspace;
  fill_mask(a, mask_kind);
  if (a.padded) fill_lengths(a, key_lengths, 0);  // B <= kLaunchBatch here
  const LaunchEvents e_part = next_events(tm);
  const LaunchEvents e_merge = next_events(tm);
  return launch_status(launch_attn_decode_split_bf16_d64(a, stream, e_part, e_merge));
}

int sdpa_decode(const void* Q, const void* K, const void* V, void* O, int B, int h, int n_q, int n_k,
                int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lengths, int dtype,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(Q, K, V, O, B, h, n_q, n_k, d_k, d_v, scale, mask_kind, key_lengths, dtype,
                     workspace, workspace_bytes, stream, nullptr);
}

int sdpa_decode_timed(const void* Q, const void* K, const void* V, void* O, int B, int h, int n_q,
                      int n_k, int d_k, int d_v, float scale, int mask_kind,
                      const int32_t* key_lengths, int dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, hipEvent_t* events, int capacity,
                      int* n_launches) {
  if (events == nullptr || capacity < 2) return MHA_ERR_EVENTS;
  for (int i = 0; i < 2; ++i)
    if (events[i] == nullptr) return MHA_ERR_EVENTS;
  Timer tm{events, capacity, 0};
  const int st = decode_impl(Q, K, V, O, B, h, n_q, n_k, d_k, d_v, scale, mask_kind, key_lengths,
                             dtype, workspace, workspace_bytes, stream, &tm);
  if (n_launches) *n_launches = tm.used;
  return st;
}

int sdpa_forward_lse(const void* Q, const void* K, const void* V, void* O, float* lse, int B,
                     int h, int n_q, int n_k, int d_k, int d_v, float scale, int mask_kind,
                     const int32_t* key_lengths, int dtype, hipStream_t stream) {
  if (!Q || !K || !V || !O || !lse) return MHA_ERR_NULL;
  int st = check_attn_dims(B, h, n_q, n_k, d_k, d_v);
  if (st != MHA_OK) return st;
  if (!(isfinite(scale) && scale > 0.f)) return MHA_ERR_SCALE;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  if (dtype != MHA_DTYPE_BF16) return MHA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || ((uintptr_t)lse & 3u))
    return MHA_ERR_UNSUPPORTED;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.lse = lse;
  set_head_major(a.q_sb, a.q_sh, a.q_sr, h, n_q, d_k);
  set_head_major(a.k_sb, a.k_sh, a.k_sr, h, n_k, d_k);
  set_head_major(a.v_sb, a.v_sh, a.v_sr, h, n_k, d_v);
  set_head_major(a.o_sb, a.o_sh, a.o_sr, h, n_q, d_v);
  a.B = B;
  a.h = h;
  a.n_q = n_q;
  a.n_k = n_k;
  a.scale = scale;
  fill_mask(a, mask_kind);
  return launch_status(launch_attention(a, key_lengths, 0, stream, nullptr));
}

size_t sdpa_backward_workspace_bytes(int B, int h, int n_q) {
  if (B <= 0 || h <= 0 || n_q <= 0) return 0;
  return 2 * round_up((size_t)4 * B * h * n_q);
}


static int bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* lse, void* dQ, void* dK, void* dV, int B, int h, int n_q, int n_k,
                    int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lengths,
                    int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream,
                    Timer* tm) {
  const int st = check_backward_args(Q, K, V, O, dO, lse, dQ, dK, dV, B, h, n_q, n_k, d_k, d_v, scale,
                                     mask_kind, key_lengths, dtype);
  if (st != MHA_OK) return st;
  const size_t row_terms = round_up((size_t)4 * B * h * n_q);
  if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0 ||
      workspace_bytes < 2 * row_terms)
    return MHA_ERR_WORKSPACE;
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.lse = lse;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.Dw = (float*)workspace;
  a.Lw = (float*)((char*)workspace + row_terms);
  set_head_major(a.o_sb, a.o_sh, a.o_sr, h, n_q, d_v);
  set_head_major(a.dq_sb, a.dq_sh, a.dq_sr, h, n_q, d_k);
  set_head_major(a.dk_sb, a.dk_sh, a.dk_sr, h, n_k, d_k);
  set_head_major(a.dv_sb, a.dv_sh, a.dv_sr, h, n_k, d_v);
  a.B = B;
  a.h = h;
  a.n_q = n_q;
  a.n_k = n_k;
  a.scale = scale;
  a.causal = (mask_kind & MHA_MASK_CAUSAL) ? 1 : 0;
  a.padded = (mask_kind & MHA_MASK_KEY_PADDING) ? 1 : 0;
  return launch_status(launch_backward(a, key_lengths, stream, tm));
}

int sdpa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* lse, void* dQ, void* dK, void* dV, int B, int h, int n_q, int n_k,
                  int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lengths,
                  int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(Q, K, V, O, dO, lse, dQ, dK, dV, B, h, n_q, n_k, d_k, d_v, scale, mask_kind,
                  key_lengths, dtype, workspace, workspace_bytes, stream, nullptr);
}

int sdpa_backward_timed(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* lse, void* dQ, void* dK, void* dV, int B,
                        int h, int n_q, int n_k, int d_k, int d_v, float scale, int mask_kind,
                        const int32_t* key_lengths, int dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                        int capacity, int* n_launches) {
  if (events == nullptr || capacity < 4) return MHA_ERR_EVENTS;
  for (int i = 0; i < 4; ++i)
    if (events[i] == nullptr) return MHA_ERR_EVENTS;
  Timer tm{events, capacity, 0};
  const int st = bwd_impl(Q, K, V, O, dO, lse, dQ, dK, dV, B, h, n_q, n_k, d_k, d_v, scale,
                          mask_kind, key_lengths, dtype, workspace, workspace_bytes, stream, &tm);
  if (n_launches) *n_launches = tm.used;
  return st;
}

size_t mha_train_workspace_bytes(int B, int n_q, int n_k, int h, int d_k, int d_v, int dtype) {
  if (B <= 0 || n_q <= 0 || n_k <= 0 || h <= 0 || d_k <= 0 || d_v <= 0) return 0;
  if (dtype != MHA_DTYPE_BF16) return 0;
  return carve_train(nullptr, B, n_q, n_k, h, d_k, d_v).bytes;
}

int mha_forward_train(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                      const void* Wv, const void* Wo, void* Y, int B, int n_q, int n_k,
                      int d_model, int h, int d_k, int d_v, int mask_kind,
                      const int32_t* key_lengths, int dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (!X_q || !X_kv || !Wq || !Wk || !Wv || !Wo || !Y) return MHA_ERR_NULL;
  int st = check_mha(workspace, workspace_bytes, B, n_q, n_k, d_model, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
  if (workspace_bytes < carve_train(nullptr, B, n_q, n_k, h, d_k, d_v).bytes) return MHA_ERR_WORKSPACE;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  if (!aligned16(X_q) || !aligned16(X_kv) || !aligned16(Wq) || !aligned16(Wk) ||
      !aligned16(Wv) || !aligned16(Wo) || !aligned16(Y))
    return MHA_ERR_UNSUPPORTED;
  const TrainWs t = carve_train(workspace, B, n_q, n_k, h, d_k, d_v);
  st = do_project_in(X_q, X_kv, Wq, Wk, Wv, B, n_q, n_k, d_model, h, d_k, d_v, t.blk, stream, nullptr);
  if (st != MHA_OK) return st;
  st = do_attend(B, n_q, n_k, h, d_k, d_v, mask_kind, key_lengths, t.blk, stream, nullptr, t.lse);
  if (st != MHA_OK) return st;
  return do_project_out(Wo, Y, B, n_q, d_model, h, d_v, t.blk, stream, nullptr);
}

size_t mha_backward_workspace_bytes(int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                                    int self_attention, int dtype) {
  if (B <= 0 || n_q <= 0 || n_k <= 0 || d_model <= 0 || h <= 0 || d_k <= 0 || d_v <= 0) return 0;
  if (dtype != MHA_DTYPE_BF16 || d_k != d_v) return 0;
  return carve_bwd(nullptr, self_attention && n_q == n_k, B, n_q, n_k, d_model, h, d_k).bytes;
}

static int mha_bwd_impl(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                        const void* Wv, const void* Wo, const void* dY, void* dX_q, void* dX_kv,
                        void* dWq, void* dWk, void* dWv, void* dWo, int B, int n_q, int n_k,
                        int d_model, int h, int d_k, int d_v, int mask_kind,
                        const int32_t* key_lengths, int dtype, const void* train_ws,
                        size_t train_ws_bytes, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, Timer* tm) {
  const bool self_attn = X_q == X_kv && n_q == n_k;
  if (!X_q || !X_kv || !Wq || !Wk || !Wv || !Wo || !dY || !dX_q || !dWq || !dWk || !dWv || !dWo)
    return MHA_ERR_NULL;
  if (!self_attn && !dX_kv) return MHA_ERR_NULL;
  int st = check_mha(train_ws, train_ws_bytes, B, n_q, n_k, d_model, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st == MHA_ERR_WORKSPACE ? MHA_ERR_WORKSPACE : st;
  if (train_ws_bytes < carve_train(nullptr, B, n_q, n_k, h, d_k, d_v).bytes) return MHA_ERR_WORKSPACE;
  st = check_mask(mask_kind, B, n_q, n_k, key_lengths);
  if (st != MHA_OK) return st;
  const int64_t Mq = (int64_t)B * n_q, Mk = (int64_t)B * n_k;
  // The transposed activations are GEMM operands with Mq (Mk) columns.
  if (Mq % 8 != 0 || Mk % 8 != 0) return MHA_ERR_UNSUPPORTED;
  if (Mq > (int64_t)65535 * 64 || Mk > (int64_t)65535 * 64) return MHA_ERR_DIM;
  if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0 ||
      workspace_bytes < carve_bwd(nullptr, self_attn, B, n_q, n_k, d_model, h, d_k).bytes)
    return MHA_ERR_WORKSPACE;
  const void* p16[] = {X_q, X_kv, Wq, Wk, Wv, Wo, dY, dX_q, dWq, dWk, dWv, dWo};
  for (const void* p : p16)
    if (!aligned16(p)) return MHA_ERR_UNSUPPORTED;
  if (!self_attn && !aligned16(dX_kv)) return MHA_ERR_UNSUPPORTED;

  const TrainWs t = carve_train((void*)train_ws, B, n_q, n_k, h, d_k, d_v);
  const BwdWs w = carve_bwd(workspace, self_attn, B, n_q, n_k, d_model, h, d_k);
  const int hd = h * d_k, dm = d_model;
  const size_t wblock = (size_t)hd * dm;  // elements of one transposed weight
  // Every transposed operand in one launch: W^O^T, C^T, the input weights'
  // transposes (stacked for self-attention) and the inputs' transposes.
  {
    Transposes tr;
    tr.add(Wo, w.WoT, hd, dm);
    tr.add(t.blk.O, w.OcT, (int)Mq, hd);
    if (self_attn) {
      tr.add(Wq, w.WT, dm, hd);
      tr.add(Wk, (__bf16*)w.WT + wblock, dm, hd);
      tr.add(Wv, (__bf16*)w.WT + 2 * wblock, dm, hd);
      tr.add(X_q, w.XqT, (int)Mq, dm);
    } else {
      tr.add(Wq, w.WT, dm, hd);
      tr.add(Wk, w.WkvT, dm, hd);
      tr.add(Wv, (__bf16*)w.WkvT + wblock, dm, hd);
      tr.add(X_q, w.XqT, (int)Mq, dm);
      tr.add(X_kv, w.XkvT, (int)Mk, dm);
    }
    st = tr.launch(stream, tm);
    if (st != MHA_OK) return st;
  }
  // One launch: dC = dY W^O^T, scattered per head into dO [B][h][n_q][d],
  // and the split-K partial sums of dW^O = C^T dY (reduced in a later launch).
  GemmArgs g_dwo;
  {
    GemmArgs g{};
    g.A = dY;
    g.M = (int)Mq;
    g.K = dm;
    g.nseg = 1;
    g.seg[0] = GemmSeg{w.WoT, w.dO, hd, d_v, h, n_q, 0};
    g.col_start[0] = 0;
    g.col_start[1] = hd;
    const void* W[1] = {dY};
    void* D[1] = {dWo};
    const int wd[1] = {dm};
    g_dwo = rm_args(w.OcT, hd, (int)Mq, 1, W, D, wd, 0, w.partial);
    st = Group().gemm(g).gemm(g_dwo).launch(stream, tm);
    if (st != MHA_OK) return st;
  }
  // attention gradients, written with the heads concatenated
  {
    BwdArgs a;
    memset(&a, 0, sizeof(a));
    a.Q = t.blk.Q;
    a.K = t.blk.K;
    a.V = t.blk.V;
    a.O = t.blk.O;
    a.dO = w.dO;
    a.lse = t.lse;
    a.Dw = w.rows;
    a.Lw = (float*)((char*)w.rows + w.rows_each);
    a.o_sb = (int64_t)n_q * hd;
    a.o_sh = d_v;
    a.o_sr = hd;
    const int ldq = self_attn ? 3 * hd : hd;  // row stride of the dQ buffer
    const int ldkv = self_attn ? 3 * hd : 2 * hd;
    __bf16* dq = (__bf16*)w.dQKV;
    __bf16* dk = self_attn ? dq + hd : (__bf16*)w.dKV;
    __bf16* dv = dk + hd;
    a.dQ = dq;
    a.dK = dk;
    a.dV = dv;
    a.dq_sb = (int64_t)n_q * ldq;
    a.dq_sh = d_k;
    a.dq_sr = ldq;
    a.dk_sb = a.dv_sb = (int64_t)n_k * ldkv;
    a.dk_sh = a.dv_sh = d_k;
    a.dk_sr = a.dv_sr = ldkv;
    a.B = B;
    a.h = h;
    a.n_q = n_q;
    a.n_k = n_k;
    a.scale = 1.0f / sqrtf((float)d_k);
    a.causal = (mask_kind & MHA_MASK_CAUSAL) ? 1 : 0;
    a.padded = (mask_kind & MHA_MASK_KEY_PADDING) ? 1 : 0;
    st = launch_status(launch_backward(a, key_lengths, stream, tm));
    if (st != MHA_OK) return st;
  }
  if (self_attn) {
    // One launch: dX = [dQ | dK | dV] [W^Q | W^K | W^V]^T, the partial sums
    // of [dW^Q | dW^K | dW^V] = X^T [dQ | dK | dV], and the reduction of dW^O.
    const void* W[1] = {w.WT};
    void* D[1] = {dX_q};
    const int wd[1] = {dm};
    const GemmArgs g_dx = rm_args(w.dQKV, (int)Mq, 3 * hd, 1, W, D, wd, 0);
    const void* W3[3] = {w.dQKV, (__bf16*)w.dQKV + hd, (__bf16*)w.dQKV + 2 * hd};
    void* D3[3] = {dWq, dWk, dWv};
    const int wd3[3] = {hd, hd, hd};
    const GemmArgs g_dw = rm_args(w.XqT, dm, (int)Mq, 3, W3, D3, wd3, 3 * hd, w.partial1);
    st = Group().gemm(g_dx).gemm(g_dw).reduce(g_dwo).launch(stream, tm);
    if (st != MHA_OK) return st;
    return Group().reduce(g_dw).launch(stream, tm);
  }
  // cross-attention.  One launch: dX_q = dQ W^Q^T, dX_kv = [dK | dV]
  // [W^K | W^V]^T and the reduction of dW^O; one launch: the partial sums of
  // dW^Q = X_q^T dQ and [dW^K | dW^V] = X_kv^T [dK | dV]; one launch: their
  // reductions.
  {
    const void* W[1] = {w.WT};
    void* D[1] = {dX_q};
    const int wd[1] = {dm};
    const GemmArgs g_dxq = rm_args(w.dQKV, (int)Mq, hd, 1, W, D, wd, 0);
    const void* W2[1] = {w.WkvT};
    void* D2[1] = {dX_kv};
    const GemmArgs g_dxkv = rm_args(w.dKV, (int)Mk, 2 * hd, 1, W2, D2, wd, 0);
    st = Group().gemm(g_dxq).gemm(g_dxkv).reduce(g_dwo).launch(stream, tm);
    if (st != MHA_OK) return st;
  }
  {
    const void* W[1] = {w.dQKV};
    void* D[1] = {dWq};
    const int wd[1] = {hd};
    const GemmArgs g_dwq = rm_args(w.XqT, dm, (int)Mq, 1, W, D, wd, 0, w.partial1);
    const void* W2[2] = {w.dKV, (__bf16*)w.dKV + hd};
    void* D2[2] = {dWk, dWv};
    const int wd2[2] = {hd, hd};
    const GemmArgs g_dwkv = rm_args(w.XkvT, dm, (int)Mk, 2, W2, D2, wd2, 2 * hd, w.partial2);
    st = Group().gemm(g_dwq).gemm(g_dwkv).launch(stream, tm);
    if (st != MHA_OK) return st;
    return Group().reduce(g_dwq).reduce(g_dwkv).launch(stream, tm);
  }
}

int mha_backward(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                 const void* Wv, const void* Wo, const void* dY, void* dX_q, void* dX_kv,
                 void* dWq, void* dWk, void* dWv, void* dWo, int B, int n_q, int n_k,
                 int d_model, int h, int d_k, int d_v, int mask_kind, const int32_t* key_lengths,
                 int dtype, const void* train_workspace, size_t train_workspace_bytes,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mha_bwd_impl(X_q, X_kv, Wq, Wk, Wv, Wo, dY, dX_q, dX_kv, dWq, dWk, dWv, dWo, B, n_q, n_k,
                      d_model, h, d_k, d_v, mask_kind, key_lengths, dtype, train_workspace,
                      train_workspace_bytes, workspace, workspace_bytes, stream, nullptr);
}

int mha_backward_timed(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                       const void* Wv, const void* Wo, const void* dY, void* dX_q, void* dX_kv,
                       void* dWq, void* dWk, void* dWv, void* dWo, int B, int n_q, int n_k,
                       int d_model, int h, int d_k, int d_v, int mask_kind,
                       const int32_t* key_lengths, int dtype, const void* train_workspace,
                       size_t train_workspace_bytes, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, hipEvent_t* events, int capacity, int* n_launches) {
  const int need = 2 * mha_bwd_launch_count(X_q == X_kv && n_q == n_k);
  if (events == nullptr || capacity < need) return MHA_ERR_EVENTS;
  for (int i = 0; i < need; ++i)
    if (events[i] == nullptr) return MHA_ERR_EVENTS;
  Timer tm{events, capacity, 0};
  const int st = mha_bwd_impl(X_q, X_kv, Wq, Wk, Wv, Wo, dY, dX_q, dX_kv, dWq, dWk, dWv, dWo, B, n_q,
                              n_k, d_model, h, d_k, d_v, mask_kind, key_lengths, dtype,
                              train_workspace, train_workspace_bytes, workspace, workspace_bytes,
                              stream, &tm);
  if (n_launches) *n_launches = tm.used;
  return st;
}

int mha_backward_launches(int self_attention) {
  return mha_bwd_launch_count(self_attention != 0);
}

}  // extern "C"
