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

void fill_mask(AttnArgs& a, int mask_kind, const int32_t* key_lengths) {
  a.causal = (mask_kind & MHA_MASK_CAUSAL) ? 1 : 0;
  a.padded = (mask_kind & MHA_MASK_KEY_PADDING) ? 1 : 0;
  if (a.padded)
    for (int b = 0; b < a.B; ++b) a.key_len[b] = key_lengths[b];
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
  if (d_model <= 0 || d_model >= kIndexLimit / 8) return MHA_ERR_DIM;
  int st = check_block(ws, ws_bytes, B, n_q, n_k, h, d_k, d_v, dtype);
  if (st != MHA_OK) return st;
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
              const int32_t* key_lengths, const Workspace& w, hipStream_t stream, Timer* tm) {
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
  fill_mask(a, mask_kind, key_lengths);
  return launch_status(launch_attn_bf16_d64(a, stream, next_events(tm)));
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

}  // namespace
}  // namespace mha

using namespace mha;

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
  fill_mask(a, mask_kind, key_lengths);
  const LaunchEvents le = next_events(tm);
  const hipError_t e = dtype == MHA_DTYPE_BF16 ? launch_attn_bf16_d64(a, stream, le)
                                               : launch_attn_f32_d64(a, stream, le);
  return launch_status(e);
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
    if (pa.padded)
      for (int b = 0; b < B; ++b) pa.key_len[b] = key_lengths[b];
    st = launch_status(launch_proj_attn_bf16(pa, stream, next_events(tm)));
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

}  // extern "C"
