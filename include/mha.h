/*
 * mha.h -- C ABI of libmha: multi-head scaled dot-product attention, forward,
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are web pages on the 2017 paper "Attention Is
 * All You Need"; each entry point cites the passage that defines it):
 *
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k) + M) V           per head
 *   head_i   = Attention(X_q W_i^Q, X_kv W_i^K, X_kv W_i^V)
 *   MultiHead = Concat(head_1, ..., head_h) W^O
 *
 * with M an additive 0 / -inf mask applied before the row softmax; and,
 * around the block, one Post-LN encoder layer:
 *
 *   x1 = LayerNorm(X + MultiHead(X, X, X)),  Y = LayerNorm(x1 + FFN(x1)),
 *   FFN(x) = max(0, x W1 + b1) W2 + b2,
 *
 * and the layer's input, X = E[tokens] * sqrt(d_model) + PE (sinusoidal).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers to caller-owned, row-major,
 *   densely packed memory, in the dtype given by `dtype`, except
 *   `key_lengths`, which is a HOST pointer (read during the call only).
 * - Math orientation is X.W as on the pages: W^Q, W^K are d_model x (h*d_k),
 *   W^V is d_model x (h*d_v), W^O is (h*d_v) x d_model.  Holders of weights in
 *   [out][in] layout pass the transpose.  The attention block has no biases
 *   (the feed-forward and LayerNorm entry points at the end carry theirs).
 * - Head i owns the contiguous column block [i*d, (i+1)*d) of a stacked
 *   projection and the row block [i*d_v, (i+1)*d_v) of W^O.
 * - Accumulation is always fp32.  bf16 intermediates (Q, K, V, softmax
 *   weights fed to the second product, the concatenated heads) are rounded
 *   to nearest even.
 * - Work is enqueued on `stream` and the call returns before it completes.
 *   The library allocates nothing, keeps no pointer after returning and
 *   holds no global state; calls on different streams may run concurrently
 *   as long as their output buffers do not overlap.
 * - Every argument check runs on the host before any HIP call; a failed
 *   check returns a negative status and enqueues nothing.  MHA_ERR_HIP
 *   reports a launch failure (hipGetLastError after the launches).  No C++
 *   exception crosses this interface.
 *
 * Supported on the GPU in this version: d_k = d_v = 64 for attention;
 * bf16 for every entry point; fp32 for sdpa_forward and
 * embed_positional_forward.  Other combinations return MHA_ERR_UNSUPPORTED.
 */
#ifndef MHA_H
#define MHA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MHA_OK                 0
#define MHA_ERR_NULL          -1  /* a required pointer is NULL                    */
#define MHA_ERR_DIM           -2  /* a size is <= 0, or an index would overflow    */
#define MHA_ERR_MASK          -3  /* unknown mask kind, or causal with n_q != n_k  */
#define MHA_ERR_KEYLEN        -4  /* key_lengths missing, or a length outside [1, n_k] */
#define MHA_ERR_UNSUPPORTED   -5  /* head size / dtype / batch limit not supported */
#define MHA_ERR_WORKSPACE     -6  /* workspace missing or smaller than required    */
#define MHA_ERR_HIP           -7  /* a HIP launch failed                           */
#define MHA_ERR_SCALE         -8  /* scale not finite or not > 0                   */
#define MHA_ERR_EVENTS        -9  /* timing events missing or too few              */

/* Mask kinds (bit 0: causal, bit 1: key padding). */
#define MHA_MASK_NONE              0
#define MHA_MASK_CAUSAL            1  /* key j hidden from query i when j > i      */
#define MHA_MASK_KEY_PADDING       2  /* key j hidden in batch b when j >= L_b     */
#define MHA_MASK_CAUSAL_KEY_PADDING 3

/* Element types. */
#define MHA_DTYPE_BF16  0
#define MHA_DTYPE_F32   1

/* Largest batch accepted together with key padding.  The lengths travel to
 * the kernels inside their argument blocks, 256 batches per launch: a padded
 * call over more batches is split on the host into launches of at most 256
 * batches each (a *_timed call then records one event pair per launch). */
#define MHA_MAX_PADDED_BATCH 1024

/*
 * sdpa_forward -- bare scaled dot-product attention for every (batch, head).
 *
 * Defines: softmax(Q K^T * scale + M) V, rows = queries, columns = keys,
 * softmax along each row.  Sources: hex4c59.cc "读懂 Attention Is All You
 * Need", sections "六步算完一行注意力", "把所有位置合并，就是那条核心公式" and
 * "为什么要按键的维度缩放？"; devpress.csdn.net "【深度学习】Transformer",
 * section 2.1, equation (2.4).  The mask is added before the softmax
 * (hex4c59.cc, section "掩码必须在 softmax 之前生效"; devpress.csdn.net
 * section 3.1 prints the causal pattern).
 *
 *   Q [B][h][n_q][d_k], K [B][h][n_k][d_k], V [B][h][n_k][d_v]  (inputs)
 *   O [B][h][n_q][d_v]                                           (output)
 *   scale       finite and > 0 (the method uses 1/sqrt(d_k))
 *   mask_kind   MHA_MASK_*; causal needs n_q == n_k
 *   key_lengths host int32[B], each in [1, n_k]; required iff the padding bit
 *               is set (B <= MHA_MAX_PADDED_BATCH), ignored otherwise
 *   dtype       MHA_DTYPE_BF16 or MHA_DTYPE_F32 (Q, K, V, O all of it)
 *
 * The n_q x n_k score matrix is never stored: one fused kernel streams K/V
 * tiles and keeps a running row maximum and row sum (an exact reformulation
 * of the row softmax).  With bf16, at most 32 queries, no causal bit and
 * more than 128 keys (one new query per sequence against its cached keys,
 * the incremental-decoding shape), the kernel splits each head's keys over
 * its waves and merges their partial row states: the same softmax, summed in
 * another order.  O must not overlap Q, K or V.
 */
int sdpa_forward(const void* Q, const void* K, const void* V, void* O,
                 int B, int h, int n_q, int n_k, int d_k, int d_v,
                 float scale, int mask_kind, const int32_t* key_lengths,
                 int dtype, hipStream_t stream);

/*
 * sdpa_decode -- sdpa_forward for the incremental-decoding shape (few new
 * queries per sequence against long cached key ranges; hex4c59.cc
 * "读懂 Attention Is All You Need", section "训练能并行，不意味着一次生成整句话":
 * generation produces one position per step).  Same arguments, result and
 * checks as sdpa_forward, plus a workspace.  When n_q <= 32, no causal bit,
 * n_k > 128, B <= 256 and B * h is below the device's compute-unit count,
 * the key tiles of each (batch, head) are dealt to several workgroups, each
 * leaving its partial softmax state (reference m, sum l, accumulator) in the
 * workspace, and a second launch merges them (the same softmax: the split
 * only reorders the sum over keys).  Otherwise it is sdpa_forward and the
 * workspace is not touched.
 *   workspace  >= sdpa_decode_workspace_bytes(B, h, n_q, n_k), 256-byte
 *              aligned, caller-owned device memory (contents need no init).
 * Errors as sdpa_forward; MHA_ERR_WORKSPACE if a split call's workspace is
 * missing, misaligned or too small.
 */
int sdpa_decode(const void* Q, const void* K, const void* V, void* O,
                int B, int h, int n_q, int n_k, int d_k, int d_v,
                float scale, int mask_kind, const int32_t* key_lengths, int dtype,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of sdpa_decode (at least 256; the split count depends on
 * the current device's compute units); 0 for non-positive sizes. */
size_t sdpa_decode_workspace_bytes(int B, int h, int n_q, int n_k);

/* Launches an sdpa_decode call makes on the current device (2 when it
 * splits); a negative status for invalid sizes. */
int sdpa_decode_launches(int B, int h, int n_q, int n_k, int mask_kind);

/* sdpa_decode with launch events, as the other _timed variants. */
int sdpa_decode_timed(const void* Q, const void* K, const void* V, void* O,
                      int B, int h, int n_q, int n_k, int d_k, int d_v,
                      float scale, int mask_kind, const int32_t* key_lengths, int dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t* events, int capacity, int* n_launches);

/*
 * mha_workspace_bytes -- device scratch that mha_forward and the stage calls
 * need for the projected heads and the concatenated attention output:
 *   Q [B][h][n_q][d_k], K [B][h][n_k][d_k], V [B][h][n_k][d_v],
 *   O concat [B][n_q][h*d_v], each 256-byte aligned, in the element type.
 * Returns 0 for invalid sizes.
 */
size_t mha_workspace_bytes(int B, int n_q, int n_k, int h, int d_k, int d_v, int dtype);

/*
 * mha_forward -- the multi-head attention block, Concat(head_1..head_h) W^O.
 *
 * Sources: devpress.csdn.net "【深度学习】Transformer", section 2.2 (MultiHead
 * formula and the shapes W_i^Q, W_i^K in R^{d x d_k}, W_i^V in R^{d x d_v},
 * W^O in R^{h d_v x d}); hex4c59.cc, sections "Q、K、V 是三种计算角色" and
 * "多头注意力让一次读取有多组投影".  The three uses of the block
 * (hex4c59.cc, section "解码器有两种读取：看前缀，以及看源句"; wiki.hugogu.cn
 * table of attention uses; devpress.csdn.net section 3.2):
 *   encoder self-attention     X_kv == X_q, mask NONE
 *   decoder masked self-attn   X_kv == X_q, mask CAUSAL
 *   encoder-decoder (cross)    X_q from the decoder, X_kv from the encoder,
 *                              n_q may differ from n_k, optional key padding
 *
 *   X_q [B][n_q][d_model], X_kv [B][n_k][d_model]  (X_kv may equal X_q)
 *   Wq, Wk [d_model][h*d_k], Wv [d_model][h*d_v], Wo [h*d_v][d_model]
 *   Y [B][n_q][d_model]                            (output)
 *   scale is fixed at 1/sqrt(d_k).
 *   workspace   device buffer of at least mha_workspace_bytes(...) bytes,
 *               owned by the caller, not read before it is written.
 *   dtype       MHA_DTYPE_BF16.
 *
 * Launch plan (see mha_forward_launches): when n_q <= 128, n_k <= 128 and
 * d_model is a multiple of 64, one fused kernel per (batch, head) computes
 * that head's Q, K, V tiles in on-chip memory and its attention output
 * (written to the workspace's concatenated-heads region), then the output
 * projection runs.  Otherwise, when X_kv == X_q (same pointer) and
 * n_q == n_k, the three input projections run as one GEMM over the stacked
 * weights (two GEMMs for cross-attention), then attention, then the output
 * projection.  Both plans compute the same products in the same order and
 * give identical results.  Y must not overlap any input or the workspace.
 */
int mha_forward(const void* X_q, const void* X_kv,
                const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                void* Y,
                int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                int mask_kind, const int32_t* key_lengths, int dtype,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The three stages of mha_forward, callable on their own with the same
 * arguments (each ignores what it does not use).  mha_project_in;
 * mha_attend; mha_project_out on one stream gives exactly mha_forward's
 * result (and fills the workspace Q, K, V, which the fused plan of
 * mha_forward does not write).  They share the workspace layout documented
 * at mha_workspace_bytes.
 *
 * mha_project_in  -- Q = X_q W^Q, K = X_kv W^K, V = X_kv W^V, written per head
 *                    into the workspace (devpress.csdn.net section 2.1,
 *                    equations (2.1)-(2.3); hex4c59.cc section
 *                    "Q、K、V 是三种计算角色").
 * mha_attend      -- per-head attention of the workspace Q, K, V, written in
 *                    concatenated layout [B][n_q][h*d_v] (the Concat of the
 *                    MultiHead formula).
 * mha_project_out -- Y = Concat . W^O.
 */
int mha_project_in(const void* X_q, const void* X_kv, const void* Wq, const void* Wk,
                   const void* Wv,
                   int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                   int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

int mha_attend(int B, int n_q, int n_k, int h, int d_k, int d_v,
               int mask_kind, const int32_t* key_lengths, int dtype,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

int mha_project_out(const void* Wo, void* Y,
                    int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                    int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Instrumented variants of sdpa_forward and mha_forward, for benchmarks and
 * profilers: the same checks, launches and results, and in addition kernel
 * launch i (in launch order, i = 0, 1, ...) records events[2i] when the
 * kernel starts and events[2i+1] when it ends (AMD hipExtLaunchKernel launch
 * events; elapsed times between them are pure kernel execution).  The caller
 * creates the events (default flags) and owns them.  Launch counts:
 * sdpa_forward 1; mha_forward as mha_forward_launches returns (2: fused
 * projection + attention, output projection; 3: stacked input projection,
 * attention, output projection; 4: Q projection, K/V projection,
 * attention, output projection).  `capacity` is the number of
 * events passed; fewer than two per launch, or a NULL event among them, is
 * MHA_ERR_EVENTS.  *n_launches (if not NULL) receives the launch count.
 */
int sdpa_forward_timed(const void* Q, const void* K, const void* V, void* O,
                       int B, int h, int n_q, int n_k, int d_k, int d_v,
                       float scale, int mask_kind, const int32_t* key_lengths,
                       int dtype, hipStream_t stream,
                       hipEvent_t* events, int capacity, int* n_launches);

int mha_forward_timed(const void* X_q, const void* X_kv,
                      const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                      void* Y,
                      int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                      int mask_kind, const int32_t* key_lengths, int dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t* events, int capacity, int* n_launches);

/*
 * mha_forward_launches -- number of kernels mha_forward launches for these
 * sizes (2, 3 or 4, see the launch plan at mha_forward); self_attention is
 * nonzero when X_kv will be the same pointer as X_q.  Host-only, no HIP
 * call.  MHA_ERR_DIM for non-positive sizes.
 */
int mha_forward_launches(int n_q, int n_k, int d_model, int self_attention);

/*
 * ---------------------------------------------------------------------------
 * Training: the forward with its row log-sum-exp, and the backward pass.
 * ---------------------------------------------------------------------------
 */

/*
 * sdpa_forward_lse -- sdpa_forward (bf16 only) that also writes, for every
 * query row, the log-sum-exp the backward pass recomputes the weights from:
 *   lse[(b*h + head)*n_q + i] = ln( sum over visible keys j of
 *                                   exp(scale * q_i . k_j) )
 * so that softmax weight P_ij = exp(scale * q_i . k_j - lse_i).
 *   lse  DEVICE float [B][h][n_q], 4-byte aligned, caller-owned.
 * Other arguments, results and errors as sdpa_forward (O is bit-identical).
 * The sum is the one the forward normalises by (its weights rounded to bf16
 * as they enter the second product).
 */
int sdpa_forward_lse(const void* Q, const void* K, const void* V, void* O, float* lse,
                     int B, int h, int n_q, int n_k, int d_k, int d_v,
                     float scale, int mask_kind, const int32_t* key_lengths,
                     int dtype, hipStream_t stream);

/*
 * sdpa_backward_workspace_bytes -- scratch of sdpa_backward: two fp32 row
 * arrays [B][h][n_q], each 256-byte rounded: -D_i (D_i = sum_d dO_id O_id)
 * and -lse_i / scale.  0 for invalid sizes.
 */
size_t sdpa_backward_workspace_bytes(int B, int h, int n_q);

/*
 * sdpa_backward -- gradients of O = softmax(Q K^T * scale + M) V:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale * dS K,  dK = scale * dS^T Q,   P = exp(S - lse)
 * The gradient of the forward's definition (devpress.csdn.net
 * "【深度学习】Transformer", section 2.1, equation (2.4)) through its steps in
 * reverse order; training back-propagates the losses of all positions at
 * once (hex4c59.cc "读懂 Attention Is All You Need", sections "训练能并行，
 * 不意味着一次生成整句话" and "参数是怎样学出来的？").
 *
 *   Q, K, V, O  the forward's inputs and output; lse from sdpa_forward_lse
 *   dO          upstream gradient [B][h][n_q][d_v]
 *   dQ, dK, dV  outputs, shaped as Q, K, V; must not overlap any input.
 *               Keys no query can see get zero dK and dV.
 *   scale, mask_kind, key_lengths  as the forward (they must be the same)
 *   workspace   >= sdpa_backward_workspace_bytes(B, h, n_q), 256-byte aligned
 *   dtype       MHA_DTYPE_BF16 (d_k = d_v = 64), fp32 accumulation; P and
 *               dS are rounded to bf16 as they enter the accumulating
 *               products.
 * Two launches, no atomics (results are deterministic): one kernel per
 * 128-query block computes dQ and D; one per 128-key block computes dK, dV.
 */
int sdpa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* lse, void* dQ, void* dK, void* dV,
                  int B, int h, int n_q, int n_k, int d_k, int d_v,
                  float scale, int mask_kind, const int32_t* key_lengths, int dtype,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sdpa_backward_noalloc -- sdpa_backward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc.  Same arguments, checks and
 * kernels as sdpa_backward, without the workspace: the row terms live in an
 * 8 MiB device array of the library (one per GPU, held until the process
 * ends), so B * h * n_q may be at most 2^20 (else MHA_ERR_WORKSPACE, before
 * any HIP call).  The array's device address is looked up on the first call
 * on each device; MHA_ERR_HIP if that lookup fails.  Calls on one GPU share
 * the array: calls that overlap in time on one GPU (different streams) race
 * and must be ordered by the caller.  Allocates nothing.
 */
int sdpa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O,
                          const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                          int B, int h, int n_q, int n_k, int d_k, int d_v,
                          float scale, int mask_kind, const int32_t* key_lengths, int dtype,
                          hipStream_t stream);

/* sdpa_backward with launch events (2 launches), as the other _timed variants. */
int sdpa_backward_timed(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                        int B, int h, int n_q, int n_k, int d_k, int d_v,
                        float scale, int mask_kind, const int32_t* key_lengths, int dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                        hipEvent_t* events, int capacity, int* n_launches);

/*
 * mha_train_workspace_bytes -- state mha_forward_train keeps for
 * mha_backward: the block workspace of mha_workspace_bytes (Q, K, V
 * head-major, the concatenated heads) followed by the row log-sum-exp
 * [B][h][n_q] (fp32), 256-byte aligned.  0 for invalid sizes; bf16 only.
 */
size_t mha_train_workspace_bytes(int B, int n_q, int n_k, int h, int d_k, int d_v, int dtype);

/*
 * mha_forward_train -- mha_forward for training: the same Y (same kernels
 * as the staged plan: stacked or split input projections, attention,
 * output projection), keeping in the workspace everything mha_backward
 * needs.  Arguments as mha_forward; workspace >=
 * mha_train_workspace_bytes(...).
 */
int mha_forward_train(const void* X_q, const void* X_kv,
                      const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                      void* Y,
                      int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                      int mask_kind, const int32_t* key_lengths, int dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mha_backward_workspace_bytes -- scratch of mha_backward (transposed
 * operands, the per-head upstream gradient, the attention gradients with
 * their heads concatenated, row terms).  self_attention nonzero when X_kv
 * will be the same pointer as X_q (and n_q == n_k).  0 for invalid sizes.
 */
size_t mha_backward_workspace_bytes(int B, int n_q, int n_k, int d_model, int h, int d_k,
                                    int d_v, int self_attention, int dtype);

/*
 * mha_backward -- gradients of the multi-head block Y = Concat(head_1..h) W^O
 * (devpress.csdn.net "【深度学习】Transformer", section 2.2) for the upstream
 * gradient dY [B][n_q][d_model], through the block's steps in reverse:
 *   dC = dY W^O^T,  dW^O = C^T dY            (C: concatenated heads)
 *   dQ, dK, dV of each head                  (as sdpa_backward)
 *   dW^Q = X_q^T dQ_c,  dW^K = X_kv^T dK_c,  dW^V = X_kv^T dV_c
 *   dX_q = dQ_c W^Q^T,  dX_kv = dK_c W^K^T + dV_c W^V^T
 * (_c: heads concatenated, [rows][h*d]).  Training back-propagates through
 * every part (hex4c59.cc "读懂 Attention Is All You Need", section
 * "参数是怎样学出来的？").
 *
 *   X_q, X_kv, Wq, Wk, Wv, Wo, B ... key_lengths, dtype: exactly as the
 *       mha_forward_train call whose workspace is passed as train_workspace
 *       (read only).
 *   dY  [B][n_q][d_model];  outputs dWq, dWk [d_model][h*d_k], dWv
 *       [d_model][h*d_v], dWo [h*d_v][d_model], dX_q [B][n_q][d_model] and,
 *       for cross-attention, dX_kv [B][n_k][d_model].  Self-attention (X_kv
 *       the same pointer as X_q, n_q == n_k): dX_q receives the gradient
 *       with respect to the shared input (both paths summed) and dX_kv is
 *       ignored.  Outputs must not overlap inputs or workspaces.
 *   workspace >= mha_backward_workspace_bytes(...), 256-byte aligned.
 *   B*n_q and B*n_k must be multiples of 8 (MHA_ERR_UNSUPPORTED): the
 *   transposed activations are GEMM operands of that width.
 * Launches (mha_backward_launches): one batched transpose of W^O, C, the
 * input weights (stacked for self-attention) and the inputs (bandwidth-bound
 * copies that let the projection GEMM take every product as A . B with
 * row-major operands); the GEMMs for dC and dX and the weight-gradient GEMMs
 * split over K (fp32 partial sums in the workspace, each added up and
 * rounded once by a reduction), with independent GEMMs and reductions
 * sharing a launch; and the two attention-backward kernels.  bf16 in and
 * out, fp32 accumulation.
 */
int mha_backward(const void* X_q, const void* X_kv,
                 const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                 const void* dY, void* dX_q, void* dX_kv,
                 void* dWq, void* dWk, void* dWv, void* dWo,
                 int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                 int mask_kind, const int32_t* key_lengths, int dtype,
                 const void* train_workspace, size_t train_workspace_bytes,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* mha_backward with launch events, as the other _timed variants. */
int mha_backward_timed(const void* X_q, const void* X_kv,
                       const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                       const void* dY, void* dX_q, void* dX_kv,
                       void* dWq, void* dWk, void* dWv, void* dWo,
                       int B, int n_q, int n_k, int d_model, int h, int d_k, int d_v,
                       int mask_kind, const int32_t* key_lengths, int dtype,
                       const void* train_workspace, size_t train_workspace_bytes,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       hipEvent_t* events, int capacity, int* n_launches);

/* mha_backward_launches -- kernels mha_backward launches: 6 for
 * self-attention, 7 for cross-attention.  Host-only. */
int mha_backward_launches(int self_attention);

/*
 * ---------------------------------------------------------------------------
 * The rest of an encoder layer around the attention block: residual +
 * LayerNorm (Post-LN) and the position-wise feed-forward network.  These
 * entry points DO take biases and per-feature scale/shift vectors, because
 * their defining formulas carry them.  All vectors (gamma, beta, b1, b2) are
 * device arrays in the element type (bf16).  Only MHA_DTYPE_BF16.
 * ---------------------------------------------------------------------------
 */

/*
 * add_layernorm_forward -- Y = LayerNorm(X + F), row by row:
 *   u = X[m] + F[m];  Y[m] = gamma * (u - mean(u)) / sqrt(var(u) + eps) + beta
 * with mean and variance over the row's d features; the variance is the
 * population variance (divides by d).  Sources: hex4c59.cc "读懂 Attention Is
 * All You Need", section "Add & Norm 里究竟发生了什么？" (the sublayer output is
 * added back to its input and the sum normalised over one token's features,
 * then scaled and shifted per feature: Post-LN); devpress.csdn.net
 * "【深度学习】Transformer", section 2.3 (x + sublayer(x), then the norm).
 *
 *   X, F [M][d]   input and sublayer output;  gamma, beta [d];  Y [M][d]
 *   Y may be the same buffer as X or as F (not a partial overlap).
 *   eps finite and >= 0 (else MHA_ERR_SCALE); the pages give no value.
 *   d % 8 == 0 and d <= 4096, pointers 16-byte aligned (else
 *   MHA_ERR_UNSUPPORTED).  Sums in fp32, two-pass variance, Y rounded to bf16.
 */
int add_layernorm_forward(const void* X, const void* F, const void* gamma, const void* beta,
                          void* Y, int M, int d, float eps, int dtype, hipStream_t stream);

/*
 * ffn_workspace_bytes -- device scratch of ffn_forward: the hidden layer
 * H [M][d_ff] in the element type.  0 for invalid or unsupported sizes.
 */
size_t ffn_workspace_bytes(int M, int d_model, int d_ff, int dtype);

/*
 * ffn_forward -- position-wise feed-forward network, each row on its own:
 *   Y = max(0, X W1 + b1) W2 + b2
 * Sources: devpress.csdn.net "【深度学习】Transformer", section 2.3 (the FFN
 * formula); hex4c59.cc "读懂 Attention Is All You Need", section "前馈网络为什么
 * 放在注意力后面？" (ReLU between two linear maps, applied per position;
 * 512 -> 2048 -> 512 in the base model).
 *
 *   X [M][d_model], W1 [d_model][d_ff], b1 [d_ff], W2 [d_ff][d_model],
 *   b2 [d_model], Y [M][d_model] (must not overlap X or the workspace).
 *   workspace   >= ffn_workspace_bytes(...), 256-byte aligned, caller-owned;
 *               receives H = max(0, X W1 + b1) rounded to bf16.
 *   d_model, d_ff multiples of 8 (else MHA_ERR_UNSUPPORTED), at most 2^20
 *               (else MHA_ERR_DIM).
 * Two GEMM launches; the bias (and the ReLU) are applied to the fp32
 * accumulators before rounding.
 */
int ffn_forward(const void* X, const void* W1, const void* b1, const void* W2, const void* b2,
                void* Y, int M, int d_model, int d_ff, int dtype, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * encoder_layer_workspace_bytes -- device scratch of encoder_layer_forward:
 * the multi-head block's workspace (as mha_workspace_bytes with n_q = n_k =
 * n), then the sublayer output [B*n][d_model], x1 [B*n][d_model] and the FFN
 * hidden layer [B*n][d_ff], each 256-byte aligned.  0 for invalid sizes.
 */
size_t encoder_layer_workspace_bytes(int B, int n, int d_model, int h, int d_k, int d_v,
                                     int d_ff, int dtype);

/*
 * encoder_layer_forward -- one encoder layer, self-attention, Post-LN:
 *   x1 = LayerNorm1(X + MultiHead(X, X, X))
 *   Y  = LayerNorm2(x1 + FFN(x1))
 * Sources: hex4c59.cc "读懂 Attention Is All You Need", sections "前馈网络为什么
 * 放在注意力后面？" and "Add & Norm 里究竟发生了什么？" (two sublayers, each
 * wrapped as LayerNorm(x + Sublayer(x))); devpress.csdn.net
 * "【深度学习】Transformer", section 2.3 (the block's order); wiki.hugogu.cn
 * "Attention Is All You Need", the FFN and normalisation paragraph (the
 * encoder layer's data flow).  No dropout (inference).
 *
 *   X [B][n][d_model]; Wq, Wk, Wv, Wo as mha_forward; ln1_gamma, ln1_beta,
 *   ln2_gamma, ln2_beta, b2 [d_model]; W1, b1, W2 as ffn_forward;
 *   Y [B][n][d_model] (must not overlap X or the workspace).
 *   mask_kind / key_lengths as mha_forward (self-attention: n_q = n_k = n;
 *   the encoder uses NONE or KEY_PADDING for padded source sentences).
 *   eps as add_layernorm_forward; d_model % 8 == 0 and <= 4096.
 * Launches, in order (see encoder_layer_launches): the multi-head block
 * (mha_forward's plan, writing the sublayer output into the workspace),
 * residual + LayerNorm1, FFN first GEMM (+ b1, ReLU), FFN second GEMM (+ b2),
 * residual + LayerNorm2.
 */
int encoder_layer_forward(const void* X, const void* Wq, const void* Wk, const void* Wv,
                          const void* Wo, const void* ln1_gamma, const void* ln1_beta,
                          const void* W1, const void* b1, const void* W2, const void* b2,
                          const void* ln2_gamma, const void* ln2_beta, void* Y,
                          int B, int n, int d_model, int h, int d_k, int d_v, int d_ff,
                          float eps, int mask_kind, const int32_t* key_lengths, int dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * encoder_layer_forward_timed -- encoder_layer_forward with launch events,
 * as the other _timed variants (events[2i], events[2i+1] around launch i).
 */
int encoder_layer_forward_timed(const void* X, const void* Wq, const void* Wk, const void* Wv,
                                const void* Wo, const void* ln1_gamma, const void* ln1_beta,
                                const void* W1, const void* b1, const void* W2, const void* b2,
                                const void* ln2_gamma, const void* ln2_beta, void* Y,
                                int B, int n, int d_model, int h, int d_k, int d_v, int d_ff,
                                float eps, int mask_kind, const int32_t* key_lengths, int dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* events, int capacity, int* n_launches);

/*
 * encoder_layer_launches -- kernels encoder_layer_forward launches for
 * sequences of n positions and width d_model: the block's (2 on the fused
 * short-sequence plan, else 3) plus 4.  Host-only.  MHA_ERR_DIM for
 * non-positive sizes.
 */
int encoder_layer_launches(int n, int d_model);

/*
 * embed_positional_forward -- the model's input: token embedding scaled by
 * sqrt(d_model) plus the sinusoidal positional encoding, fused:
 *   out[b][p][j] = E[tokens[b][p]][j] * sqrt(d_model) + PE(pos0 + p, j)
 *   PE(pos, 2i) = sin(pos / 10000^(2i/d_model)), PE(pos, 2i+1) = cos(same)
 * Sources: devpress.csdn.net "【深度学习】Transformer", section 4 (equation
 * (4.1), Table 4.1, the worked example scaling the input by sqrt(d_model)
 * before the encoding is added); hex4c59.cc "读懂 Attention Is All You Need",
 * section "没有循环，模型怎样知道词序？" (embedding row looked up by token id,
 * times sqrt(d_model), plus the encoding of the same width).
 *
 *   tokens  DEVICE int32 [B][n], token ids; an id outside [0, vocab) gives
 *           a row of NaN (nothing is read for it) -- ids are device data and
 *           are not checked on the host.
 *   E       [vocab][d_model] embedding table;  out [B][n][d_model]
 *   pos0    position of each sequence's first token (>= 0; 0 for whole
 *           sentences, the step index when one new token is embedded during
 *           incremental decoding); positions are pos0 .. pos0 + n - 1.
 *   dtype   MHA_DTYPE_BF16 or MHA_DTYPE_F32 (E and out).
 *   d_model % 8 == 0 (else MHA_ERR_UNSUPPORTED); B <= 524280.
 * Frequencies and angles are formed in double precision and reduced to one
 * turn there; sine and cosine of the reduced angle are single precision
 * (error ~2e-7 up to positions of 2^24); the sum is formed in fp32 and
 * rounded once to the output type.  One launch.
 */
int embed_positional_forward(const int32_t* tokens, const void* E, void* out, int B, int n,
                             int vocab, int d_model, int pos0, int dtype, hipStream_t stream);

/* embed_positional_forward with launch events (one launch), as the other
 * _timed variants. */
int embed_positional_forward_timed(const int32_t* tokens, const void* E, void* out, int B, int n,
                                   int vocab, int d_model, int pos0, int dtype, hipStream_t stream,
                                   hipEvent_t* events, int capacity, int* n_launches);

/* Text of a status code (static storage; never NULL). */
const char* mha_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H */
