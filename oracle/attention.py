"""Matrix-form oracle: numpy, float64, one function per step of the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

Every array is float64.  Callers upcast the exact values the GPU received
(bf16 or fp32 values convert to float64 without rounding).  Nothing here is
blocked, fused or reordered: the n_q x n_k score and weight matrices are
materialised per head exactly as the formula reads.

Layouts (row-major, batch first):
  X_q [B][n_q][d_model], X_kv [B][n_k][d_model]
  Wq, Wk [d_model][h*d_k], Wv [d_model][h*d_v], Wo [h*d_v][d_model]
  Q [B][h][n_q][d_k], K [B][h][n_k][d_k], V [B][h][n_k][d_v]
  O [B][h][n_q][d_v], Y [B][n_q][d_model]
"""

import math

import numpy as np

# Mask kinds.  Bit 0: causal (decoder self-attention); bit 1: key padding.
MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEY_PADDING = 2
MASK_CAUSAL_KEY_PADDING = 3


def _f64(a):
    a = np.asarray(a)
    if a.dtype != np.float64:
        raise TypeError("oracle works on float64 arrays (upcast exactly first)")
    return a


def _check_mask(mask_kind, n_q, n_k, key_lengths, B):
    if mask_kind not in (MASK_NONE, MASK_CAUSAL, MASK_KEY_PADDING, MASK_CAUSAL_KEY_PADDING):
        raise ValueError(f"unknown mask kind {mask_kind}")
    if mask_kind & MASK_CAUSAL and n_q != n_k:
        # Causal masking is defined for decoder self-attention, where queries
        # and keys index the same positions; it has no meaning otherwise.
        raise ValueError("causal mask needs n_q == n_k")
    if mask_kind & MASK_KEY_PADDING:
        if key_lengths is None:
            raise ValueError("key padding needs key_lengths")
        kl = np.asarray(key_lengths)
        if kl.shape != (B,):
            raise ValueError("key_lengths must have one entry per batch")
        if np.any(kl < 1) or np.any(kl > n_k):
            raise ValueError("key lengths must lie in [1, n_k]")


def project(X, W):
    """Linear input/output projection X.W (no bias).

    hex4c59.cc "读懂 Attention Is All You Need", section "Q、K、V 是三种计算角色":
    each position's row is multiplied by a learned d_model x d_k (or d_v)
    matrix; devpress.csdn.net "【深度学习】Transformer", section 2.1,
    equations (2.1)-(2.3): Q = X W^Q, K = X W^K, V = X W^V.
    """
    X = _f64(X)
    W = _f64(W)
    return X @ W


def split_heads(Y, h):
    """[B][n][h*d] -> [B][h][n][d]; head i owns the contiguous column block
    [i*d, (i+1)*d) of the stacked projection.

    The stacked projection [W_1 ... W_h] gives each head its own W_i
    (hex4c59.cc, section "多头注意力让一次读取有多组投影"); the block
    assignment is the one the pages' reshapes use (wiki.hugogu.cn listing,
    MultiHeadAttention.forward; devpress.csdn.net section 2.2, head split).
    """
    B, n, hd = Y.shape
    if hd % h:
        raise ValueError("width not divisible by head count")
    d = hd // h
    return Y.reshape(B, n, h, d).transpose(0, 2, 1, 3)


def concat_heads(O):
    """[B][h][n][d] -> [B][n][h*d]: Concat(head_1..head_h) along features
    (hex4c59.cc, section "多头注意力让一次读取有多组投影"; devpress.csdn.net
    section 2.2, the MultiHead formula)."""
    B, h, n, d = O.shape
    return O.transpose(0, 2, 1, 3).reshape(B, n, h * d)


def scaled_scores(Q, K, scale):
    """S = Q K^T * scale over the last two axes.

    Row r of S belongs to query r, column c to key c (hex4c59.cc, section
    "把所有位置合并，就是那条核心公式"); the scale is 1/sqrt(d_k) in the
    method (section "为什么要按键的维度缩放？"; research-heat.pages.dev
    "做法", section "点积随维度增大，因而除以根号"; devpress.csdn.net
    equation (2.4)).  The caller passes the scale explicitly.
    """
    Q = _f64(Q)
    K = _f64(K)
    return (Q @ np.swapaxes(K, -1, -2)) * float(scale)


def additive_mask(n_q, n_k, mask_kind, key_length=None):
    """The additive 0 / -inf mask for one (batch, head), shape [n_q][n_k].

    Causal: entry (r, c) is -inf when c > r, 0 otherwise -- the diagonal stays
    visible (hex4c59.cc, section "掩码必须在 softmax 之前生效": position t
    reads inputs 1..t; devpress.csdn.net section 3.1 prints the 5x5 pattern;
    wiki.hugogu.cn masked self-attention paragraph: upper triangle -inf).
    Key padding: entry (r, c) is -inf when c >= key_length (hex4c59.cc, same
    section, padding mask paragraph).  Both: the union.
    """
    M = np.zeros((n_q, n_k), dtype=np.float64)
    r = np.arange(n_q)[:, None]
    c = np.arange(n_k)[None, :]
    if mask_kind & MASK_CAUSAL:
        M[np.broadcast_to(c > r, M.shape)] = -np.inf
    if mask_kind & MASK_KEY_PADDING:
        M[np.broadcast_to(c >= key_length, M.shape)] = -np.inf
    return M


def softmax_rows(S):
    """Row softmax over the last axis, computed stably by subtracting the row
    maximum (mathematically identical to the unshifted form; hex4c59.cc,
    section "用几十行代码核对刚才的数值").  exp(-inf) = 0, so masked entries
    get weight exactly 0 (section "掩码必须在 softmax 之前生效").

    Every row must hold at least one finite entry (an all-masked row is 0/0;
    the library's preconditions exclude it).
    """
    S = _f64(S)
    m = np.max(S, axis=-1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("softmax row with no visible entry")
    e = np.exp(S - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_weights(Q, K, scale, mask_kind=MASK_NONE, key_lengths=None):
    """P = softmax(Q K^T * scale + M) per (batch, head): [B][h][n_q][n_k].

    The mask is added to the scores before the softmax (hex4c59.cc, section
    "掩码必须在 softmax 之前生效"; devpress.csdn.net section 3.1 flow:
    scores, then attn_mask + scores, then softmax)."""
    Q = _f64(Q)
    K = _f64(K)
    B, h, n_q, _ = Q.shape
    n_k = K.shape[2]
    _check_mask(mask_kind, n_q, n_k, key_lengths, B)
    S = scaled_scores(Q, K, scale)
    for b in range(B):
        L = None if key_lengths is None else int(key_lengths[b])
        S[b] = S[b] + additive_mask(n_q, n_k, mask_kind, L)[None]
    return softmax_rows(S)


def sdpa_ref(Q, K, V, scale, mask_kind=MASK_NONE, key_lengths=None):
    """Scaled dot-product attention softmax(Q K^T * scale + M) V, per
    (batch, head).  Q [B][h][n_q][d_k], K [B][h][n_k][d_k], V [B][h][n_k][d_v]
    -> O [B][h][n_q][d_v].

    devpress.csdn.net section 2.1 equation (2.4); hex4c59.cc section
    "六步算完一行注意力" (weights multiply the value rows, then sum).
    Parity: pinned (printed values, closed forms, invariants, brute force,
    library cross-check; see tests/test_oracle.py)."""
    V = _f64(V)
    P = attention_weights(Q, K, scale, mask_kind, key_lengths)
    return P @ V


def sdpa_ref_rows(Q, K, V, scale, mask_kind, key_lengths, idx):
    """The same definition evaluated for selected query rows only.

    idx: integer array [R][3] of (batch, head, query).  Returns [R][d_v].
    Each row is computed on its own: scores of that query against every key
    of its (batch, head), the mask row, the row softmax, the weighted sum of
    value rows.  Used to check sampled outputs of shapes too large to
    materialise whole."""
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    B, h, n_q, _ = Q.shape
    n_k = K.shape[2]
    _check_mask(mask_kind, n_q, n_k, key_lengths, B)
    idx = np.asarray(idx, dtype=np.int64).reshape(-1, 3)
    out = np.empty((idx.shape[0], V.shape[3]), dtype=np.float64)
    for t, (b, hh, q) in enumerate(idx):
        s = (K[b, hh] @ Q[b, hh, q]) * float(scale)
        L = None if key_lengths is None else int(key_lengths[b])
        s = s + additive_mask(n_q, n_k, mask_kind, L)[q]
        p = softmax_rows(s[None, :])[0]
        out[t] = p @ V[b, hh]
    return out


def mha_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, mask_kind=MASK_NONE, key_lengths=None,
            return_intermediates=False):
    """Multi-head attention block: Concat(head_1..head_h) W^O with
    head_i = Attention(X_q W_i^Q, X_kv W_i^K, X_kv W_i^V), scale 1/sqrt(d_k).

    devpress.csdn.net section 2.2 (MultiHead formula; W_i^Q, W_i^K in
    R^{d x d_k}, W_i^V in R^{d x d_v}, W^O in R^{h d_v x d}); hex4c59.cc
    section "多头注意力让一次读取有多组投影".  Self-attention passes the same
    array as X_q and X_kv; cross-attention takes queries from the decoder
    side and keys/values from the encoder output, so n_q may differ from n_k
    (hex4c59.cc, section "解码器有两种读取：看前缀，以及看源句";
    devpress.csdn.net section 3.2).  No biases: the formula has none.
    Parity: pinned by composition of pinned steps, brute force on tiny
    inputs, and the block identities in tests/test_oracle.py."""
    X_q = _f64(X_q)
    X_kv = _f64(X_kv)
    hdk = Wq.shape[1]
    hdv = Wv.shape[1]
    if hdk % h or hdv % h or Wk.shape[1] != hdk or Wo.shape[0] != hdv:
        raise ValueError("inconsistent projection shapes")
    d_k = hdk // h
    Q = split_heads(project(X_q, Wq), h)
    K = split_heads(project(X_kv, Wk), h)
    V = split_heads(project(X_kv, Wv), h)
    O = sdpa_ref(Q, K, V, 1.0 / math.sqrt(d_k), mask_kind, key_lengths)
    C = concat_heads(O)
    Y = project(C, Wo)
    if return_intermediates:
        return Y, dict(Q=Q, K=K, V=V, O=O, concat=C)
    return Y
