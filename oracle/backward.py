"""Gradients of scaled dot-product attention (the backward pass) and the
row log-sum-exp a forward pass keeps for it.  numpy, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

Sources: hex4c59.cc, "读懂 Attention Is All You Need", sections "训练能并行，
不意味着一次生成整句话" (in training all target positions are computed, and
their losses back-propagated, at once) and "参数是怎样学出来的？" (the loss is
turned into gradients that flow back along the computation's steps to every
part).  The pages give no formulas for this pass; what is computed here is
the gradient of the forward definition, softmax(Q K^T * scale + M) V
(devpress.csdn.net "【深度学习】Transformer", section 2.1, equation (2.4)),
taken through its steps in reverse order:

    S = Q K^T * scale + M      ->  dQ = scale * dS K,  dK = scale * dS^T Q
    P = softmax over each row  ->  dS = P * (dP - rowsum(P * dP))
    O = P V                    ->  dP = dO V^T,        dV = P^T dO

(M is constant; a masked entry has P = 0, hence dS = 0.)  rowsum(P * dP)
equals rowsum(dO * O), which is how a kernel can form it from its inputs.

Parity: pinned by central finite differences of the loss sum(dO * O) in
float64, exact invariants (the key gradients of each sequence sum to zero;
keys hidden from every query get zero gradients) and the uniform-weight
closed form; see tests/oracle_pins.py.
"""

import numpy as np

from .attention import _f64, attention_weights, scaled_scores, additive_mask, _check_mask


def row_logsumexp(Q, K, scale, mask_kind=0, key_lengths=None):
    """ln(sum over visible keys j of exp(scale * q_i . k_j)) for every query
    row: [B][h][n_q].  With it, P_ij = exp(scale q_i . k_j - lse_i).
    Parity: pinned (brute force with math.fsum; rows of exp(S - lse) sum to 1)."""
    Q = _f64(Q)
    K = _f64(K)
    B, h, n_q, _ = Q.shape
    n_k = K.shape[2]
    _check_mask(mask_kind, n_q, n_k, key_lengths, B)
    S = scaled_scores(Q, K, scale)
    for b in range(B):
        L = None if key_lengths is None else int(key_lengths[b])
        S[b] = S[b] + additive_mask(n_q, n_k, mask_kind, L)[None]
    m = S.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(S - m).sum(axis=-1, keepdims=True)))[..., 0]


def sdpa_backward_ref(Q, K, V, dO, scale, mask_kind=0, key_lengths=None):
    """(dQ, dK, dV) of O = softmax(Q K^T * scale + M) V for the upstream
    gradient dO [B][h][n_q][d_v].  Shapes as sdpa_ref.
    Parity: pinned by finite differences and invariants."""
    Q, K, V, dO = (_f64(t) for t in (Q, K, V, dO))
    P = attention_weights(Q, K, scale, mask_kind, key_lengths)
    # O = P V
    dV = np.swapaxes(P, -1, -2) @ dO
    dP = dO @ np.swapaxes(V, -1, -2)
    # P = softmax(S) along each row
    dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
    # S = Q K^T * scale + M
    dQ = scale * (dS @ K)
    dK = scale * (np.swapaxes(dS, -1, -2) @ Q)
    return dQ, dK, dV


def mha_backward_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, dY, mask_kind=0, key_lengths=None):
    """Gradients of the multi-head block Y = Concat(head_1..head_h) W^O,
    head_i = Attention(X_q W_i^Q, X_kv W_i^K, X_kv W_i^V) (devpress.csdn.net
    section 2.2), for the upstream gradient dY [B][n_q][d_model], taken
    through the block's steps in reverse:

        Y = C W^O            ->  dC = dY W^O^T,   dW^O = sum over rows C^T dY
        C = concat(heads)    ->  dO = split(dC)
        O = attention        ->  dQ, dK, dV (sdpa_backward_ref)
        Q = X_q W^Q, ...     ->  dW^Q = X_q^T dQ_c,  dX_q = dQ_c W^Q^T
                                 dX_kv = dK_c W^K^T + dV_c W^V^T, ...

    (_c: heads concatenated back into [rows][h*d]).  Returns dX_q, dX_kv,
    dWq, dWk, dWv, dWo; for self-attention (X_kv the same array as X_q) the
    gradient with respect to the shared input is dX_q + dX_kv.
    Parity: pinned by finite differences of sum(dY * Y)."""
    from .attention import concat_heads, mha_ref, split_heads
    X_q, X_kv, Wq, Wk, Wv, Wo, dY = (_f64(t) for t in (X_q, X_kv, Wq, Wk, Wv, Wo, dY))
    _, it = mha_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, mask_kind, key_lengths, return_intermediates=True)
    d_k = Wq.shape[1] // h
    C = it["concat"]
    dWo = np.einsum("bni,bnj->ij", C, dY)
    dC = dY @ Wo.T
    dO = split_heads(dC, h)
    dQ, dK, dV = sdpa_backward_ref(it["Q"], it["K"], it["V"], dO, 1.0 / np.sqrt(d_k), mask_kind,
                                   key_lengths)
    dQc, dKc, dVc = concat_heads(dQ), concat_heads(dK), concat_heads(dV)
    dWq = np.einsum("bni,bnj->ij", X_q, dQc)
    dWk = np.einsum("bni,bnj->ij", X_kv, dKc)
    dWv = np.einsum("bni,bnj->ij", X_kv, dVc)
    dX_q = dQc @ Wq.T
    dX_kv = dKc @ Wk.T + dVc @ Wv.T
    return dX_q, dX_kv, dWq, dWk, dWv, dWo
