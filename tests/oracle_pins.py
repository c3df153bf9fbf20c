"""Pins for the attention oracle: checks against what the pages and the
mathematics fix, independent of the oracle's own formulas.

Each ``check_*`` function takes the implementation under test (the oracle, or
a mutant with one planted mistake) and raises AssertionError on a violation.
``tests/test_oracle.py`` runs them on the oracle; ``tests/test_oracle_mutants.py``
runs them on mutants and requires each mutant to fail at least one.

Implementation interface (a module or a SimpleNamespace):
  softmax_rows(S) -> P
  additive_mask(n_q, n_k, mask_kind, key_length) -> [n_q][n_k] of 0 / -inf
  sdpa_ref(Q, K, V, scale, mask_kind, key_lengths) -> O   (float64, [B][h][n][d])
  mha_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, mask_kind, key_lengths) -> Y
"""

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

NONE, CAUSAL, PAD, BOTH = 0, 1, 2, 3


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _weights(impl, Q, K, scale, mask_kind=NONE, key_lengths=None):
    """Attention weights observed through the public sdpa call: with V the
    n_k x n_k identity, O = P."""
    B, h, _, _ = Q.shape
    n_k = K.shape[2]
    V = np.broadcast_to(np.eye(n_k), (B, h, n_k, n_k)).copy()
    return impl.sdpa_ref(Q, K, V, scale, mask_kind, key_lengths)


def _visible(n_q, n_k, mask_kind, L):
    """Visibility by integer comparison (its own definition, not the oracle's)."""
    vis = np.ones((n_q, n_k), dtype=bool)
    for r in range(n_q):
        for c in range(n_k):
            if mask_kind & CAUSAL and c > r:
                vis[r, c] = False
            if mask_kind & PAD and c >= L:
                vis[r, c] = False
    return vis


# ---------------------------------------------------------------- printed values

def check_softmax_printed(impl):
    """Printed: softmax([1,2,3]) ~ [0.090, 0.245, 0.665]; [10,20,30] puts
    weight close to 1 on the last entry (hex4c59.cc, section
    "为什么要按键的维度缩放？")."""
    g = _golden("softmax_printed.json")
    c0, c1 = g["cases"]
    p = impl.softmax_rows(np.array([c0["scores"]], dtype=np.float64))[0]
    assert np.array_equal(np.round(p, c0["decimals"]), np.array(c0["printed_weights"])), p
    p = impl.softmax_rows(np.array([c1["scores"]], dtype=np.float64))[0]
    assert p[-1] >= c1["min_last_weight"] and p[-1] < 1.0, p


def check_worked_example(impl):
    """Printed weights [0.4011, 0.1978, 0.4011] and output [1.6044, 1.1978]
    for one query over three keys, d_k = 2 (hex4c59.cc, sections
    "六步算完一行注意力" and "用几十行代码核对刚才的数值"), on a derived
    instance consistent with them, plus the closed form of the weights."""
    g = _golden("worked_example_one_row.json")
    scale = 1.0 / math.sqrt(g["d_k"])
    Q = np.array(g["q"], dtype=np.float64).reshape(1, 1, 1, 2)
    K = np.array(g["K"], dtype=np.float64).reshape(1, 1, 3, 2)
    V = np.array(g["V"], dtype=np.float64).reshape(1, 1, 3, 2)
    w = _weights(impl, Q, K, scale)[0, 0, 0]
    o = impl.sdpa_ref(Q, K, V, scale, NONE, None)[0, 0, 0]
    assert np.array_equal(np.round(w, g["decimals"]), np.array(g["printed_weights"])), w
    assert np.array_equal(np.round(o, g["decimals"]), np.array(g["printed_output"])), o
    a = math.exp(1.0 / math.sqrt(2.0))
    closed = np.array([a, 1.0, a]) / (2.0 * a + 1.0)
    assert np.allclose(w, closed, rtol=0, atol=1e-14), (w, closed)


def check_causal_pattern(impl):
    """The printed 5x5 causal mask (devpress.csdn.net, section 3.1)."""
    g = _golden("causal_mask_5x5.json")
    want = np.array([[0.0 if x == "0" else -np.inf for x in row] for row in g["printed"]])
    got = impl.additive_mask(g["n"], g["n"], CAUSAL, None)
    assert np.array_equal(got, want), got


# ---------------------------------------------------------------- invariants

def check_rows_are_distributions(impl):
    """Weights are non-negative, each row sums to 1, masked entries are
    exactly 0 (hex4c59.cc, section "六步算完一行注意力": softmax gives
    non-negative weights summing to 1; section "掩码必须在 softmax 之前生效":
    future weight becomes 0)."""
    r = _rng(1)
    for kind, n_q, n_k in ((NONE, 5, 7), (CAUSAL, 6, 6), (PAD, 4, 9), (BOTH, 8, 8)):
        B, h, d = 2, 2, 5
        Q = r.standard_normal((B, h, n_q, d)) * 2
        K = r.standard_normal((B, h, n_k, d))
        kl = np.array([3, n_k]) if kind & PAD else None
        P = _weights(impl, Q, K, 1 / math.sqrt(d), kind, kl)
        assert np.all(P >= 0)
        assert np.allclose(P.sum(-1), 1.0, atol=1e-13)
        for b in range(B):
            vis = _visible(n_q, n_k, kind, None if kl is None else kl[b])
            assert np.all(P[b][:, ~vis] == 0.0)
            assert np.all(P[b][:, vis] > 0.0)


def check_convex_combination(impl):
    """Each output row is a convex combination of the visible value rows
    (hex4c59.cc, section "六步算完一行注意力"), so every coordinate lies in
    [min, max] of that coordinate over the visible rows."""
    r = _rng(2)
    for kind in (NONE, CAUSAL, PAD, BOTH):
        B, h, n, d = 2, 3, 9, 4
        Q = r.standard_normal((B, h, n, d)) * 3
        K = r.standard_normal((B, h, n, d))
        V = r.standard_normal((B, h, n, d)) * 5
        kl = np.array([2, 7]) if kind & PAD else None
        O = impl.sdpa_ref(Q, K, V, 0.5, kind, kl)
        for b in range(B):
            vis = _visible(n, n, kind, None if kl is None else kl[b])
            for hh in range(h):
                for q in range(n):
                    rows = V[b, hh][vis[q]]
                    assert np.all(O[b, hh, q] >= rows.min(0) - 1e-12)
                    assert np.all(O[b, hh, q] <= rows.max(0) + 1e-12)


def check_permutation_equivariance(impl):
    """Unmasked attention commutes with a permutation of the positions:
    Attn(PQ, PK, PV) = P Attn(Q, K, V) (hex4c59.cc, section
    "没有循环，模型怎样知道词序？").  For cross-attention, permuting K and V
    rows jointly changes nothing."""
    r = _rng(3)
    B, h, n, d = 1, 2, 7, 6
    Q = r.standard_normal((B, h, n, d))
    K = r.standard_normal((B, h, n, d))
    V = r.standard_normal((B, h, n, 5))
    perm = r.permutation(n)
    O = impl.sdpa_ref(Q, K, V, 0.4, NONE, None)
    Op = impl.sdpa_ref(Q[:, :, perm], K[:, :, perm], V[:, :, perm], 0.4, NONE, None)
    assert np.allclose(Op, O[:, :, perm], atol=1e-13)
    K2 = r.standard_normal((B, h, 11, d))
    V2 = r.standard_normal((B, h, 11, 5))
    perm2 = r.permutation(11)
    O2 = impl.sdpa_ref(Q, K2, V2, 0.4, NONE, None)
    O2p = impl.sdpa_ref(Q, K2[:, :, perm2], V2[:, :, perm2], 0.4, NONE, None)
    assert np.allclose(O2, O2p, atol=1e-13)


def check_causal_row0_and_last(impl):
    """Causal: query 0 sees only key 0, so output row 0 is value row 0
    exactly; the last query sees every key, so its row equals the unmasked
    result (hex4c59.cc, section "掩码必须在 softmax 之前生效")."""
    r = _rng(4)
    B, h, n, d = 2, 2, 6, 4
    Q, K, V = (r.standard_normal((B, h, n, d)) for _ in range(3))
    O = impl.sdpa_ref(Q, K, V, 0.5, CAUSAL, None)
    assert np.array_equal(O[:, :, 0], V[:, :, 0])
    U = impl.sdpa_ref(Q, K, V, 0.5, NONE, None)
    assert np.allclose(O[:, :, -1], U[:, :, -1], atol=1e-14)


def check_zero_query_means(impl):
    """Q = 0 makes every visible score equal, so the weights are uniform and
    the output is the mean of the visible value rows: all rows unmasked,
    prefix means under the causal mask, the first L_b rows under padding
    (closed form)."""
    r = _rng(5)
    B, h, n, d = 2, 1, 8, 3
    Q = np.zeros((B, h, n, d))
    K = r.standard_normal((B, h, n, d))
    V = r.standard_normal((B, h, n, d))
    kl = np.array([3, 8])
    for kind in (NONE, CAUSAL, PAD, BOTH):
        O = impl.sdpa_ref(Q, K, V, 1.0, kind, kl if kind & PAD else None)
        for b in range(B):
            vis = _visible(n, n, kind, kl[b])
            for q in range(n):
                assert np.allclose(O[b, 0, q], V[b, 0][vis[q]].mean(0), atol=1e-14)


def check_identical_keys_uniform(impl):
    """Identical key rows give identical scores, hence uniform weights for any
    query (closed form)."""
    r = _rng(6)
    B, h, n, d = 1, 1, 5, 4
    Q = r.standard_normal((B, h, 3, d)) * 4
    K = np.broadcast_to(r.standard_normal((1, 1, 1, d)), (B, h, n, d)).copy()
    P = _weights(impl, Q, K, 0.5)
    assert np.allclose(P, 1.0 / n, atol=1e-15)


def check_future_perturbation(impl):
    """Causal: changing key/value rows j > i leaves output row i unchanged,
    bit for bit (future positions get weight exactly 0)."""
    r = _rng(7)
    B, h, n, d = 1, 2, 9, 4
    Q, K, V = (r.standard_normal((B, h, n, d)) for _ in range(3))
    O = impl.sdpa_ref(Q, K, V, 0.5, CAUSAL, None)
    for i in range(n - 1):
        K2, V2 = K.copy(), V.copy()
        K2[:, :, i + 1:] = r.standard_normal(K2[:, :, i + 1:].shape) * 10
        V2[:, :, i + 1:] = r.standard_normal(V2[:, :, i + 1:].shape) * 10
        O2 = impl.sdpa_ref(Q, K2, V2, 0.5, CAUSAL, None)
        assert np.array_equal(O2[:, :, : i + 1], O[:, :, : i + 1])


def check_padding_truncation(impl):
    """Key padding with length L equals unmasked attention over K[:L], V[:L]
    (the plain formula on the valid keys), and changing padded rows changes
    nothing."""
    r = _rng(8)
    B, h, n_q, n_k, d = 3, 2, 5, 9, 4
    Q = r.standard_normal((B, h, n_q, d))
    K = r.standard_normal((B, h, n_k, d))
    V = r.standard_normal((B, h, n_k, d))
    kl = np.array([1, 4, 9])
    O = impl.sdpa_ref(Q, K, V, 0.5, PAD, kl)
    for b in range(B):
        L = kl[b]
        Ob = impl.sdpa_ref(Q[b:b + 1], K[b:b + 1, :, :L], V[b:b + 1, :, :L], 0.5, NONE, None)
        assert np.allclose(O[b:b + 1], Ob, atol=1e-14)
    K2, V2 = K.copy(), V.copy()
    for b in range(B):
        K2[b, :, kl[b]:] = 1e3
        V2[b, :, kl[b]:] = -1e3
    assert np.array_equal(impl.sdpa_ref(Q, K2, V2, 0.5, PAD, kl), O)


def check_saturation(impl):
    """Scores of magnitude ~1e3 must neither overflow nor give NaN: the row
    softmax is computed stably (hex4c59.cc, section "用几十行代码核对刚才的数值");
    the largest score takes all the weight."""
    B, h, n, d = 1, 1, 4, 2
    Q = np.array([[[[30.0, 0.0]] * n]])
    K = np.array([[[[100.0, 0.0], [99.0, 0.0], [-50.0, 0.0], [98.0, 0.0]]]])
    V = np.array([[[[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]]]])
    O = impl.sdpa_ref(Q, K, V, 1.0, NONE, None)
    assert np.all(np.isfinite(O))
    assert np.allclose(O[0, 0, 0], V[0, 0, 0], atol=1e-12)


def check_scale_statistics(impl):
    """For i.i.d. zero-mean unit-variance q and k components the scaled score
    q.k / sqrt(d_k) has variance 1 (hex4c59.cc, section
    "为什么要按键的维度缩放？"; devpress.csdn.net, section 2.1 derivation).
    Scores are recovered from the weights: log P_j - log P_0 = s_j - s_0, whose
    variance is 2 Var(s)."""
    r = _rng(9)
    d, n, rows = 64, 16, 512
    Q = r.standard_normal((1, 1, rows, d))
    K = r.standard_normal((1, 1, n, d))
    P = _weights(impl, Q, K, 1.0 / math.sqrt(d))[0, 0]
    diff = np.log(P[:, 1:]) - np.log(P[:, :1])
    v = diff.var() / 2.0
    assert 0.85 < v < 1.15, v


# ---------------------------------------------------------------- brute force / library

def _nested(a):
    return a.tolist()


def check_bruteforce_sdpa(impl):
    """Matrix form against the pure-Python loops on tiny shapes: n_q != n_k,
    causal, padding, both, h > 1, d_v != d_k."""
    from oracle.bruteforce import attention_bruteforce
    r = _rng(10)
    for kind, n_q, n_k, d_k, d_v in ((NONE, 3, 5, 4, 2), (CAUSAL, 4, 4, 3, 5), (PAD, 2, 6, 2, 3),
                                     (BOTH, 5, 5, 4, 4), (NONE, 1, 1, 3, 3)):
        B, h = 2, 2
        Q = r.standard_normal((B, h, n_q, d_k))
        K = r.standard_normal((B, h, n_k, d_k))
        V = r.standard_normal((B, h, n_k, d_v))
        kl = [max(1, n_k - 2), n_k] if kind & PAD else None
        got = impl.sdpa_ref(Q, K, V, 0.7, kind, None if kl is None else np.array(kl))
        want = np.array(attention_bruteforce(_nested(Q), _nested(K), _nested(V), 0.7, kind, kl))
        assert np.allclose(got, want, rtol=0, atol=1e-13), np.abs(got - want).max()


def check_library_sdpa(impl):
    """Cross-check against torch.nn.functional.scaled_dot_product_attention in
    float64 on the CPU (a library routine computing the same definition; its
    output only is used)."""
    import torch
    import torch.nn.functional as F
    r = _rng(11)
    B, h, n_q, n_k, d = 2, 3, 17, 23, 8
    Q = r.standard_normal((B, h, n_q, d))
    K = r.standard_normal((B, h, n_k, d))
    V = r.standard_normal((B, h, n_k, d))
    got = impl.sdpa_ref(Q, K, V, 0.3, NONE, None)
    want = F.scaled_dot_product_attention(torch.from_numpy(Q), torch.from_numpy(K),
                                          torch.from_numpy(V), scale=0.3).numpy()
    assert np.allclose(got, want, atol=1e-12)
    Kc, Vc = K[:, :, :n_q], V[:, :, :n_q]
    got = impl.sdpa_ref(Q, Kc, Vc, 0.3, CAUSAL, None)
    want = F.scaled_dot_product_attention(torch.from_numpy(Q), torch.from_numpy(Kc.copy()),
                                          torch.from_numpy(Vc.copy()), is_causal=True,
                                          scale=0.3).numpy()
    assert np.allclose(got, want, atol=1e-12)
    kl = np.array([5, 23])
    keep = np.zeros((B, 1, 1, n_k), dtype=bool)
    for b in range(B):
        keep[b, :, :, : kl[b]] = True
    got = impl.sdpa_ref(Q, K, V, 0.3, PAD, kl)
    want = F.scaled_dot_product_attention(torch.from_numpy(Q), torch.from_numpy(K),
                                          torch.from_numpy(V), attn_mask=torch.from_numpy(keep),
                                          scale=0.3).numpy()
    assert np.allclose(got, want, atol=1e-12)


# ---------------------------------------------------------------- multi-head block

def _mha_inputs(r, B, n_q, n_k, dm, h, d_k, d_v):
    X_q = r.standard_normal((B, n_q, dm))
    X_kv = r.standard_normal((B, n_k, dm))
    Wq = r.standard_normal((dm, h * d_k)) / math.sqrt(dm)
    Wk = r.standard_normal((dm, h * d_k)) / math.sqrt(dm)
    Wv = r.standard_normal((dm, h * d_v)) / math.sqrt(dm)
    Wo = r.standard_normal((h * d_v, dm)) / math.sqrt(h * d_v)
    return X_q, X_kv, Wq, Wk, Wv, Wo


def check_bruteforce_mha(impl):
    """Multi-head block against the loop version on tiny shapes: self
    (same array), causal, cross with padding and d_v != d_k."""
    from oracle.bruteforce import mha_bruteforce
    r = _rng(12)
    for kind, n_q, n_k, self_attn in ((NONE, 4, 4, True), (CAUSAL, 5, 5, True), (PAD, 3, 6, False)):
        B, dm, h, d_k, d_v = 2, 6, 2, 3, 4
        X_q, X_kv, Wq, Wk, Wv, Wo = _mha_inputs(r, B, n_q, n_k, dm, h, d_k, d_v)
        if self_attn:
            X_kv = X_q
        kl = [2, n_k] if kind & PAD else None
        got = impl.mha_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, kind, None if kl is None else np.array(kl))
        want = np.array(mha_bruteforce(_nested(X_q), _nested(X_kv), _nested(Wq), _nested(Wk),
                                       _nested(Wv), _nested(Wo), h, kind, kl))
        assert np.allclose(got, want, rtol=0, atol=1e-12), np.abs(got - want).max()


def check_mha_head_blocks(impl):
    """Head i owns column block i of W^Q, W^K, W^V and row block i of W^O
    (head split by contiguous blocks, concat in head order; hex4c59.cc,
    section "多头注意力让一次读取有多组投影"; devpress.csdn.net section 2.2).
    With W^V zero outside block i only head i carries values, so: zeroing
    row block i of W^O gives Y = 0, changing any other row block of W^O or
    any other column block of W^Q/W^K changes nothing, and changing block i
    of W^Q changes Y."""
    r = _rng(13)
    B, n, dm, h, d = 2, 5, 8, 4, 2
    X, _, Wq, Wk, Wv, Wo = _mha_inputs(r, B, n, n, dm, h, d, d)
    for i in (0, 2):
        Wv_i = np.zeros_like(Wv)
        Wv_i[:, i * d:(i + 1) * d] = Wv[:, i * d:(i + 1) * d]
        Y = impl.mha_ref(X, X, Wq, Wk, Wv_i, Wo, h, NONE, None)
        assert np.abs(Y).max() > 1e-3
        Wo0 = Wo.copy()
        Wo0[i * d:(i + 1) * d] = 0
        assert np.abs(impl.mha_ref(X, X, Wq, Wk, Wv_i, Wo0, h, NONE, None)).max() < 1e-14
        for j in range(h):
            if j == i:
                continue
            Wo2 = Wo.copy()
            Wo2[j * d:(j + 1) * d] = r.standard_normal((d, dm))
            Wq2 = Wq.copy()
            Wq2[:, j * d:(j + 1) * d] = r.standard_normal((dm, d))
            Wk2 = Wk.copy()
            Wk2[:, j * d:(j + 1) * d] = r.standard_normal((dm, d))
            assert np.allclose(impl.mha_ref(X, X, Wq2, Wk2, Wv_i, Wo2, h, NONE, None), Y,
                               atol=1e-13)
        Wq3 = Wq.copy()
        Wq3[:, i * d:(i + 1) * d] *= 3.0
        assert np.abs(impl.mha_ref(X, X, Wq3, Wk, Wv_i, Wo, h, NONE, None) - Y).max() > 1e-6


def check_mha_identity_reduction(impl):
    """h = 1 with identity projections reduces the block to bare attention
    SDPA(X, X, X) with scale 1/sqrt(d_model) (special case of the formula)."""
    r = _rng(14)
    B, n, dm = 2, 6, 5
    X = r.standard_normal((B, n, dm))
    I = np.eye(dm)
    for kind in (NONE, CAUSAL):
        Y = impl.mha_ref(X, X, I, I, I, I, 1, kind, None)
        X4 = X[:, None]
        O = impl.sdpa_ref(X4, X4, X4, 1.0 / math.sqrt(dm), kind, None)[:, 0]
        assert np.allclose(Y, O, atol=1e-14)


def check_mha_cross_sources(impl):
    """Cross-attention: queries come from X_q only, keys and values from X_kv
    only (hex4c59.cc, section "解码器有两种读取：看前缀，以及看源句"): rows of
    X_q act independently, and changing X_q does not change what a fixed
    query reads from X_kv."""
    r = _rng(15)
    B, n_q, n_k, dm, h, d = 1, 3, 7, 6, 2, 3
    X_q, X_kv, Wq, Wk, Wv, Wo = _mha_inputs(r, B, n_q, n_k, dm, h, d, d)
    Y = impl.mha_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, NONE, None)
    X_q2 = X_q.copy()
    X_q2[:, 1:] = r.standard_normal(X_q2[:, 1:].shape)
    Y2 = impl.mha_ref(X_q2, X_kv, Wq, Wk, Wv, Wo, h, NONE, None)
    assert np.allclose(Y2[:, 0], Y[:, 0], atol=1e-14)
    X_kv2 = X_kv.copy()
    X_kv2[:, 2] += 1.0
    assert np.abs(impl.mha_ref(X_q, X_kv2, Wq, Wk, Wv, Wo, h, NONE, None) - Y).max() > 1e-6


ALL_SDPA_CHECKS = [
    check_softmax_printed,
    check_worked_example,
    check_causal_pattern,
    check_rows_are_distributions,
    check_convex_combination,
    check_permutation_equivariance,
    check_causal_row0_and_last,
    check_zero_query_means,
    check_identical_keys_uniform,
    check_future_perturbation,
    check_padding_truncation,
    check_saturation,
    check_scale_statistics,
    check_bruteforce_sdpa,
    check_library_sdpa,
]

ALL_MHA_CHECKS = [
    check_bruteforce_mha,
    check_mha_head_blocks,
    check_mha_identity_reduction,
    check_mha_cross_sources,
]


# ------------------------------------------------------------ encoder layer pins
# Implementation interface for these: layer_norm(U, gamma, beta, eps),
# ffn(X, W1, b1, W2, b2), encoder_layer_ref(X, Wq, Wk, Wv, Wo, h, g1, be1,
# W1, b1, W2, b2, g2, be2, eps, mask_kind, key_lengths).

def check_layernorm_worked_row(impl):
    """u = (1, 2, 3, 4): mean 2.5, population variance 1.25 (the mean and
    variance of the row's own features, hex4c59.cc section "Add & Norm 里究竟
    发生了什么？"), so with gamma = 1, beta = 0, eps = 1e-5 the outputs are
    (-1.5, -0.5, 0.5, 1.5) / sqrt(1.25001)."""
    u = np.array([[1.0, 2.0, 3.0, 4.0]])
    out = impl.layer_norm(u, np.ones(4), np.zeros(4), 1e-5)
    den = math.sqrt(1.25001)
    assert np.allclose(out, [[-1.5 / den, -0.5 / den, 0.5 / den, 1.5 / den]], atol=1e-14, rtol=0)


def check_layernorm_moments(impl):
    """With eps = 0, gamma = 1, beta = 0 every normalised row has mean 0 and
    mean square 1 (closed form of standardisation)."""
    r = _rng(21)
    U = r.standard_normal((7, 33)) * 3.0 + 1.5
    out = impl.layer_norm(U, np.ones(33), np.zeros(33), 0.0)
    assert np.allclose(out.mean(axis=1), 0.0, atol=1e-14)
    assert np.allclose((out ** 2).mean(axis=1), 1.0, atol=1e-13)


def check_layernorm_affine_and_invariances(impl):
    """gamma and beta act per feature after normalising; adding a constant to
    a row changes nothing; scaling a row by a > 0 (eps = 0) changes nothing,
    by a < 0 flips the sign."""
    r = _rng(22)
    U = r.standard_normal((5, 12))
    g = r.standard_normal(12)
    b = r.standard_normal(12)
    base = impl.layer_norm(U, np.ones(12), np.zeros(12), 1e-5)
    assert np.allclose(impl.layer_norm(U, g, b, 1e-5), g * base + b, atol=1e-14)
    assert np.allclose(impl.layer_norm(U + 7.25, np.ones(12), np.zeros(12), 1e-5), base, atol=1e-12)
    n0 = impl.layer_norm(U, np.ones(12), np.zeros(12), 0.0)
    assert np.allclose(impl.layer_norm(3.5 * U, np.ones(12), np.zeros(12), 0.0), n0, atol=1e-13)
    assert np.allclose(impl.layer_norm(-2.0 * U, np.ones(12), np.zeros(12), 0.0), -n0, atol=1e-13)


def check_layernorm_bruteforce(impl):
    """The matrix form against the loop form on a small input."""
    import oracle
    r = _rng(23)
    U = r.standard_normal((4, 9))
    g = r.standard_normal(9)
    b = r.standard_normal(9)
    want = np.array(oracle.layer_norm_bruteforce(U.tolist(), g.tolist(), b.tolist(), 1e-5))
    assert np.allclose(impl.layer_norm(U, g, b, 1e-5), want, atol=1e-13)


def check_ffn_relu_identity(impl):
    """W1 = W2 = identity, b2 = 0: FFN(x) = max(0, x + b1) -- the bias enters
    before the ReLU (devpress.csdn.net section 2.3, max(0, x W1 + b1) W2 + b2)."""
    r = _rng(24)
    d = 6
    X = r.standard_normal((5, d))
    b1 = r.standard_normal(d)
    I = np.eye(d)
    out = impl.ffn(X, I, b1, I, np.zeros(d))
    assert np.allclose(out, np.maximum(0.0, X + b1), atol=1e-15)
    b2 = r.standard_normal(d)
    assert np.allclose(impl.ffn(X, I, b1, I, b2), np.maximum(0.0, X + b1) + b2, atol=1e-15)


def check_ffn_position_wise(impl):
    """Each row is transformed on its own (hex4c59.cc section "前馈网络为什么放在
    注意力后面？": a row does not read another row): permuting rows permutes
    the outputs, changing one row changes only its output."""
    r = _rng(25)
    X = r.standard_normal((6, 5))
    W1, b1 = r.standard_normal((5, 11)), r.standard_normal(11)
    W2, b2 = r.standard_normal((11, 5)), r.standard_normal(5)
    Y = impl.ffn(X, W1, b1, W2, b2)
    p = r.permutation(6)
    assert np.allclose(impl.ffn(X[p], W1, b1, W2, b2), Y[p], atol=1e-13)
    X2 = X.copy()
    X2[2] += 1.0
    Y2 = impl.ffn(X2, W1, b1, W2, b2)
    assert np.allclose(np.delete(Y2, 2, axis=0), np.delete(Y, 2, axis=0), atol=1e-14)
    assert np.abs(Y2[2] - Y[2]).max() > 1e-6


def check_ffn_bruteforce(impl):
    import oracle
    r = _rng(26)
    X = r.standard_normal((3, 4))
    W1, b1 = r.standard_normal((4, 7)), r.standard_normal(7)
    W2, b2 = r.standard_normal((7, 4)), r.standard_normal(4)
    want = np.array(oracle.ffn_bruteforce(X.tolist(), W1.tolist(), b1.tolist(), W2.tolist(), b2.tolist()))
    assert np.allclose(impl.ffn(X, W1, b1, W2, b2), want, atol=1e-13)


def _layer_weights(r, dm, h, d, dff):
    return dict(Wq=r.standard_normal((dm, h * d)), Wk=r.standard_normal((dm, h * d)),
                Wv=r.standard_normal((dm, h * d)), Wo=r.standard_normal((h * d, dm)),
                W1=r.standard_normal((dm, dff)), b1=r.standard_normal(dff),
                W2=r.standard_normal((dff, dm)), b2=r.standard_normal(dm))


def _layer(impl, X, w, h, g1, be1, g2, be2, eps, kind=NONE, kl=None):
    return impl.encoder_layer_ref(X, w["Wq"], w["Wk"], w["Wv"], w["Wo"], h, g1, be1, w["W1"], w["b1"],
                                  w["W2"], w["b2"], g2, be2, eps, kind, kl)


def check_layer_zero_sublayers(impl):
    """Post-LN with both sublayers silenced (W^O = 0, W2 = 0, b2 = 0, gamma = 1,
    beta = 0, eps = 0): each wrapper is LayerNorm(x + 0), so the layer is
    LayerNorm(LayerNorm(X)) = LayerNorm(X) (standardisation is idempotent).
    A missing residual, a residual outside the norm, or Pre-LN all differ."""
    r = _rng(27)
    B, n, dm, h, d, dff = 2, 5, 8, 2, 4, 16
    X = r.standard_normal((B, n, dm)) * 2.0 + 0.5
    w = _layer_weights(r, dm, h, d, dff)
    w["Wo"] = np.zeros_like(w["Wo"])
    w["W2"] = np.zeros_like(w["W2"])
    w["b2"] = np.zeros_like(w["b2"])
    one, zero = np.ones(dm), np.zeros(dm)
    out = _layer(impl, X, w, h, one, zero, one, zero, 0.0)
    mu = X.mean(axis=-1, keepdims=True)
    sd = np.sqrt(((X - mu) ** 2).mean(axis=-1, keepdims=True))
    assert np.allclose(out, (X - mu) / sd, atol=1e-12)


def check_layer_output_normalised(impl):
    """The layer ends in LayerNorm: with gamma2 = 1, beta2 = 0, eps = 0 every
    output row has mean 0 and mean square 1; beta2 then shifts the row mean
    to mean(beta2)."""
    r = _rng(28)
    B, n, dm, h, d, dff = 2, 4, 8, 2, 4, 12
    X = r.standard_normal((B, n, dm))
    w = _layer_weights(r, dm, h, d, dff)
    g1, be1 = r.standard_normal(dm), r.standard_normal(dm)
    out = _layer(impl, X, w, h, g1, be1, np.ones(dm), np.zeros(dm), 0.0)
    assert np.allclose(out.mean(axis=-1), 0.0, atol=1e-13)
    assert np.allclose((out ** 2).mean(axis=-1), 1.0, atol=1e-12)
    be2 = r.standard_normal(dm)
    out2 = _layer(impl, X, w, h, g1, be1, np.ones(dm), be2, 0.0)
    assert np.allclose(out2.mean(axis=-1), be2.mean(), atol=1e-13)


def check_layer_ffn_residual(impl):
    """With W2 = 0 the FFN sublayer is the constant b2: a b2 that is the same
    for every feature is removed by the second norm (shift invariance), a
    b2 that varies across features is not -- the FFN output is added to x1
    inside the norm."""
    r = _rng(29)
    B, n, dm, h, d, dff = 1, 4, 6, 2, 3, 8
    X = r.standard_normal((B, n, dm))
    w = _layer_weights(r, dm, h, d, dff)
    w["W2"] = np.zeros_like(w["W2"])
    one, zero = np.ones(dm), np.zeros(dm)
    w["b2"] = np.zeros(dm)
    base = _layer(impl, X, w, h, one, zero, one, zero, 1e-5)
    w["b2"] = np.full(dm, 3.0)
    assert np.allclose(_layer(impl, X, w, h, one, zero, one, zero, 1e-5), base, atol=1e-12)
    w["b2"] = np.linspace(-1.0, 1.0, dm)
    assert np.abs(_layer(impl, X, w, h, one, zero, one, zero, 1e-5) - base).max() > 1e-3


def check_layer_bruteforce(impl):
    """Tiny layer against the loop forms of every step (multi-head block,
    LayerNorm, FFN), composed in the pages' order, with a padding mask."""
    import oracle
    r = _rng(30)
    B, n, dm, h, d, dff = 2, 3, 4, 2, 2, 6
    X = r.standard_normal((B, n, dm))
    w = _layer_weights(r, dm, h, d, dff)
    g1, be1, g2, be2 = (r.standard_normal(dm) for _ in range(4))
    kl = [3, 2]
    got = _layer(impl, X, w, h, g1, be1, g2, be2, 1e-5, PAD, np.array(kl))
    for b in range(B):
        A = oracle.mha_bruteforce([X[b].tolist()], [X[b].tolist()], w["Wq"].tolist(), w["Wk"].tolist(),
                                  w["Wv"].tolist(), w["Wo"].tolist(), h, PAD, [kl[b]])[0]
        s1 = [[X[b][i][j] + A[i][j] for j in range(dm)] for i in range(n)]
        x1 = oracle.layer_norm_bruteforce(s1, g1.tolist(), be1.tolist(), 1e-5)
        F = oracle.ffn_bruteforce(x1, w["W1"].tolist(), w["b1"].tolist(), w["W2"].tolist(), w["b2"].tolist())
        s2 = [[x1[i][j] + F[i][j] for j in range(dm)] for i in range(n)]
        want = oracle.layer_norm_bruteforce(s2, g2.tolist(), be2.tolist(), 1e-5)
        assert np.allclose(got[b], np.array(want), atol=1e-12)


ALL_LAYER_CHECKS = [
    check_layernorm_worked_row,
    check_layernorm_moments,
    check_layernorm_affine_and_invariances,
    check_layernorm_bruteforce,
    check_ffn_relu_identity,
    check_ffn_position_wise,
    check_ffn_bruteforce,
    check_layer_zero_sublayers,
    check_layer_output_normalised,
    check_layer_ffn_residual,
    check_layer_bruteforce,
]


# ------------------------------------------------------------ input embedding pins
# Implementation interface: positional_encoding(n, d_model, pos0),
# embed_positional_ref(tokens, E, pos0).

def check_pe_printed_table(impl):
    """Table 4.1 of devpress.csdn.net section 4: d_model = 4, positions 0..4,
    printed to 4 decimals.  Tolerance one unit of the last printed digit:
    cos(0.01) = 0.999950000... is printed 0.9999 (the page's single-precision
    value lies just below the rounding point), every other entry is the
    correctly rounded value."""
    g = _golden("positional_encoding_table_4_1.json")
    pe = impl.positional_encoding(len(g["pe"]), g["d_model"], 0)
    assert np.abs(pe - np.array(g["pe"])).max() <= 1e-4 + 1e-12, pe


def check_embedding_worked_example(impl):
    """The worked example of the same section: x (5 positions, d_model 4) is
    scaled by sqrt(4) = 2 and the Table 4.1 encoding added.  Token p picks
    row p of a 5-row table holding the printed x."""
    g = _golden("positional_encoding_table_4_1.json")
    x = np.array(g["x"])
    out = impl.embed_positional_ref(np.arange(5)[None, :], x, 0)
    want = g["xscale"] * x + np.array(g["pe"])
    assert g["xscale"] == math.sqrt(g["d_model"])
    assert np.abs(out[0] - want).max() <= 1e-4 + 1e-12, out


def check_pe_pairs_and_origin(impl):
    """Each (sin, cos) pair has unit norm; position 0 is (0, 1, 0, 1, ...);
    the first pair turns at frequency 1 (sin pos, cos pos); positions
    pos0 .. pos0+n-1 are rows pos0.. of the encoding from 0."""
    d = 512
    pe = impl.positional_encoding(300, d, 0)
    assert np.allclose(pe[:, 0::2] ** 2 + pe[:, 1::2] ** 2, 1.0, atol=1e-15)
    assert np.array_equal(pe[0], np.tile([0.0, 1.0], d // 2))
    pos = np.arange(300.0)
    assert np.allclose(pe[:, 0], np.sin(pos), atol=1e-15) and np.allclose(pe[:, 1], np.cos(pos), atol=1e-15)
    assert np.allclose(impl.positional_encoding(40, d, 123), pe[123:163], atol=1e-15)


def check_pe_shift_identity(impl):
    """devpress.csdn.net section 4: PE(pos + k) is PE(pos) with each pair
    rotated by omega_i k, omega_i = 10000^(-2i/d_model) -- pins every
    pair's frequency at d_model = 512."""
    d = 512
    pe = impl.positional_encoding(200, d, 0)
    omega = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    for k in (1, 7, 50):
        s, c = pe[:-k, 0::2], pe[:-k, 1::2]
        rs = s * np.cos(omega * k) + c * np.sin(omega * k)
        rc = c * np.cos(omega * k) - s * np.sin(omega * k)
        assert np.allclose(pe[k:, 0::2], rs, atol=1e-12) and np.allclose(pe[k:, 1::2], rc, atol=1e-12)


def check_embedding_bruteforce(impl):
    import oracle
    r = _rng(31)
    E = r.standard_normal((11, 6))
    tokens = r.integers(0, 11, (2, 5))
    want = np.array(oracle.embed_positional_bruteforce(tokens.tolist(), E.tolist(), 3))
    assert np.allclose(impl.embed_positional_ref(tokens, E, 3), want, atol=1e-13)


ALL_EMBED_CHECKS = [
    check_pe_printed_table,
    check_embedding_worked_example,
    check_pe_pairs_and_origin,
    check_pe_shift_identity,
    check_embedding_bruteforce,
]


# ------------------------------------------------------------ backward pass pins
# Implementation interface: sdpa_backward_ref(Q, K, V, dO, scale, mask_kind,
# key_lengths) -> (dQ, dK, dV); row_logsumexp(Q, K, scale, mask_kind, key_lengths).

def _bwd_inputs(seed, B, h, n_q, n_k, d):
    r = _rng(seed)
    return (r.standard_normal((B, h, n_q, d)), r.standard_normal((B, h, n_k, d)),
            r.standard_normal((B, h, n_k, d)), r.standard_normal((B, h, n_q, d)))


def check_bwd_finite_differences(impl):
    """Every gradient element against the central difference of the loss
    sum(dO * O) in float64 (step 1e-5: truncation ~1e-10, rounding ~1e-11),
    for each mask kind.  The forward is the oracle's sdpa_ref, already
    pinned on its own; the backward is never consulted for the reference."""
    import oracle
    cases = [(NONE, 3, 4, None), (CAUSAL, 4, 4, None), (PAD, 3, 5, [5, 2]), (BOTH, 4, 4, [3, 1])]
    for kind, n_q, n_k, kl in cases:
        Q, K, V, dO = _bwd_inputs(40 + kind, 2, 2, n_q, n_k, 3)
        kl = None if kl is None else np.array(kl)
        scale = 0.7
        got = impl.sdpa_backward_ref(Q, K, V, dO, scale, kind, kl)
        base = [Q, K, V]
        for which in range(3):
            want = np.zeros_like(base[which])
            it = np.nditer(base[which], flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                vals = []
                for sgn in (1.0, -1.0):
                    args = [t.copy() for t in base]
                    args[which][idx] += sgn * 1e-5
                    vals.append(float((dO * oracle.sdpa_ref(*args, scale, kind, kl)).sum()))
                want[idx] = (vals[0] - vals[1]) / 2e-5
            assert np.abs(got[which] - want).max() <= 1e-7, (kind, which, np.abs(got[which] - want).max())


def check_bwd_invariants(impl):
    """Shifting every key of a sequence by the same vector adds a constant to
    each row of scores and leaves the softmax unchanged, so the key gradients
    of each (batch, head) sum to zero; keys no query can see (padding) get
    exactly zero dK and dV; under the causal mask the last key is seen by the
    last query only."""
    Q, K, V, dO = _bwd_inputs(45, 2, 3, 6, 6, 4)
    for kind, kl in ((NONE, None), (CAUSAL, None), (PAD, np.array([4, 6])), (BOTH, np.array([2, 5]))):
        dQ, dK, dV = impl.sdpa_backward_ref(Q, K, V, dO, 0.5, kind, kl)
        assert np.abs(dK.sum(axis=2)).max() <= 1e-12
        if kl is not None:
            assert np.all(dK[0, :, kl[0]:] == 0) and np.all(dV[0, :, kl[0]:] == 0)
    _, dK, dV = impl.sdpa_backward_ref(Q, K, V, dO, 0.5, CAUSAL, None)
    dO2 = dO.copy()
    dO2[:, :, :5] = _rng(46).standard_normal(dO2[:, :, :5].shape)
    _, dK2, dV2 = impl.sdpa_backward_ref(Q, K, V, dO2, 0.5, CAUSAL, None)
    assert np.array_equal(dK2[:, :, 5], dK[:, :, 5]) and np.array_equal(dV2[:, :, 5], dV[:, :, 5])
    assert not np.allclose(dV2[:, :, 4], dV[:, :, 4])


def check_bwd_uniform_weights(impl):
    """Q = 0: every visible key has weight 1/n.  Then dV_j = (1/n) sum_i dO_i,
    dK = 0 exactly, and dQ_i = (scale/n) sum_j (dO_i . (V_j - mean V)) K_j
    (unmasked, written out with loops)."""
    _, K, V, dO = _bwd_inputs(47, 1, 2, 3, 5, 4)
    Q = np.zeros((1, 2, 3, 4))
    scale = 0.8
    dQ, dK, dV = impl.sdpa_backward_ref(Q, K, V, dO, scale, NONE, None)
    n = 5
    assert np.array_equal(dK, np.zeros_like(dK))
    for hh in range(2):
        vbar = V[0, hh].mean(axis=0)
        for j in range(n):
            assert np.allclose(dV[0, hh, j], dO[0, hh].sum(axis=0) / n, atol=1e-14)
        for i in range(3):
            want = sum((dO[0, hh, i] @ (V[0, hh, j] - vbar)) * K[0, hh, j] for j in range(n)) * scale / n
            assert np.allclose(dQ[0, hh, i], want, atol=1e-13)


def check_row_logsumexp(impl):
    """Against a loop with math.fsum over the visible keys; exp(S - lse) rows
    then sum to one."""
    Q, K, _, _ = _bwd_inputs(48, 2, 2, 4, 4, 3)
    kl = np.array([4, 2])
    for kind in (NONE, CAUSAL, PAD, BOTH):
        lse = impl.row_logsumexp(Q, K, 0.6, kind, kl if kind & PAD else None)
        for b in range(2):
            for hh in range(2):
                for i in range(4):
                    vis = [j for j in range(4) if not ((kind & CAUSAL and j > i) or (kind & PAD and j >= kl[b]))]
                    s = [0.6 * float(Q[b, hh, i] @ K[b, hh, j]) for j in vis]
                    want = math.log(math.fsum(math.exp(x) for x in s))
                    assert abs(lse[b, hh, i] - want) <= 1e-13


def check_mha_bwd_finite_differences(impl):
    """Block gradients against central differences of sum(dY * Y), cross-
    attention with padding and self-attention with the causal mask (there the
    shared input's gradient is dX_q + dX_kv), every element of every input
    and weight.  The forward is the oracle's mha_ref, pinned on its own."""
    import oracle
    r = _rng(49)
    for self_attn, kind, kl in ((False, PAD, np.array([3, 2])), (True, CAUSAL, None)):
        B, n_q, n_k, dm, h, d = 2, 3, (3 if self_attn else 4), 4, 2, 2
        X_q = r.standard_normal((B, n_q, dm))
        X_kv = X_q if self_attn else r.standard_normal((B, n_k, dm))
        W = [r.standard_normal((dm, h * d)) for _ in range(3)] + [r.standard_normal((h * d, dm))]
        dY = r.standard_normal((B, n_q, dm))
        got = impl.mha_backward_ref(X_q, X_kv, *W, h, dY, kind, kl)
        dX_want = got[0] + got[1] if self_attn else None

        def loss(Xq, Xkv, Ws):
            return float((dY * oracle.mha_ref(Xq, Xkv, *Ws, h, kind, kl)).sum())

        def fd(arr, setter):
            g = np.zeros_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                vals = []
                for sgn in (1.0, -1.0):
                    a2 = arr.copy()
                    a2[it.multi_index] += sgn * 1e-5
                    vals.append(setter(a2))
                g[it.multi_index] = (vals[0] - vals[1]) / 2e-5
            return g
        if self_attn:
            assert np.abs(fd(X_q, lambda a: loss(a, a, W)) - dX_want).max() <= 1e-7
        else:
            assert np.abs(fd(X_q, lambda a: loss(a, X_kv, W)) - got[0]).max() <= 1e-7
            assert np.abs(fd(X_kv, lambda a: loss(X_q, a, W)) - got[1]).max() <= 1e-7
        for j in range(4):
            def set_w(a, j=j):
                W2 = list(W)
                W2[j] = a
                return loss(X_q, X_kv, W2)
            assert np.abs(fd(W[j], set_w) - got[2 + j]).max() <= 1e-7, (self_attn, j)


ALL_BWD_CHECKS = [
    check_bwd_finite_differences,
    check_mha_bwd_finite_differences,
    check_bwd_invariants,
    check_bwd_uniform_weights,
    check_row_logsumexp,
]
