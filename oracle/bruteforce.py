"""Brute-force oracle: pure-Python loops, one query row at a time.

TEST INFRASTRUCTURE ONLY.  Used on tiny inputs to cross-check the numpy
matrix form in ``oracle.attention``; it shares no code with it (no numpy
arithmetic, its own mask test, its own softmax).

For each (batch, head, query r): the visible keys are c with
  c <= r            when causal   (hex4c59.cc "读懂 Attention Is All You Need",
                                   section "掩码必须在 softmax 之前生效")
  c <  L_b          when padded   (same section, padding-mask paragraph)
scores s_c = (q . k_c) * scale over visible c only (a masked key gets weight
exactly 0, which is what adding -inf before the softmax achieves), weights
w_c = exp(s_c - max s) / sum exp(s - max s), output sum_c w_c v_c
(section "六步算完一行注意力": dot products, divide by sqrt(d_k), softmax,
weighted sum of values).
"""

import math


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def attention_bruteforce(Q, K, V, scale, mask_kind=0, key_lengths=None):
    """Q, K, V: nested Python sequences [B][h][n][d] (anything indexable that
    yields floats).  Returns nested lists [B][h][n_q][d_v]."""
    B = len(Q)
    out = []
    for b in range(B):
        ob = []
        for hh in range(len(Q[b])):
            q_rows = Q[b][hh]
            k_rows = K[b][hh]
            v_rows = V[b][hh]
            n_k = len(k_rows)
            oh = []
            for r in range(len(q_rows)):
                vis = []
                for c in range(n_k):
                    if (mask_kind & 1) and c > r:
                        continue
                    if (mask_kind & 2) and c >= key_lengths[b]:
                        continue
                    vis.append(c)
                if not vis:
                    raise ValueError("query with no visible key")
                s = [float(_dot(q_rows[r], k_rows[c])) * scale for c in vis]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = math.fsum(e)
                w = [x / z for x in e]
                d_v = len(v_rows[0])
                oh.append([math.fsum(w[t] * float(v_rows[c][j]) for t, c in enumerate(vis))
                           for j in range(d_v)])
            ob.append(oh)
        out.append(ob)
    return out


def _matmul(A, W):
    """Triple loop A[n][k] . W[k][m]."""
    kdim = len(W)
    m = len(W[0])
    return [[math.fsum(float(A[i][t]) * float(W[t][j]) for t in range(kdim)) for j in range(m)]
            for i in range(len(A))]


def mha_bruteforce(X_q, X_kv, Wq, Wk, Wv, Wo, h, mask_kind=0, key_lengths=None):
    """Multi-head block by loops: per-batch projections, head i takes columns
    [i*d, (i+1)*d), attention per head, concatenation, output projection.
    Inputs nested sequences; returns [B][n_q][d_model] nested lists."""
    B = len(X_q)
    d_k = len(Wq[0]) // h
    d_v = len(Wv[0]) // h
    scale = 1.0 / math.sqrt(d_k)
    Y = []
    for b in range(B):
        Qb = _matmul(X_q[b], Wq)
        Kb = _matmul(X_kv[b], Wk)
        Vb = _matmul(X_kv[b], Wv)
        heads = []
        for i in range(h):
            q = [[row[i * d_k + j] for j in range(d_k)] for row in Qb]
            k = [[row[i * d_k + j] for j in range(d_k)] for row in Kb]
            v = [[row[i * d_v + j] for j in range(d_v)] for row in Vb]
            kl = None if key_lengths is None else [key_lengths[b]]
            heads.append(attention_bruteforce([[q]], [[k]], [[v]], scale, mask_kind, kl)[0][0])
        concat = [[heads[i][r][j] for i in range(h) for j in range(d_v)] for r in range(len(Qb))]
        Y.append(_matmul(concat, Wo))
    return Y


def layer_norm_bruteforce(U, gamma, beta, eps):
    """LayerNorm by loops, one row at a time: mean and population variance of
    the row's d features with math.fsum, then gamma_j (u_j - mean) /
    sqrt(var + eps) + beta_j (hex4c59.cc, section "Add & Norm 里究竟发生了什么？").
    U nested [rows][d]; returns nested lists."""
    out = []
    for row in U:
        d = len(row)
        mean = math.fsum(float(x) for x in row) / d
        var = math.fsum((float(x) - mean) ** 2 for x in row) / d
        den = math.sqrt(var + eps)
        out.append([float(gamma[j]) * (float(row[j]) - mean) / den + float(beta[j]) for j in range(d)])
    return out


def ffn_bruteforce(X, W1, b1, W2, b2):
    """Position-wise feed-forward network by loops: for every row,
    hidden_j = max(0, sum_t x_t W1[t][j] + b1_j), out_j = sum_j' hidden_j'
    W2[j'][j] + b2_j (devpress.csdn.net, section 2.3).  X nested [rows][d]."""
    out = []
    for row in X:
        hid = [max(0.0, math.fsum(float(row[t]) * float(W1[t][j]) for t in range(len(row))) + float(b1[j]))
               for j in range(len(b1))]
        out.append([math.fsum(hid[t] * float(W2[t][j]) for t in range(len(hid))) + float(b2[j])
                    for j in range(len(b2))])
    return out


def embed_positional_bruteforce(tokens, E, pos0=0):
    """Loop form of the scaled embedding plus sinusoidal encoding: for each
    sequence b, position p and coordinate j, E[token][j] * sqrt(d) plus
    sin or cos of (pos0 + p) / 10000^(2 (j // 2) / d), sine on even j."""
    d = len(E[0])
    out = []
    for row in tokens:
        seq = []
        for p, t in enumerate(row):
            pos = pos0 + p
            vec = []
            for j in range(d):
                angle = pos / 10000.0 ** (2 * (j // 2) / d)
                enc = math.sin(angle) if j % 2 == 0 else math.cos(angle)
                vec.append(E[t][j] * math.sqrt(d) + enc)
            seq.append(vec)
        out.append(seq)
    return out
