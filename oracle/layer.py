"""Matrix-form oracle for the rest of an encoder layer: residual + LayerNorm
(Post-LN) and the position-wise feed-forward network.  numpy, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

Sources:
* hex4c59.cc, "读懂 Attention Is All You Need", section "Add & Norm 里究竟发生了
  什么？": the sublayer output is added to its input and the sum is
  normalised (Post-LN); LayerNorm normalises one token's feature vector with
  that vector's own mean and variance, then applies a learned scale gamma
  and shift beta, with a small constant eps in the denominator.  Section
  "前馈网络为什么放在注意力后面？": the feed-forward network acts on each
  position separately, ReLU between two linear maps, width 512 -> 2048 -> 512
  in the base model.
* devpress.csdn.net, "【深度学习】Transformer", section 2.3: the encoder block
  runs x + sa_block(x), norm1, x + FFN(x) with FFN(x) = max(0, x W1 + b1) W2
  + b2, norm2.
* research-heat.pages.dev, "做法 · Attention Is All You Need", section on the
  encoder-decoder shape: every sublayer is wrapped as LayerNorm(x +
  Sublayer(x)).

Readings (the pages leave these open; see the design notes):
* The variance is the population variance of the d features (divide by d):
  the pages call mu and sigma^2 the mean and variance of the d features.
* eps is an argument; the pages give no value (their code uses the library
  layer norm with its default), 1e-5 is the value used by the tests.
* Weights are applied as x W (rows are positions), as in the pages' formula.

Layouts: rows are positions, the last axis is the feature axis.
  X [M][d_model], W1 [d_model][d_ff], b1 [d_ff], W2 [d_ff][d_model], b2 [d_model]
  gamma, beta [d_model]
"""

import numpy as np

from .attention import _f64, mha_ref


def layer_norm(U, gamma, beta, eps):
    """LayerNorm over the last axis: gamma * (u - mu) / sqrt(sigma^2 + eps) + beta,
    mu and sigma^2 the mean and (population) variance of the row's features.
    Parity: pinned by closed forms (zero row mean, known mean square, a worked
    row), the affine and shift invariances, and brute force."""
    U = _f64(U)
    gamma = _f64(gamma)
    beta = _f64(beta)
    if eps < 0:
        raise ValueError("eps must be >= 0")
    mu = U.mean(axis=-1, keepdims=True)
    var = ((U - mu) ** 2).mean(axis=-1, keepdims=True)
    return gamma * (U - mu) / np.sqrt(var + eps) + beta


def add_layer_norm(X, F, gamma, beta, eps):
    """Post-LN sublayer wrapper: LayerNorm(x + Sublayer(x)), with F the
    sublayer's output.  Parity: pinned (see layer_norm; the residual by the
    zero-sublayer special case)."""
    return layer_norm(_f64(X) + _f64(F), gamma, beta, eps)


def ffn(X, W1, b1, W2, b2):
    """Position-wise feed-forward network: max(0, x W1 + b1) W2 + b2 on every
    row.  Parity: pinned by the identity/ReLU special case, row independence
    and brute force."""
    X = _f64(X)
    H = np.maximum(0.0, X @ _f64(W1) + _f64(b1))
    return H @ _f64(W2) + _f64(b2)


def encoder_layer_ref(X, Wq, Wk, Wv, Wo, h, ln1_gamma, ln1_beta, W1, b1, W2, b2,
                      ln2_gamma, ln2_beta, eps, mask_kind=0, key_lengths=None,
                      return_intermediates=False):
    """One encoder layer (self-attention), Post-LN:
        x1  = LayerNorm1(X + MultiHead(X, X, X))
        out = LayerNorm2(x1 + FFN(x1))
    X [B][n][d_model].  Parity: composition of pinned steps, with the
    zero-sublayer reductions pinned in tests/test_oracle.py."""
    X = _f64(X)
    A = mha_ref(X, X, Wq, Wk, Wv, Wo, h, mask_kind, key_lengths)
    x1 = add_layer_norm(X, A, ln1_gamma, ln1_beta, eps)
    F = ffn(x1, W1, b1, W2, b2)
    out = add_layer_norm(x1, F, ln2_gamma, ln2_beta, eps)
    if return_intermediates:
        return out, dict(attn=A, x1=x1, ffn=F)
    return out
