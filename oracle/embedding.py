"""Matrix-form oracle for the input side of the model: token embedding
scaled by sqrt(d_model) plus the sinusoidal positional encoding.  numpy,
float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

Sources:
* devpress.csdn.net, "【深度学习】Transformer（Attention Is All You Need）",
  section 4 (位置编码): equation (4.1), PE(pos, 2i) = sin(pos / 10000^(2i/d_model))
  and PE(pos, 2i+1) = cos(pos / 10000^(2i/d_model)); the angular frequency of
  pair i is 1 / 10000^(2i/d_model); Table 4.1 prints the d_model = 4 case; the
  worked example scales the input by sqrt(d_model) before adding the
  encoding; the shift identity (a fixed offset k rotates each (sin, cos)
  pair by the angle omega_i k).
* hex4c59.cc, "读懂 Attention Is All You Need", section "没有循环，模型怎样知道
  词序？": E is the embedding row looked up by token id, multiplied by
  sqrt(d_model), and the encoding is added (equal widths); pos is the
  position, i indexes a pair of adjacent even/odd coordinates.
* research-heat.pages.dev, "做法 · Attention Is All You Need", the section on
  restoring word order: even coordinates take the sine, odd the cosine.

Readings: positions count from 0 (Table 4.1 starts at pos = 0); a sequence's
positions are pos0, pos0 + 1, ... (pos0 = 0 for a whole sentence, the step
index when one new token is embedded during incremental decoding).
"""

import math

import numpy as np

from .attention import _f64


def positional_encoding(n, d_model, pos0=0):
    """PE [n][d_model] for positions pos0 .. pos0 + n - 1.
    Parity: pinned by the printed Table 4.1, closed forms at pos = 0, the
    unit norm of every (sin, cos) pair and the shift identity."""
    if d_model % 2:
        raise ValueError("d_model must be even (coordinates come in sin/cos pairs)")
    pos = np.arange(pos0, pos0 + n, dtype=np.float64)[:, None]
    i = np.arange(d_model // 2, dtype=np.float64)[None, :]
    omega = 1.0 / np.power(10000.0, 2.0 * i / d_model)
    pe = np.empty((n, d_model), dtype=np.float64)
    pe[:, 0::2] = np.sin(pos * omega)
    pe[:, 1::2] = np.cos(pos * omega)
    return pe


def embed_positional_ref(tokens, E, pos0=0):
    """out[b][p] = E[tokens[b][p]] * sqrt(d_model) + PE(pos0 + p).
    tokens int [B][n] (each in [0, vocab)), E [vocab][d_model].
    Parity: pinned by the printed worked example (scale 2 for d_model = 4),
    brute force, and the encoding's pins."""
    E = _f64(E)
    tokens = np.asarray(tokens)
    if tokens.min() < 0 or tokens.max() >= E.shape[0]:
        raise ValueError("token id outside the vocabulary")
    B, n = tokens.shape
    d = E.shape[1]
    return E[tokens] * math.sqrt(d) + positional_encoding(n, d, pos0)[None]
