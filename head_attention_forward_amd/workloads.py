"""Seeded synthetic workloads for multi-head attention.

This module only draws inputs: shapes, distributions and random numbers.  It
holds none of the attention arithmetic and is shared by the tests, the bench
and the smoke check (the oracle never imports it; callers hand it arrays).

The pages' workloads are WMT 2014 translation batches, which are not used;
seeded Gaussian tensors of the pages' model shapes stand in for them:
the base model (d_model = 512, h = 8, d_k = d_v = 64) and the big model
(d_model = 1024, h = 16).  Base shapes follow hex4c59.cc "读懂 Attention Is All
You Need" (section "多头注意力让一次读取有多组投影") and research-heat.pages.dev
"做法" (section "一次平均不够，因而切开多头"); batch 32 x length 100 matches
the worked shapes of devpress.csdn.net "【深度学习】Transformer", section 2.2.

Recipe (every workload): one ``torch.Generator('cpu')`` seeded with ``seed``;
fp32 standard-normal draws scaled by the stated standard deviation, in the
fixed order X_q, X_kv (cross-attention only), Wq, Wk, Wv, Wo, key_lengths for
the multi-head block and Q, K, V for bare attention; then a round-to-nearest-
even cast to bf16 (fp32 workloads stay fp32).  Projection weights have
variance 1/d_model.  Key lengths are integers drawn uniformly from
[lo, hi] inclusive.

Encoder layer (kind "layer"; the rest of the layer as hex4c59.cc, sections
"前馈网络为什么放在注意力后面？" and "Add & Norm 里究竟发生了什么？", describe
it: FFN width 2048 for the base model): draws in the order X, Wq, Wk, Wv,
Wo, ln1_gamma, ln1_beta, W1, b1, W2, b2, ln2_gamma, ln2_beta, key_lengths.
W1 has variance 1/d_model, W2 1/d_ff; biases and LayerNorm shifts are
0.1 * N(0, 1), LayerNorm scales 1 + 0.1 * N(0, 1) (non-trivial values, so
that every term of the layer shows in its output).

Backward pass (kind "bwd"): Q, K, V as bare attention, then the upstream
gradient dO ~ N(0, 1), then key lengths.  Block backward (kind "mha_bwd"):
the block's inputs and weights, then dY ~ N(0, 1), then key lengths.

Input embedding (kind "embed"): token ids uniform over the vocabulary, drawn
first, then the table E [vocab][d_model] with variance 1/d_model (so that
E * sqrt(d_model) has unit variance, the scale of the encoding); positions
from 0.
"""

import dataclasses
import math
from typing import Optional, Tuple

import torch

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEY_PADDING = 2
MASK_CAUSAL_KEY_PADDING = 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "sdpa" (bare attention) or "mha" (full block)
    dtype: str           # "bf16" or "f32"
    B: int
    n_q: int
    n_k: int
    h: int
    d_k: int
    d_v: int
    mask: int
    d_model: int = 0
    self_attn: bool = False
    key_len_range: Optional[Tuple[int, int]] = None
    description: str = ""
    d_ff: int = 0        # encoder layer: FFN hidden width
    eps: float = 1e-5    # encoder layer: LayerNorm epsilon
    vocab: int = 0       # input embedding: vocabulary size
    iters: int = 0       # matrix-core probe: products per chain (B is its workgroup count)
    operands: str = ""   # matrix-core probe: "dense" (random bits) or "sparse" (few set bits)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def nominal_attention_flops(self):
        """4 * B * h * n_q * n_k * d_k (QK^T and PV, dense)."""
        return 4.0 * self.B * self.h * self.n_q * self.n_k * self.d_k

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "sdpa_f32_tiny": Workload(
        "sdpa_f32_tiny", "sdpa", "f32", B=1, n_q=64, n_k=64, h=1, d_k=64, d_v=64,
        mask=MASK_NONE,
        description="bare attention, fp32, B=1 h=1 n=64 d=64, unmasked"),
    "encoder_self_base": Workload(
        "encoder_self_base", "mha", "bf16", B=32, n_q=100, n_k=100, h=8, d_k=64, d_v=64,
        mask=MASK_NONE, d_model=512, self_attn=True,
        description="encoder self-attention block, bf16, B=32 n=100 d_model=512 h=8 d=64"),
    "decoder_causal_base": Workload(
        "decoder_causal_base", "mha", "bf16", B=16, n_q=512, n_k=512, h=8, d_k=64, d_v=64,
        mask=MASK_CAUSAL, d_model=512, self_attn=True,
        description="decoder causal self-attention block, bf16, B=16 n=512 d_model=512 h=8"),
    "cross_padded_big": Workload(
        "cross_padded_big", "mha", "bf16", B=32, n_q=96, n_k=128, h=16, d_k=64, d_v=64,
        mask=MASK_KEY_PADDING, d_model=1024, self_attn=False, key_len_range=(64, 128),
        description="cross-attention block, bf16, B=32 n_q=96 n_k=128 d_model=1024 h=16, "
                    "key padding with lengths in [64,128]"),
    # The encoder block's attention alone (the staged path's middle stage):
    # per (batch, head) 100 queries over 100 keys, moving Q, K, V and O
    # through HBM -- the short, bandwidth-bound attention shape.
    "encoder_self_base_sdpa": Workload(
        "encoder_self_base_sdpa", "sdpa", "bf16", B=32, n_q=100, n_k=100, h=8, d_k=64, d_v=64,
        mask=MASK_NONE,
        description="bare attention at the encoder block's shape, bf16, B=32 h=8 n=100 d=64, "
                    "unmasked"),
    # The fixed cost of a launch at that shape, measured the same way: a
    # kernel that does nothing over the attention's grid (32 x 8 workgroups of
    # 256 threads), and one that only reads Q, K, V (9.8 MB) and writes an
    # output of O's size (3.3 MB) -- the floor under the short attention.
    "launch_floor_encoder_sdpa": Workload(
        "launch_floor_encoder_sdpa", "floor", "bf16", B=32, n_q=100, n_k=100, h=8, d_k=64, d_v=64,
        mask=MASK_NONE,
        description="launch floor at the encoder attention's shape: an empty kernel and a "
                    "kernel moving the same 13.1 MB, 256 workgroups of 256 threads"),
    # The dense bf16 throughput the matrix cores sustain on this device as it
    # runs (shader clock under that load included): the practical ceiling the
    # nominal 2516.6 TFLOP/s overstates.  1024 workgroups of four waves (four
    # per compute unit), four independent chains of 16384 products per wave,
    # with operands whose bits are as busy as those of normally distributed
    # data; the sparse variant feeds operands with few set bits, which draw
    # less power and let the clock stay higher.
    "mfma_peak_probe": Workload(
        "mfma_peak_probe", "mfma", "bf16", B=1024, n_q=1, n_k=1, h=1, d_k=64, d_v=64,
        mask=MASK_NONE, iters=16384, operands="dense",
        description="matrix-core probe: 1024 workgroups x 4 waves x 4 chains of 16384 "
                    "v_mfma_f32_32x32x16_bf16 on random-bit operands, no memory traffic"),
    "mfma_peak_probe_sparse": Workload(
        "mfma_peak_probe_sparse", "mfma", "bf16", B=1024, n_q=1, n_k=1, h=1, d_k=64, d_v=64,
        mask=MASK_NONE, iters=16384, operands="sparse",
        description="matrix-core probe as mfma_peak_probe, operands small multiples of 1/1024"),
    "long_causal_sdpa": Workload(
        "long_causal_sdpa", "sdpa", "bf16", B=4, n_q=4096, n_k=4096, h=16, d_k=64, d_v=64,
        mask=MASK_CAUSAL,
        description="bare causal attention, bf16, B=4 h=16 n=4096 d=64"),
    # The long causal attention at batch 1 and 8 heads: 256 query tiles of
    # 128, at most one workgroup per compute unit, which the launch serves
    # with two key groups per workgroup.
    "long_causal_b1_sdpa": Workload(
        "long_causal_b1_sdpa", "sdpa", "bf16", B=1, n_q=4096, n_k=4096, h=8, d_k=64, d_v=64,
        mask=MASK_CAUSAL,
        description="bare causal attention at small batch, bf16, B=1 h=8 n=4096 d=64"),
    # Training's backward pass over the long causal shape: gradients of the
    # attention for an upstream gradient dO ~ N(0, 1).
    "long_causal_sdpa_bwd": Workload(
        "long_causal_sdpa_bwd", "bwd", "bf16", B=4, n_q=4096, n_k=4096, h=16, d_k=64, d_v=64,
        mask=MASK_CAUSAL,
        description="attention backward (dQ, dK, dV), bf16, B=4 h=16 n=4096 d=64, causal"),
    # The encoder block's backward pass (training): all gradients of the
    # multi-head block for an upstream gradient dY ~ N(0, 1).
    "encoder_self_base_bwd": Workload(
        "encoder_self_base_bwd", "mha_bwd", "bf16", B=32, n_q=100, n_k=100, h=8, d_k=64, d_v=64,
        mask=MASK_NONE, d_model=512, self_attn=True,
        description="encoder self-attention block backward (dX, dW^Q, dW^K, dW^V, dW^O), bf16, "
                    "B=32 n=100 d_model=512 h=8"),
    # One generation step of incremental decoding: each sequence's newest
    # query against its cached keys and values (cache capacity 4096, current
    # lengths in [1024, 4096]); the pages give no decoding shapes, these are
    # the big model's 16 heads at batch 32.
    "decode_step_sdpa": Workload(
        "decode_step_sdpa", "sdpa", "bf16", B=32, n_q=1, n_k=4096, h=16, d_k=64, d_v=64,
        mask=MASK_KEY_PADDING, key_len_range=(1024, 4096),
        description="bare attention, one query per sequence over a 4096-key cache, bf16, "
                    "B=32 h=16 d=64, cache lengths in [1024,4096]"),
    # The same decoding step at a small batch: 8 sequences x 16 heads = 128
    # (batch, head) pairs, fewer than the compute units, each over a full
    # 4096-key cache (sdpa_decode, which splits each pair's keys over several
    # workgroups).
    "decode_small_batch_sdpa": Workload(
        "decode_small_batch_sdpa", "decode", "bf16", B=8, n_q=1, n_k=4096, h=16, d_k=64, d_v=64,
        mask=MASK_NONE,
        description="bare attention, one query per sequence over a full 4096-key cache, bf16, "
                    "B=8 h=16 d=64 (sdpa_decode)"),
    # One Post-LN encoder layer of the base model (multi-head self-attention,
    # residual + LayerNorm, FFN 512 -> 2048 -> 512, residual + LayerNorm) on
    # the encoder block's batch.
    "encoder_layer_base": Workload(
        "encoder_layer_base", "layer", "bf16", B=32, n_q=100, n_k=100, h=8, d_k=64, d_v=64,
        mask=MASK_NONE, d_model=512, self_attn=True, d_ff=2048, eps=1e-5,
        description="encoder layer (Post-LN), bf16, B=32 n=100 d_model=512 h=8 d_ff=2048"),
    # The model's input for the encoder batch: token ids into a vocabulary of
    # about 37000 sub-words (wiki.hugogu.cn "Attention Is All You Need", the
    # input-embedding paragraph), embedding rows scaled by sqrt(d_model) plus
    # the sinusoidal encoding.
    "embed_positional_base": Workload(
        "embed_positional_base", "embed", "bf16", B=32, n_q=100, n_k=100, h=0, d_k=0, d_v=0,
        mask=MASK_NONE, d_model=512, vocab=37000,
        description="token embedding x sqrt(d_model) + sinusoidal encoding, bf16, B=32 n=100 "
                    "d_model=512 vocab=37000"),
}

ORDER = ["sdpa_f32_tiny", "encoder_self_base", "decoder_causal_base", "cross_padded_big",
         "long_causal_sdpa"]


def _normal(g, shape, std, dtype):
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def generate(w: Workload, seed: int = 0):
    """Draw the inputs of ``w`` on the CPU.  Returns a dict of tensors.

    sdpa: Q [B][h][n_q][d_k], K [B][h][n_k][d_k], V [B][h][n_k][d_v], scale,
          key_lengths (int32 [B] or None).
    decode, floor: the same draws as sdpa.
    bwd:  as sdpa, then the upstream gradient dO [B][h][n_q][d_v].
    mha_bwd: as mha, then the upstream gradient dY [B][n_q][d_model].
    mha:  X_q [B][n_q][d_model], X_kv (the same tensor object for
          self-attention), Wq/Wk [d_model][h*d_k], Wv [d_model][h*d_v],
          Wo [h*d_v][d_model], key_lengths.
    embed: tokens int32 [B][n], E [vocab][d_model], pos0.
    layer: X [B][n][d_model], the block's Wq, Wk, Wv, Wo, then ln1_gamma,
          ln1_beta [d_model], W1 [d_model][d_ff], b1 [d_ff], W2 [d_ff][d_model],
          b2, ln2_gamma, ln2_beta [d_model], key_lengths.
    """
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    dt = w.torch_dtype
    out = {}
    if w.kind == "mfma":  # the probe reads no inputs
        out["key_lengths"] = None
        return out
    if w.kind in ("sdpa", "decode", "bwd", "floor"):
        out["Q"] = _normal(g, (w.B, w.h, w.n_q, w.d_k), 1.0, dt)
        out["K"] = _normal(g, (w.B, w.h, w.n_k, w.d_k), 1.0, dt)
        out["V"] = _normal(g, (w.B, w.h, w.n_k, w.d_v), 1.0, dt)
        out["scale"] = 1.0 / math.sqrt(w.d_k)
        if w.kind == "bwd":
            out["dO"] = _normal(g, (w.B, w.h, w.n_q, w.d_v), 1.0, dt)
    elif w.kind == "embed":
        out["tokens"] = torch.randint(0, w.vocab, (w.B, w.n_q), generator=g, dtype=torch.int32)
        out["E"] = _normal(g, (w.vocab, w.d_model), 1.0 / math.sqrt(w.d_model), dt)
        out["pos0"] = 0
    elif w.kind == "layer":
        if w.n_q != w.n_k:
            raise ValueError("an encoder layer attends to its own positions (n_q == n_k)")
        D, F = w.d_model, w.d_ff
        std = 1.0 / math.sqrt(D)
        out["X"] = _normal(g, (w.B, w.n_q, D), 1.0, dt)
        out["Wq"] = _normal(g, (D, w.h * w.d_k), std, dt)
        out["Wk"] = _normal(g, (D, w.h * w.d_k), std, dt)
        out["Wv"] = _normal(g, (D, w.h * w.d_v), std, dt)
        out["Wo"] = _normal(g, (w.h * w.d_v, D), std, dt)
        out["ln1_gamma"] = (1.0 + 0.1 * torch.randn((D,), generator=g)).to(dt)
        out["ln1_beta"] = _normal(g, (D,), 0.1, dt)
        out["W1"] = _normal(g, (D, F), std, dt)
        out["b1"] = _normal(g, (F,), 0.1, dt)
        out["W2"] = _normal(g, (F, D), 1.0 / math.sqrt(F), dt)
        out["b2"] = _normal(g, (D,), 0.1, dt)
        out["ln2_gamma"] = (1.0 + 0.1 * torch.randn((D,), generator=g)).to(dt)
        out["ln2_beta"] = _normal(g, (D,), 0.1, dt)
    else:  # "mha" and "mha_bwd"
        std = 1.0 / math.sqrt(w.d_model)
        out["X_q"] = _normal(g, (w.B, w.n_q, w.d_model), 1.0, dt)
        if w.self_attn:
            if w.n_q != w.n_k:
                raise ValueError("self-attention needs n_q == n_k")
            out["X_kv"] = out["X_q"]
        else:
            out["X_kv"] = _normal(g, (w.B, w.n_k, w.d_model), 1.0, dt)
        out["Wq"] = _normal(g, (w.d_model, w.h * w.d_k), std, dt)
        out["Wk"] = _normal(g, (w.d_model, w.h * w.d_k), std, dt)
        out["Wv"] = _normal(g, (w.d_model, w.h * w.d_v), std, dt)
        out["Wo"] = _normal(g, (w.h * w.d_v, w.d_model), std, dt)
        if w.kind == "mha_bwd":
            out["dY"] = _normal(g, (w.B, w.n_q, w.d_model), 1.0, dt)
    if w.mask & MASK_KEY_PADDING:
        lo, hi = w.key_len_range if w.key_len_range else (1, w.n_k)
        out["key_lengths"] = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int32)
    else:
        out["key_lengths"] = None
    return out


def to_f64(t):
    """Exact upcast of a CPU tensor (bf16 or fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
