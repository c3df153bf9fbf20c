"""Reference oracle for multi-head scaled dot-product attention (forward).

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU implementation of what the GPU library computes.  It exists to prove the
GPU path right; it is never a fallback.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``head_attention_forward_amd`` and imports
nothing from it (inputs are handed in as arrays).

Two independent formulations are provided:

* ``oracle.attention``  -- numpy, float64, the matrix form of the definition
  (projections, per-head scores, additive mask, row softmax, weighted sum of
  values, concat, output projection), one function per step;
  ``oracle.layer`` -- the same for residual + LayerNorm and the
  position-wise feed-forward network of an encoder layer;
  ``oracle.embedding`` -- the scaled token embedding plus the sinusoidal
  positional encoding;
  ``oracle.backward`` -- the gradients of attention (dQ, dK, dV), of the
  multi-head block (inputs and the four projection weights) and the row
  log-sum-exp a forward pass saves for them.
* ``oracle.bruteforce`` -- pure-Python loops with ``math.exp``/``math.fsum``,
  one query row at a time, for tiny inputs; it cross-checks the matrix form.

Sources (page title and section; the pages are the authority on what is
computed):

* hex4c59.cc, "读懂 Attention Is All You Need：从一次加权求和到完整 Transformer"
  (an explainer of the 2017 paper): sections "Q、K、V 是三种计算角色",
  "六步算完一行注意力", "把所有位置合并，就是那条核心公式",
  "为什么要按键的维度缩放？", "多头注意力让一次读取有多组投影",
  "解码器有两种读取：看前缀，以及看源句", "掩码必须在 softmax 之前生效",
  "用几十行代码核对刚才的数值".
* research-heat.pages.dev, "做法 · Attention Is All You Need": sections
  "点积随维度增大，因而除以根号", "一次平均不够，因而切开多头",
  "解码器不能看见尚未写出的词，因而加遮罩".
* devpress.csdn.net, "【深度学习】Transformer（Attention Is All You Need）":
  section 2.1 equations (2.1)-(2.4), section 2.2 (multi-head formula and
  shapes of W_i^Q, W_i^K, W_i^V, W^O), section 3.1 (causal mask print),
  section 3.2 (cross-attention).
* wiki.hugogu.cn, "Attention Is All You Need" notes: the masked
  self-attention paragraph and the table of the three attention uses.
* For the rest of the encoder layer (``oracle.layer``): hex4c59.cc sections
  "前馈网络为什么放在注意力后面？" and "Add & Norm 里究竟发生了什么？";
  devpress.csdn.net section 2.3 (encoder block order, FFN formula).
* For the input side (``oracle.embedding``): devpress.csdn.net section 4
  (equation (4.1), Table 4.1, the worked example, the shift identity);
  hex4c59.cc section "没有循环，模型怎样知道词序？".
* For the backward pass (``oracle.backward``): hex4c59.cc sections
  "训练能并行，不意味着一次生成整句话" and "参数是怎样学出来的？"; the
  gradients are those of devpress.csdn.net section 2.1 equation (2.4).

Parity status of every function is stated in its docstring.  All functions
are pinned by ``tests/test_oracle.py`` (printed values from the pages,
closed forms, invariants, brute force, and a library cross-check).
"""

from .attention import (  # noqa: F401
    MASK_NONE,
    MASK_CAUSAL,
    MASK_KEY_PADDING,
    MASK_CAUSAL_KEY_PADDING,
    additive_mask,
    attention_weights,
    mha_ref,
    project,
    scaled_scores,
    sdpa_ref,
    sdpa_ref_rows,
    softmax_rows,
    split_heads,
    concat_heads,
)
from .bruteforce import (  # noqa: F401
    attention_bruteforce,
    embed_positional_bruteforce,
    ffn_bruteforce,
    layer_norm_bruteforce,
    mha_bruteforce,
)
from .backward import mha_backward_ref, row_logsumexp, sdpa_backward_ref  # noqa: F401
from .embedding import embed_positional_ref, positional_encoding  # noqa: F401
from .layer import add_layer_norm, encoder_layer_ref, ffn, layer_norm  # noqa: F401
