"""GPU parity of the training entry points: sdpa_forward_lse (the forward
with its row log-sum-exp) and sdpa_backward (dQ, dK, dV) against the fp64
oracle, through the C ABI.

Tolerances.  lse: the forward normalises by the sum of its weights rounded
to bf16 (relative error of each weight <= u = 2^-8, of the sum at most the
same), so |lse - exact| <= u + 1e-6 (ln(1 + u) < u).  Gradients: inputs and
outputs bf16, fp32 accumulation, and one bf16 rounding of P (dV) or dS
(dQ, dK) as it enters the accumulating product, plus the output rounding:
each gradient within relative L2 error 2u = 7.8e-3 of the exact one, and
every element within 4u * max(max|exact|, 1) of it (elements of a gradient
are sums of terms of both signs, so the bar is set on the tensor's scale,
at least the unit scale of the inputs).

Each GPU step prints the case it runs (flushed) before launching it."""

import numpy as np
import pytest
import torch

import oracle
import head_attention_forward_amd as hafa
from head_attention_forward_amd.workloads import to_f64

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def announce(*what):
    print("[gpu case]", *what, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda")


def inputs(B, h, n_q, n_k, seed):
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    mk = lambda n: torch.randn((B, h, n, 64), generator=g).to(torch.bfloat16)  # noqa: E731
    return mk(n_q), mk(n_k), mk(n_k), mk(n_q)


def check_grad(got, want, what):
    """A gradient that is exactly zero (one visible key: the softmax is
    constant) is held to the elementwise bar on the inputs' unit scale."""
    g = to_f64(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - want)
    scale = max(float(np.abs(want).max()), 1.0)
    worst = float(err.max()) / (4 * U * scale)
    norm = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(g - want) / norm) if norm > 0 else 0.0
    print(f"  {what}: rel_l2={rel:.2e} max_abs={float(err.max()):.2e} "
          f"(max|want| {float(np.abs(want).max()):.2e}, worst/bound {worst:.3f})", flush=True)
    assert rel <= 2 * U, f"{what}: rel-L2 {rel}"
    assert worst <= 1.0, f"{what}: max-abs {float(err.max())}"


CASES = [
    # B, h, n_q, n_k, mask, key_lengths, label
    (2, 4, 128, 128, 0, None, "one block each, unmasked"),
    (2, 2, 256, 256, 1, None, "causal"),
    (2, 3, 96, 160, 2, [160, 37], "key padding, cross shape"),
    (3, 2, 100, 77, 0, None, "ragged query and key tiles"),
    (2, 2, 200, 200, 3, [200, 150], "causal + key padding"),
    (1, 1, 1, 1, 0, None, "one query, one key"),
    (1, 2, 1, 300, 0, None, "one query over 300 keys"),
    (4, 8, 100, 100, 0, None, "the encoder block's heads"),
    # more padded batches than one launch carries lengths for (two launches per kernel)
    (300, 1, 20, 20, 3, [1 + (i * 7) % 20 for i in range(300)], "300 padded batches"),
    # forwards whose workgroups split the keys over two or four groups of waves
    (1, 2, 200, 1500, 0, None, "two key groups in the forward"),
    (1, 2, 1100, 1100, 1, None, "causal, two key groups in the forward"),
    (1, 2, 300, 2500, 2, [2500], "four key groups in the forward"),
]


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl,label", CASES)
def test_backward(dev, B, h, n_q, n_k, mask, kl, label):
    Q, K, V, dO = inputs(B, h, n_q, n_k, seed=B * 1000 + n_q + n_k + mask)
    scale = 1.0 / 8.0
    announce("backward", B, h, n_q, n_k, mask, kl, label)
    Qd, Kd, Vd, dOd = (t.to(dev) for t in (Q, K, V, dO))
    O, lse = hafa.sdpa_forward_lse(Qd, Kd, Vd, scale, mask, kl)
    dQ, dK, dV = hafa.sdpa_backward(Qd, Kd, Vd, O, dOd, lse, scale, mask, kl)
    torch.cuda.synchronize()
    kla = None if kl is None else np.array(kl)
    args = [to_f64(t) for t in (Q, K, V)]
    want_lse = oracle.row_logsumexp(args[0], args[1], scale, mask, kla)
    lerr = float(np.abs(to_f64(lse) - want_lse).max())
    print(f"  lse max_abs={lerr:.2e}", flush=True)
    assert lerr <= U + 1e-6
    # The backward is checked against the oracle's gradients at the GPU's own
    # forward output (the identity D = rowsum(dO * O) uses O; the oracle's
    # gradient formula uses P only, so the exact gradients are what is compared).
    wQ, wK, wV = oracle.sdpa_backward_ref(*args, to_f64(dO), scale, mask, kla)
    check_grad(dQ, wQ, f"dQ {label}")
    check_grad(dK, wK, f"dK {label}")
    check_grad(dV, wV, f"dV {label}")
    if kl is not None:
        for b, L in enumerate(kl):
            assert torch.count_nonzero(dK[b, :, L:]) == 0 and torch.count_nonzero(dV[b, :, L:]) == 0


def test_forward_lse_leaves_output_unchanged(dev):
    Q, K, V, _ = inputs(2, 4, 300, 300, seed=5)
    Qd, Kd, Vd = (t.to(dev) for t in (Q, K, V))
    announce("forward with lse vs plain forward", 2, 4, 300)
    O1 = hafa.sdpa_forward(Qd, Kd, Vd, 0.125, 1)
    O2, _ = hafa.sdpa_forward_lse(Qd, Kd, Vd, 0.125, 1)
    Qs = Qd[:, :, :1].contiguous()
    # a decode shape (one query over many keys) takes the key-split kernel
    O3 = hafa.sdpa_forward(Qs, Kd, Vd, 0.125, 0)
    O4, l4 = hafa.sdpa_forward_lse(Qs, Kd, Vd, 0.125, 0)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(O3, O4)
    want = oracle.row_logsumexp(to_f64(Q[:, :, :1]), to_f64(K), 0.125, 0, None)
    assert float(np.abs(to_f64(l4) - want).max()) <= U + 1e-6


def test_backward_deterministic(dev):
    Q, K, V, dO = inputs(2, 2, 384, 384, seed=7)
    Qd, Kd, Vd, dOd = (t.to(dev) for t in (Q, K, V, dO))
    announce("backward determinism", 2, 2, 384)
    O, lse = hafa.sdpa_forward_lse(Qd, Kd, Vd, 0.125, 1)
    r1 = hafa.sdpa_backward(Qd, Kd, Vd, O, dOd, lse, 0.125, 1)
    r2 = hafa.sdpa_backward(Qd, Kd, Vd, O, dOd, lse, 0.125, 1)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_backward_long_causal(dev):
    """B = 1, h = 2, n = 2048, causal: the whole gradients against the
    oracle (fp64 over 2 x 2048 x 2048 weights)."""
    Q, K, V, dO = inputs(1, 2, 2048, 2048, seed=11)
    Qd, Kd, Vd, dOd = (t.to(dev) for t in (Q, K, V, dO))
    announce("backward long causal", 1, 2, 2048)
    O, lse = hafa.sdpa_forward_lse(Qd, Kd, Vd, 0.125, 1)
    dQ, dK, dV = hafa.sdpa_backward(Qd, Kd, Vd, O, dOd, lse, 0.125, 1)
    torch.cuda.synchronize()
    wQ, wK, wV = oracle.sdpa_backward_ref(*(to_f64(t) for t in (Q, K, V, dO)), 0.125, 1, None)
    check_grad(dQ, wQ, "dQ long causal")
    check_grad(dK, wK, "dK long causal")
    check_grad(dV, wV, "dV long causal")


# ------------------------------------------------------------------ the block's gradients

def check_block_grad(got, want, what):
    """Block gradients pass through more bf16 roundings (the per-head upstream
    gradient, the concatenated dQ/dK/dV, the GEMM outputs): relative L2 <= 4u
    and every element within 8u * max|exact|."""
    g = to_f64(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - want)
    scale = max(float(np.abs(want).max()), 1e-30)
    rel = float(np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-300))
    worst = float(err.max()) / (8 * U * scale)
    print(f"  {what}: rel_l2={rel:.2e} worst/bound {worst:.3f}", flush=True)
    assert rel <= 4 * U, f"{what}: rel-L2 {rel}"
    assert worst <= 1.0, f"{what}: max-abs {float(err.max())}"


BLOCK_CASES = [
    # B, n_q, n_k, d_model, h, self_attn, mask, key_lengths, label
    (4, 100, 100, 512, 8, True, 0, None, "encoder self-attention (fused forward shape)"),
    (2, 256, 256, 512, 8, True, 1, None, "causal self-attention"),
    (4, 96, 128, 256, 4, False, 2, [128, 64, 100, 1], "cross-attention, key padding"),
    (8, 7, 9, 128, 2, False, 0, None, "tiny ragged cross-attention (B n multiples of 8)"),
    (4, 30, 30, 72, 1, True, 1, None, "d_model 72: grouped GEMM jobs with 72 columns"),
]


@pytest.mark.parametrize("B,n_q,n_k,dm,h,self_attn,mask,kl,label", BLOCK_CASES)
def test_mha_backward(dev, B, n_q, n_k, dm, h, self_attn, mask, kl, label):
    g = torch.Generator("cpu")
    g.manual_seed(B + n_q + dm)
    Xq = torch.randn((B, n_q, dm), generator=g).to(torch.bfloat16)
    Xkv = Xq if self_attn else torch.randn((B, n_k, dm), generator=g).to(torch.bfloat16)
    Ws = [(torch.randn((dm, h * 64), generator=g) / dm ** 0.5).to(torch.bfloat16) for _ in range(3)]
    Ws.append((torch.randn((h * 64, dm), generator=g) / (h * 64) ** 0.5).to(torch.bfloat16))
    dY = torch.randn((B, n_q, dm), generator=g).to(torch.bfloat16)
    announce("mha backward", B, n_q, n_k, dm, h, self_attn, mask, kl, label)
    Xqd = Xq.to(dev)
    Xkvd = Xqd if self_attn else Xkv.to(dev)
    Wd = [w.to(dev) for w in Ws]
    Y, state = hafa.mha_forward_train(Xqd, Xkvd, *Wd, h, mask, kl)
    Y0 = hafa.mha_forward(Xqd, Xkvd, *Wd, h, mask, kl)
    grads = hafa.mha_backward(Xqd, Xkvd, *Wd, h, dY.to(dev), state, mask, kl)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0)  # the training forward gives the same output
    kla = None if kl is None else np.array(kl)
    want = oracle.mha_backward_ref(to_f64(Xq), to_f64(Xkv), *[to_f64(w) for w in Ws], h, to_f64(dY),
                                   mask, kla)
    if self_attn:
        assert grads[1] is None
        check_block_grad(grads[0], want[0] + want[1], f"dX {label}")
    else:
        check_block_grad(grads[0], want[0], f"dX_q {label}")
        check_block_grad(grads[1], want[1], f"dX_kv {label}")
    for name, gt, wt in zip(("dWq", "dWk", "dWv", "dWo"), grads[2:], want[2:]):
        check_block_grad(gt, wt, f"{name} {label}")


def test_key_range_past_32bit_byte_offsets(dev):
    """One head with 2^25 + 37 keys (4.3 GB of K): the last, ragged key tile
    starts at byte 2^32 of the head's K and V.  Every query has q[0] = 64;
    the first 2^25 keys are (-64, 0, ..., 0), score -512, so their weights
    are below e^-500 and exactly zero in fp32; the last 37 keys are ordinary
    (N(0,1), first component 0).  The forward output, the forward's lse and
    the gradients therefore equal the oracle's on those 37 keys alone, and
    every other key's gradient is exactly zero.  Copies addressed with 32-bit
    byte offsets from the head's first row would read the first rows of the
    buffer for the last tile instead."""
    n_k = (1 << 25) + 37
    tail = 37
    announce("key range past 32-bit byte offsets", n_k)
    K = torch.zeros((1, 1, n_k, 64), dtype=torch.bfloat16, device=dev)
    V = torch.zeros((1, 1, n_k, 64), dtype=torch.bfloat16, device=dev)
    K[:, :, : n_k - tail, 0] = -64.0
    g = torch.Generator("cpu")
    g.manual_seed(25)
    Kt = torch.randn((1, 1, tail, 64), generator=g).to(torch.bfloat16)
    Kt[..., 0] = 0.0
    Vt = torch.randn((1, 1, tail, 64), generator=g).to(torch.bfloat16)
    K[:, :, n_k - tail:] = Kt.to(dev)
    V[:, :, n_k - tail:] = Vt.to(dev)
    for n_q in (1, 40, 64):  # the few-query kernel, then the streaming kernel
        Q = torch.randn((1, 1, n_q, 64), generator=g).to(torch.bfloat16)
        Q[..., 0] = 64.0
        dO = torch.randn((1, 1, n_q, 64), generator=g).to(torch.bfloat16)
        print(f"  n_q={n_q}", flush=True)
        Qd = Q.to(dev)
        O = hafa.sdpa_forward(Qd, K, V, 0.125, 0)
        torch.cuda.synchronize()
        args = [to_f64(t) for t in (Q, Kt, Vt)]
        want = oracle.sdpa_ref(*args, 0.125, 0, None)
        got = to_f64(O.cpu())
        assert float(np.abs(got - want).max()) <= 2e-2, "forward"
        if n_q != 64:
            continue
        O2, lse = hafa.sdpa_forward_lse(Qd, K, V, 0.125, 0)
        dQ, dK, dV = hafa.sdpa_backward(Qd, K, V, O2, dO.to(dev), lse, 0.125, 0)
        torch.cuda.synchronize()
        assert torch.equal(O2, O)
        assert float(np.abs(to_f64(lse.cpu()) - oracle.row_logsumexp(args[0], args[1], 0.125, 0, None)).max()) <= U + 1e-6
        assert int(torch.count_nonzero(dK[:, :, : n_k - tail])) == 0
        assert int(torch.count_nonzero(dV[:, :, : n_k - tail])) == 0
        wQ, wK, wV = oracle.sdpa_backward_ref(*args, to_f64(dO), 0.125, 0, None)
        check_grad(dQ.cpu(), wQ, "dQ past 2^32 bytes")
        check_grad(dK[:, :, n_k - tail:].cpu(), wK, "dK past 2^32 bytes")
        check_grad(dV[:, :, n_k - tail:].cpu(), wV, "dV past 2^32 bytes")
    del K, V
    torch.cuda.empty_cache()
