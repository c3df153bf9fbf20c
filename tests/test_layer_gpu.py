"""GPU parity of the encoder-layer entry points (residual + LayerNorm, the
position-wise FFN, the whole Post-LN layer) against the fp64 oracle, through
the C ABI.

Tolerance (bf16 in and out, fp32 arithmetic): every element within
2e-2 + 2u |want| of the oracle, u = 2^-8 the unit roundoff of bf16, and
relative L2 error <= 5e-3.  The 2e-2 is the attention outputs' bar; the
2u |want| term is there because these outputs are not bounded by the
inputs' scale: a LayerNorm output of magnitude 5 already carries up to
u * 5 = 0.02 of error from its own rounding to bf16, and the bf16-rounded
intermediates it is computed from (the sublayer output, x1, the FFN hidden
layer) add about as much again.

Each GPU step prints the case it runs (flushed) before launching it."""

import numpy as np
import pytest
import torch

import oracle
import head_attention_forward_amd as hafa
from head_attention_forward_amd import _binding as bnd
from head_attention_forward_amd.workloads import WORKLOADS, generate, to_f64

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8
ATOL = 2e-2
RTOL = 2 * U_BF16
REL_L2 = 5e-3


def announce(*what):
    print("[gpu case]", *what, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda")


def assert_close(got, want, what=""):
    g = to_f64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - want)
    bound = ATOL + RTOL * np.abs(want)
    worst = float((err / bound).max())
    rel = float(np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-300))
    print(f"  {what}: max_abs={float(err.max()):.3e} worst/bound={worst:.3f} rel_l2={rel:.3e}",
          flush=True)
    assert worst <= 1.0, f"{what}: an element is outside {ATOL} + {RTOL} |want| ({worst:.3f}x)"
    assert rel <= REL_L2, f"{what}: rel-L2 {rel}"


def _gen(seed):
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    return g


def _bf(g, shape, std=1.0, mean=0.0):
    return (torch.randn(shape, generator=g) * std + mean).to(torch.bfloat16)


# ------------------------------------------------------------------ residual + LayerNorm

LN_CASES = [
    # M, d, eps, x_mean, label
    (3200, 512, 1e-5, 0.0, "the encoder layer's rows"),
    (1, 8, 1e-5, 0.0, "one row of one chunk"),
    (7, 520, 1e-5, 0.0, "second chunk of a lane partly used"),
    (33, 1000, 0.0, 0.0, "eps = 0, ragged width"),
    (5, 4096, 1e-5, 0.0, "widest row"),
    (64, 512, 1e-5, 40.0, "rows far from zero mean (two-pass variance)"),
    (1001, 72, 1e-5, 0.0, "narrow rows, ragged row count"),
]


@pytest.mark.parametrize("M,d,eps,x_mean,label", LN_CASES)
def test_add_layernorm(dev, M, d, eps, x_mean, label):
    g = _gen(M * 7 + d)
    X = _bf(g, (M, d), 1.0, x_mean)
    F = _bf(g, (M, d), 0.7)
    gamma = (1.0 + 0.1 * torch.randn((d,), generator=g)).to(torch.bfloat16)
    beta = _bf(g, (d,), 0.1)
    announce("add_layernorm", M, d, eps, label)
    Y = hafa.add_layernorm_forward(X.to(dev), F.to(dev), gamma.to(dev), beta.to(dev), eps)
    torch.cuda.synchronize()
    want = oracle.add_layer_norm(to_f64(X), to_f64(F), to_f64(gamma), to_f64(beta), eps)
    assert_close(Y, want, f"LN {label}")


def test_add_layernorm_in_place_and_constant_rows(dev):
    """Y may be X or F; a row whose sum is constant normalises to beta."""
    g = _gen(5)
    M, d = 96, 512
    X = _bf(g, (M, d))
    F = _bf(g, (M, d))
    X[3] = 2.5
    F[3] = -0.5
    gamma = (1.0 + 0.1 * torch.randn((d,), generator=g)).to(torch.bfloat16)
    beta = _bf(g, (d,), 0.1)
    Xd, Fd, gd, bd = X.to(dev), F.to(dev), gamma.to(dev), beta.to(dev)
    announce("add_layernorm in place", M, d)
    ref = hafa.add_layernorm_forward(Xd, Fd, gd, bd, 1e-5)
    x_copy, f_copy = Xd.clone(), Fd.clone()
    hafa.add_layernorm_forward(x_copy, Fd, gd, bd, 1e-5, out=x_copy)
    hafa.add_layernorm_forward(Xd, f_copy, gd, bd, 1e-5, out=f_copy)
    torch.cuda.synchronize()
    assert torch.equal(x_copy, ref) and torch.equal(f_copy, ref)
    assert torch.equal(ref[3].cpu(), beta)
    want = oracle.add_layer_norm(to_f64(X), to_f64(F), to_f64(gamma), to_f64(beta), 1e-5)
    assert_close(ref, want, "LN in place")


# ------------------------------------------------------------------ feed-forward network

FFN_CASES = [
    # M, d_model, d_ff, b1_mean, label
    (3200, 512, 2048, 0.0, "the base model's FFN on the encoder layer's rows"),
    (1, 64, 64, 0.0, "one row"),
    (77, 72, 200, 0.0, "ragged rows, widths not multiples of 64"),
    (129, 512, 2048, -2.0, "most hidden units below zero (ReLU)"),
    (256, 1024, 4096, 0.0, "the big model's FFN widths"),
]


@pytest.mark.parametrize("M,d_model,d_ff,b1_mean,label", FFN_CASES)
def test_ffn(dev, M, d_model, d_ff, b1_mean, label):
    g = _gen(M + d_model + d_ff)
    X = _bf(g, (M, d_model))
    W1 = _bf(g, (d_model, d_ff), d_model ** -0.5)
    b1 = _bf(g, (d_ff,), 0.1, b1_mean)
    W2 = _bf(g, (d_ff, d_model), d_ff ** -0.5)
    b2 = _bf(g, (d_model,), 0.1)
    announce("ffn", M, d_model, d_ff, label)
    Y = hafa.ffn_forward(*(t.to(dev) for t in (X, W1, b1, W2, b2)))
    torch.cuda.synchronize()
    want = oracle.ffn(to_f64(X), to_f64(W1), to_f64(b1), to_f64(W2), to_f64(b2))
    assert_close(Y, want, f"FFN {label}")
    if b1_mean < 0:
        hidden = to_f64(X) @ to_f64(W1) + to_f64(b1)
        assert (hidden < 0).mean() > 0.9  # the case exercises the ReLU


# ------------------------------------------------------------------ encoder layer

def _layer_ref(x, w, kl):
    p = [to_f64(x[k]) for k in bnd.LAYER_PARAMS]
    return oracle.encoder_layer_ref(to_f64(x["X"]), *p[:4], w.h, *p[4:], w.eps, w.mask,
                                    None if kl is None else np.asarray(kl))


def _layer_gpu(dev, x, w):
    params = {k: x[k].to(dev) for k in bnd.LAYER_PARAMS}
    return hafa.encoder_layer_forward(x["X"].to(dev), params, w.h, w.eps, w.mask, x["key_lengths"])


LAYER_CASES = [
    # overrides of the base encoder layer, label
    (dict(), "encoder layer, base model, B=32 n=100"),
    (dict(B=3, n_q=37, n_k=37, d_model=128, h=2, d_ff=264), "ragged small layer"),
    (dict(B=4, mask=2, key_len_range=(1, 100)), "padded source sentences"),
    (dict(B=2, n_q=129, n_k=129), "n = 129 (unfused projection plan)"),
    (dict(B=2, n_q=50, n_k=50, d_model=72, h=1, d_ff=136), "d_model 72 (not a multiple of 64)"),
    (dict(B=2, n_q=64, n_k=64, mask=1), "causal self-attention"),
    (dict(B=1, n_q=7, n_k=7, d_model=256, h=4, d_ff=128), "7 rows, d_model 256"),
    (dict(B=2, n_q=40, n_k=40, d_model=1024, h=16, d_ff=256), "d_model 1024 (the big model's width)"),
]


@pytest.mark.parametrize("over,label", LAYER_CASES)
def test_encoder_layer(dev, over, label):
    w = WORKLOADS["encoder_layer_base"].replace(**over)
    x = generate(w, seed=3)
    announce("encoder_layer", label, w.B, w.n_q, w.d_model, w.h, w.d_ff, w.mask,
             None if x["key_lengths"] is None else x["key_lengths"].tolist())
    Y = _layer_gpu(dev, x, w)
    torch.cuda.synchronize()
    assert_close(Y, _layer_ref(x, w, x["key_lengths"]), label)


@pytest.mark.parametrize("B,n", [(4, 100), (3, 77)])
def test_encoder_layer_equals_its_entry_points(dev, B, n):
    """The layer is mha_forward, add_layernorm_forward, ffn_forward,
    add_layernorm_forward on one stream: bit-identical results (also for a
    row count, 231, that no tile size divides)."""
    w = WORKLOADS["encoder_layer_base"].replace(B=B, n_q=n, n_k=n)
    x = generate(w, seed=4)
    d = {k: v.to(dev) for k, v in x.items() if v is not None}
    announce("encoder_layer vs entry points", w.B, w.n_q)
    Y = _layer_gpu(dev, x, w)
    A = hafa.mha_forward(d["X"], d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], w.h, w.mask)
    x1 = hafa.add_layernorm_forward(d["X"], A, d["ln1_gamma"], d["ln1_beta"], w.eps)
    F = hafa.ffn_forward(x1, d["W1"], d["b1"], d["W2"], d["b2"])
    Y2 = hafa.add_layernorm_forward(x1, F, d["ln2_gamma"], d["ln2_beta"], w.eps)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    # and the first sublayer alone against the oracle's intermediate x1
    _, inter = oracle.encoder_layer_ref(to_f64(x["X"]), *[to_f64(x[k]) for k in bnd.LAYER_PARAMS[:4]],
                                        w.h, *[to_f64(x[k]) for k in bnd.LAYER_PARAMS[4:]], w.eps,
                                        w.mask, None, return_intermediates=True)
    assert_close(x1, inter["x1"], "x1 = LN1(X + MultiHead(X))")


def test_encoder_layer_timed_launches(dev):
    """The instrumented variant launches encoder_layer_launches kernels and
    gives the same output."""
    import ctypes
    from head_attention_forward_amd import _hip
    w = WORKLOADS["encoder_layer_base"].replace(B=2)
    x = generate(w, seed=6)
    params = {k: x[k].to(dev) for k in bnd.LAYER_PARAMS}
    X = x["X"].to(dev)
    announce("encoder_layer timed", w.B, w.n_q)
    Y = hafa.encoder_layer_forward(X, params, w.h, w.eps)
    L = bnd.lib()
    nl = L.encoder_layer_launches(w.n_q, w.d_model)
    assert nl == 6
    Y2 = torch.empty_like(Y)
    nbytes = hafa.encoder_layer_workspace_bytes(w.B, w.n_q, w.d_model, w.h, 64, 64, w.d_ff)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    pool = _hip.EventPool(2 * nl)
    n = ctypes.c_int()
    P = ctypes.c_void_p
    st = L.encoder_layer_forward_timed(
        P(X.data_ptr()), *[P(params[k].data_ptr()) for k in bnd.LAYER_PARAMS], P(Y2.data_ptr()),
        w.B, w.n_q, w.d_model, w.h, 64, 64, w.d_ff, w.eps, 0, None, bnd.DTYPE_BF16,
        P(ws.data_ptr()), nbytes, P(torch.cuda.current_stream().cuda_stream), pool.ptr(0), 2 * nl,
        ctypes.byref(n))
    torch.cuda.synchronize()
    assert st == 0 and n.value == nl
    assert torch.equal(Y, Y2)
    for i in range(nl):
        assert pool.elapsed_ms(2 * i, 2 * i + 1) > 0
    pool.close()
