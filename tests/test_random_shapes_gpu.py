"""GPU parity on seeded random shapes: bare attention (one and two key
groups per workgroup, and fp32), the multi-head block (one- and
two-heads-per-workgroup fused kernels, the staged path) and the small-batch
decoding step, each against the fp64 oracle within the parity bars (bf16:
max-abs 2e-2, relative L2 5e-3; fp32: max-abs 1e-5).

The shapes come from a fixed numpy generator, so every run checks the same
cases; each case is announced (flushed) before its launch.  Sizes are kept
to what the oracle evaluates in well under a second per case: model widths
equal 64 heads (outputs of order one), and the large-batch block cases use
a small width so that the batch can exceed the compute units."""

import numpy as np
import pytest
import torch

import oracle
import head_attention_forward_amd as hafa
from head_attention_forward_amd.workloads import WORKLOADS, generate, to_f64

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def _close(got, want, what):
    g = to_f64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = g - want
    max_abs = float(np.abs(err).max())
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300))
    print(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, rel)


def _sdpa_cases(n=12, seed=11):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B, h = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        mask = int(rng.integers(0, 4))
        n_q = int(rng.integers(1, 700))
        n_k = n_q if mask & 1 else int(rng.integers(1, 900))
        if B * h * n_q * n_k > 4_000_000:
            continue
        cases.append((B, h, n_q, n_k, mask))
    return cases


def _mha_cases(n=12, seed=12):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        if len(cases) % 3 == 2:
            # more (batch, head) units than compute units: h = 2, d_model = 128
            B, h = int(rng.integers(129, 200)), 2
            nq = int(rng.integers(1, 129))
        else:
            B, h = int(rng.integers(1, 9)), int(rng.integers(1, 9))
            nq = int(rng.integers(1, 300))
        self_attn = bool(rng.integers(0, 2))
        nk = nq if self_attn else int(rng.integers(1, 300 if B < 100 else 129))
        mask = int(rng.integers(0, 4)) if self_attn else 2 * int(rng.integers(0, 2))
        cost = B * (nq + nk) * (64 * h) ** 2 * 3 + B * h * nq * nk * 128
        if cost > 3e8:
            continue
        cases.append((B, h, nq, nk, self_attn, mask))
    return cases


def _decode_cases(n=10, seed=13):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B, h = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        n_q = int(rng.integers(1, 33))
        n_k = int(rng.integers(129, 3000))
        mask = 2 * int(rng.integers(0, 2))
        cases.append((B, h, n_q, n_k, mask))
    return cases


def _key_split_cases(n=8, seed=14):
    """Shapes with at most one 128-query workgroup per compute unit over at
    least 1024 keys (the launch takes two key groups per workgroup)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B, h = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        mask = int(rng.integers(0, 4))
        if mask & 1:  # causal: as many queries as keys
            n_q = n_k = int(rng.integers(1024, 1500))
        else:
            n_q, n_k = int(rng.integers(33, 600)), int(rng.integers(1024, 3000))
        if B * h * n_q * n_k > 6_000_000:
            continue
        cases.append((B, h, n_q, n_k, mask))
    return cases


def _f32_cases(n=8, seed=15):
    """Small fp32 launches (the wave-per-query kernel)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B, h = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        mask = int(rng.integers(0, 4))
        n_q = int(rng.integers(1, 300))
        n_k = n_q if mask & 1 else int(rng.integers(1, 400))
        cases.append((B, h, n_q, n_k, mask))
    return cases


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda")


@pytest.mark.parametrize("B,h,n_q,n_k,mask", _sdpa_cases())
def test_random_sdpa(dev, B, h, n_q, n_k, mask):
    w = WORKLOADS["long_causal_sdpa"].replace(name="random", B=B, h=h, n_q=n_q, n_k=n_k, mask=mask,
                                              key_len_range=None, description="random")
    x = generate(w, seed=B * 7919 + n_q * 31 + n_k)
    kl = x["key_lengths"]
    print(f"[gpu case] sdpa_forward B={B} h={h} n_q={n_q} n_k={n_k} mask={mask} "
          f"kl={None if kl is None else kl.tolist()}", flush=True)
    O = hafa.sdpa_forward(x["Q"].to(dev), x["K"].to(dev), x["V"].to(dev), x["scale"], mask, kl)
    torch.cuda.synchronize()
    want = oracle.sdpa_ref(to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"]), x["scale"], mask,
                           None if kl is None else kl.numpy())
    _close(O, want, f"sdpa {B}x{h}x{n_q}x{n_k} m{mask}")


@pytest.mark.parametrize("B,h,n_q,n_k,self_attn,mask", _mha_cases())
def test_random_mha(dev, B, h, n_q, n_k, self_attn, mask):
    w = WORKLOADS["cross_padded_big"].replace(name="random", B=B, h=h, n_q=n_q, n_k=n_k,
                                              d_model=64 * h, mask=mask, self_attn=self_attn,
                                              key_len_range=None, description="random")
    x = generate(w, seed=B * 104729 + n_q * 31 + n_k)
    kl = x["key_lengths"]
    print(f"[gpu case] mha_forward B={B} h={h} n_q={n_q} n_k={n_k} self={self_attn} mask={mask}",
          flush=True)
    Xq = x["X_q"].to(dev)
    Xkv = Xq if self_attn else x["X_kv"].to(dev)
    Ws = [x[k].to(dev) for k in ("Wq", "Wk", "Wv", "Wo")]
    Y = hafa.mha_forward(Xq, Xkv, *Ws, h, mask, kl)
    torch.cuda.synchronize()
    want = oracle.mha_ref(to_f64(x["X_q"]), to_f64(x["X_kv"]), *[to_f64(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")],
                          h, mask, None if kl is None else kl.numpy())
    _close(Y, want, f"mha {B}x{h}x{n_q}x{n_k} self={self_attn} m{mask}")


@pytest.mark.parametrize("B,h,n_q,n_k,mask", _decode_cases())
def test_random_decode(dev, B, h, n_q, n_k, mask):
    w = WORKLOADS["decode_small_batch_sdpa"].replace(name="random", B=B, h=h, n_q=n_q, n_k=n_k,
                                                     mask=mask, key_len_range=None, description="random")
    x = generate(w, seed=B * 15485863 + n_q * 31 + n_k)
    kl = x["key_lengths"]
    L = hafa.lib().sdpa_decode_launches(B, h, n_q, n_k, mask)
    print(f"[gpu case] sdpa_decode B={B} h={h} n_q={n_q} n_k={n_k} mask={mask} ({L} launches)",
          flush=True)
    O = hafa.sdpa_decode(x["Q"].to(dev), x["K"].to(dev), x["V"].to(dev), x["scale"], mask, kl)
    torch.cuda.synchronize()
    want = oracle.sdpa_ref(to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"]), x["scale"], mask,
                           None if kl is None else kl.numpy())
    _close(O, want, f"decode {B}x{h}x{n_q}x{n_k} m{mask}")


@pytest.mark.parametrize("B,h,n_q,n_k,mask", _key_split_cases())
def test_random_sdpa_key_split(dev, B, h, n_q, n_k, mask):
    w = WORKLOADS["long_causal_sdpa"].replace(name="random", B=B, h=h, n_q=n_q, n_k=n_k, mask=mask,
                                              key_len_range=None, description="random")
    x = generate(w, seed=B * 131 + n_q * 31 + n_k)
    kl = x["key_lengths"]
    print(f"[gpu case] sdpa_forward key split B={B} h={h} n_q={n_q} n_k={n_k} mask={mask} "
          f"kl={None if kl is None else kl.tolist()}", flush=True)
    O = hafa.sdpa_forward(x["Q"].to(dev), x["K"].to(dev), x["V"].to(dev), x["scale"], mask, kl)
    torch.cuda.synchronize()
    want = oracle.sdpa_ref(to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"]), x["scale"], mask,
                           None if kl is None else kl.numpy())
    _close(O, want, f"sdpa key split {B}x{h}x{n_q}x{n_k} m{mask}")


@pytest.mark.parametrize("B,h,n_q,n_k,mask", _f32_cases())
def test_random_sdpa_f32(dev, B, h, n_q, n_k, mask):
    w = WORKLOADS["sdpa_f32_tiny"].replace(name="random", B=B, h=h, n_q=n_q, n_k=n_k, mask=mask,
                                           key_len_range=None, description="random")
    x = generate(w, seed=B * 17 + n_q * 31 + n_k)
    kl = x["key_lengths"]
    print(f"[gpu case] sdpa_forward fp32 B={B} h={h} n_q={n_q} n_k={n_k} mask={mask}", flush=True)
    O = hafa.sdpa_forward(x["Q"].to(dev), x["K"].to(dev), x["V"].to(dev), x["scale"], mask, kl)
    torch.cuda.synchronize()
    want = oracle.sdpa_ref(to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"]), x["scale"], mask,
                           None if kl is None else kl.numpy())
    g = to_f64(O)
    assert np.all(np.isfinite(g))
    err = float(np.abs(g - want).max())
    print(f"  fp32 {B}x{h}x{n_q}x{n_k} m{mask}: max_abs={err:.3e}", flush=True)
    assert err <= 1e-5, err
