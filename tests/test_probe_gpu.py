"""GPU checks of the measurement aids (include/mha_probe.h): the byte mover
writes a ^ b ^ c bit for bit, and every workgroup of the matrix-core probe
writes the same finite values (equal to the product chain's closed form for
one product, up to the order of the fp32 sums)."""

import ctypes

import numpy as np
import pytest
import torch

import head_attention_forward_amd as hafa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda")


def test_floor_probe_xor3(dev):
    print("[gpu case] floor probe: empty kernel and xor3 over 64 KiB", flush=True)
    g = torch.Generator("cpu").manual_seed(3)
    a, b, c = (torch.randint(-2**31, 2**31 - 1, (16384,), generator=g, dtype=torch.int32).to(dev)
               for _ in range(3))
    d = torch.empty_like(a)
    P = ctypes.c_void_p
    L = hafa.lib()
    assert L.mha_floor_probe(0, None, None, None, None, 0, 64, None) == 0
    assert L.mha_floor_probe(1, P(a.data_ptr()), P(b.data_ptr()), P(c.data_ptr()), P(d.data_ptr()),
                             a.numel() * 4, 7, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(d, a ^ b ^ c)


def _operand(mode, l, j, which):
    """The probe's operand j of lane l (which = 0: A, 1: B) as a float, from
    its definition: mode 1 the multiple of 1/1024 given by the lane pattern;
    mode 0 sign, exponent (2^-2 .. 2^0) and 7 mantissa bits taken from a
    multiplicative hash of (l, j, which)."""
    if mode == 1:
        v = ((l + j) & 15) if which == 0 else ((3 * l + j) & 15)
        return v / 1024.0
    M = 0xFFFFFFFF
    x = ((l * 64 + j * 8 + which) * 2654435761) & M
    x ^= x >> 15
    x = (x * 2246822519) & M
    x ^= x >> 13
    sign = -1.0 if (x >> 31) & 1 else 1.0
    e = ((x >> 7) % 3) - 2
    return sign * (1.0 + (x & 0x7F) / 128.0) * 2.0 ** e


@pytest.mark.parametrize("mode", [0, 1])
def test_mfma_probe(dev, mode):
    print(f"[gpu case] matrix-core probe: operand mode {mode}, 40 workgroups, 3 products per chain",
          flush=True)
    grid, iters = 40, 3
    sink = torch.full((grid, 256), float("nan"), dtype=torch.float32, device=dev)
    assert hafa.lib().mha_mfma_probe(mode, grid, iters, ctypes.c_void_p(sink.data_ptr()), None) == 0
    torch.cuda.synchronize()
    s = sink.cpu()
    assert bool(torch.isfinite(s).all())
    assert bool((s == s[0:1]).all())
    # Closed form.  Lane l of a wave holds A row (l % 32), k = 8 (l / 32) + j
    # (j = 0..7), and B column (l % 32) at the same k; each of the four chains
    # accumulates iters copies of C = A B (32 x 32), and thread t sums its 16
    # accumulators over the four chains: C[i][n] for the rows
    # 8 (r / 4) + 4 (l / 32) + r % 4 of column n = l % 32.
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for l in range(64):
        for j in range(8):
            k = 8 * (l // 32) + j
            A[l % 32, k] = _operand(mode, l, j, 0)
            Bm[k, l % 32] = _operand(mode, l, j, 1)
    C = A @ Bm
    want = np.zeros(256)
    for t in range(256):
        l = t % 64
        rows = [8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)]
        want[t] = 4 * iters * sum(C[i, l % 32] for i in rows)
    # fp32 sums of up to 16 * 4 * 3 products of order one
    np.testing.assert_allclose(s[0].numpy().astype(np.float64), want, rtol=1e-4, atol=1e-3)
