"""The allocation-free backward (sdpa_backward_noalloc) against sdpa_backward
through the C ABI: two calls in a row, the second smaller, each equal bit for
bit to sdpa_backward's gradients on the same inputs (same kernels; only the
row terms' memory differs: the library's device array instead of a caller
workspace).  Each GPU step prints its case before launching."""

import ctypes

import pytest
import torch

import head_attention_forward_amd as hafa
from head_attention_forward_amd import _binding as bnd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda")


def _case(dev, B, h, n_q, n_k, mask, kl, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    mk = lambda n: torch.randn((B, h, n, 64), generator=g).to(torch.bfloat16).to(dev)  # noqa: E731
    Q, K, V, dO = mk(n_q), mk(n_k), mk(n_k), mk(n_q)
    O, lse = hafa.sdpa_forward_lse(Q, K, V, 0.125, mask, kl)
    return Q, K, V, dO, O, lse


def _grads(dev, L, Q, K, V, dO, O, lse, mask, kl, noalloc):
    B, h, n_q, _ = Q.shape
    n_k = K.shape[2]
    dQ, dK, dV = (torch.full_like(t, float("nan")) for t in (Q, K, V))
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    klp = None if kl is None else ctypes.cast((ctypes.c_int32 * B)(*kl), ctypes.c_void_p)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [P(Q), P(K), P(V), P(O), P(dO), P(lse), P(dQ), P(dK), P(dV), B, h, n_q, n_k, 64, 64,
            0.125, mask, klp, bnd.DTYPE_BF16]
    if noalloc:
        st = L.sdpa_backward_noalloc(*args, stream)
    else:
        nbytes = int(L.sdpa_backward_workspace_bytes(B, h, n_q))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        st = L.sdpa_backward(*args, P(ws), nbytes, stream)
    assert st == 0, bnd.STATUS.get(st, st)
    torch.cuda.synchronize()
    return dQ, dK, dV


def test_noalloc_backward_equals_workspace_backward(dev):
    L = bnd.lib()
    cases = [
        # larger first, then smaller: the second call reuses the same device array
        (3, 4, 640, 640, 3, [640, 333, 1], 11),
        (1, 2, 100, 77, 0, None, 12),
        # padded beyond one launch's 256 batches: two launches per kernel, each
        # with its own rows of the array
        (300, 1, 24, 24, 3, [1 + (i * 5) % 24 for i in range(300)], 13),
    ]
    for B, h, n_q, n_k, mask, kl, seed in cases:
        print("[gpu case] sdpa_backward_noalloc", B, h, n_q, n_k, mask, kl, flush=True)
        Q, K, V, dO, O, lse = _case(dev, B, h, n_q, n_k, mask, kl, seed)
        want = _grads(dev, L, Q, K, V, dO, O, lse, mask, kl, noalloc=False)
        got = _grads(dev, L, Q, K, V, dO, O, lse, mask, kl, noalloc=True)
        for name, g, w in zip(("dQ", "dK", "dV"), got, want):
            assert torch.isfinite(w.float()).all(), name
            assert torch.equal(g, w), f"{name} differs from sdpa_backward"
