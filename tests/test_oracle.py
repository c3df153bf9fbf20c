"""The oracle against its pins (CPU only).

Every check is defined in ``oracle_pins.py`` with the passage or the
mathematical fact it rests on; here they run against the oracle itself."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_SDPA_CHECKS, ids=lambda f: f.__name__)
def test_sdpa_pin(check):
    check(oracle)


@pytest.mark.parametrize("check", pins.ALL_BWD_CHECKS, ids=lambda f: f.__name__)
def test_bwd_pin(check):
    check(oracle)


@pytest.mark.parametrize("check", pins.ALL_EMBED_CHECKS, ids=lambda f: f.__name__)
def test_embed_pin(check):
    check(oracle)


def test_embedding_rejects_ids_outside_the_vocabulary():
    with pytest.raises(ValueError):
        oracle.embed_positional_ref(np.array([[0, 5]]), np.zeros((5, 4)))
    with pytest.raises(ValueError):
        oracle.embed_positional_ref(np.array([[-1]]), np.zeros((5, 4)))


@pytest.mark.parametrize("check", pins.ALL_LAYER_CHECKS, ids=lambda f: f.__name__)
def test_layer_pin(check):
    check(oracle)


@pytest.mark.parametrize("check", pins.ALL_MHA_CHECKS, ids=lambda f: f.__name__)
def test_mha_pin(check):
    check(oracle)


def test_rows_subset_matches_full():
    """sdpa_ref_rows evaluates the same definition row by row."""
    r = np.random.default_rng(20)
    B, h, n, d = 2, 3, 13, 8
    Q, K, V = (r.standard_normal((B, h, n, d)) for _ in range(3))
    kl = np.array([5, 13])
    for kind in (0, 1, 2, 3):
        full = oracle.sdpa_ref(Q, K, V, 0.35, kind, kl if kind & 2 else None)
        idx = np.array([(b, hh, q) for b in range(B) for hh in range(h) for q in range(0, n, 3)])
        part = oracle.sdpa_ref_rows(Q, K, V, 0.35, kind, kl if kind & 2 else None, idx)
        want = full[idx[:, 0], idx[:, 1], idx[:, 2]]
        assert np.allclose(part, want, rtol=0, atol=1e-14)


def test_preconditions_rejected():
    r = np.random.default_rng(21)
    Q = r.standard_normal((1, 1, 3, 2))
    K = r.standard_normal((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.sdpa_ref(Q, K, K, 1.0, oracle.MASK_CAUSAL)        # causal needs n_q == n_k
    with pytest.raises(ValueError):
        oracle.sdpa_ref(Q, K, K, 1.0, oracle.MASK_KEY_PADDING)    # lengths missing
    with pytest.raises(ValueError):
        oracle.sdpa_ref(Q, K, K, 1.0, oracle.MASK_KEY_PADDING, np.array([0]))
    with pytest.raises(ValueError):
        oracle.sdpa_ref(Q, K, K, 1.0, oracle.MASK_KEY_PADDING, np.array([5]))
    with pytest.raises(TypeError):
        oracle.sdpa_ref(Q.astype(np.float32), K, K, 1.0)
