"""The pins are discriminating: each planted mistake in an oracle copy must
fail at least one of them (CPU only; mistakes are planted in the oracle,
never in GPU code)."""

import math
import types

import numpy as np
import pytest

import oracle
import oracle_pins as pins


def _build(scores=None, mask=None, softmax=None, combine=None, split=None, concat=None,
           mha_scale=None, kv_source=None):
    """An oracle-shaped namespace with one or more steps replaced."""
    scores = scores or (lambda Q, K, s: oracle.scaled_scores(Q, K, s))
    mask = mask or oracle.additive_mask
    softmax = softmax or oracle.softmax_rows
    combine = combine or (lambda P, V: P @ V)
    split = split or oracle.split_heads
    concat = concat or oracle.concat_heads

    def sdpa_ref(Q, K, V, scale, mask_kind=0, key_lengths=None):
        B, h, n_q, _ = Q.shape
        n_k = K.shape[2]
        S = scores(Q, K, scale)
        for b in range(B):
            L = None if key_lengths is None else int(key_lengths[b])
            S[b] = S[b] + mask(n_q, n_k, mask_kind, L)[None]
        return combine(softmax(S), V)

    def mha_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, mask_kind=0, key_lengths=None):
        d_k = Wq.shape[1] // h
        src = X_q if kv_source == "q" else X_kv
        Q = split(X_q @ Wq, h)
        K = split(src @ Wk, h)
        V = split(src @ Wv, h)
        sc = mha_scale(Wq, h, X_q) if mha_scale else 1.0 / math.sqrt(d_k)
        return concat(sdpa_ref(Q, K, V, sc, mask_kind, key_lengths)) @ Wo

    return types.SimpleNamespace(softmax_rows=softmax, additive_mask=mask, sdpa_ref=sdpa_ref,
                                 mha_ref=mha_ref)


def _mask_diag_hidden(n_q, n_k, kind, L=None):
    M = oracle.additive_mask(n_q, n_k, kind & 2, L)
    if kind & 1:
        M[np.arange(n_k)[None, :] >= np.arange(n_q)[:, None]] = -np.inf
    return M


def _mask_pad_off_by_one(n_q, n_k, kind, L=None):
    M = oracle.additive_mask(n_q, n_k, kind & 1, None)
    if kind & 2:
        M[:, np.arange(n_k) > L] = -np.inf
    return M


def _softmax_no_shift(S):
    e = np.exp(S)
    return e / e.sum(-1, keepdims=True)


def _softmax_cols(S):
    m = np.max(S, axis=-2, keepdims=True)
    e = np.exp(S - m)
    return e / e.sum(-2, keepdims=True)


def _zero_fill_sdpa():
    base = _build()

    def sdpa_ref(Q, K, V, scale, mask_kind=0, key_lengths=None):
        B, h, n_q, _ = Q.shape
        n_k = K.shape[2]
        S = oracle.scaled_scores(Q, K, scale)
        for b in range(B):
            L = None if key_lengths is None else int(key_lengths[b])
            S[b][:, np.isinf(oracle.additive_mask(n_q, n_k, mask_kind, L))] = 0.0
        return oracle.softmax_rows(S) @ V
    base.sdpa_ref = sdpa_ref
    return base


def _post_softmax_zero_sdpa():
    base = _build()

    def sdpa_ref(Q, K, V, scale, mask_kind=0, key_lengths=None):
        B, h, n_q, _ = Q.shape
        n_k = K.shape[2]
        P = oracle.softmax_rows(oracle.scaled_scores(Q, K, scale))
        for b in range(B):
            L = None if key_lengths is None else int(key_lengths[b])
            P[b][:, np.isinf(oracle.additive_mask(n_q, n_k, mask_kind, L))] = 0.0
        return P @ V
    base.sdpa_ref = sdpa_ref
    return base


def _interleaved_split(Y, h):
    B, n, hd = Y.shape
    d = hd // h
    return Y.reshape(B, n, d, h).transpose(0, 3, 1, 2)


def _reversed_concat(O):
    return oracle.concat_heads(O[:, ::-1])


MUTANTS = {
    "scale_ignored": lambda: _build(scores=lambda Q, K, s: oracle.scaled_scores(Q, K, 1.0)),
    "scale_squared": lambda: _build(scores=lambda Q, K, s: oracle.scaled_scores(Q, K, s * s)),
    "score_sign": lambda: _build(scores=lambda Q, K, s: -oracle.scaled_scores(Q, K, s)),
    "keys_for_queries": lambda: _build(scores=lambda Q, K, s: oracle.scaled_scores(K, K, s)[..., :Q.shape[2], :]
                                       if K.shape[2] >= Q.shape[2] else oracle.scaled_scores(Q, K, s) * 0),
    "causal_diagonal_hidden": lambda: _build(mask=_mask_diag_hidden),
    "padding_off_by_one": lambda: _build(mask=_mask_pad_off_by_one),
    "mask_zero_fill": _zero_fill_sdpa,
    "mask_after_softmax": _post_softmax_zero_sdpa,
    "softmax_no_max_shift": lambda: _build(softmax=_softmax_no_shift),
    "softmax_over_queries": lambda: _build(softmax=_softmax_cols),
    "weights_transposed": lambda: _build(combine=lambda P, V: np.swapaxes(P, -1, -2)[..., :V.shape[-2]] @ V
                                         if P.shape[-1] == P.shape[-2] else P @ V * 0.5),
    "values_unweighted_mean": lambda: _build(combine=lambda P, V: np.broadcast_to(
        V.mean(-2, keepdims=True), P.shape[:-1] + V.shape[-1:]).copy()),
    "mha_interleaved_heads": lambda: _build(split=_interleaved_split),
    "mha_concat_reversed": lambda: _build(concat=_reversed_concat),
    "mha_scale_dmodel": lambda: _build(mha_scale=lambda Wq, h, X: 1.0 / math.sqrt(X.shape[-1]) * 0.5),
    "mha_kv_from_queries": lambda: _build(kv_source="q"),
}


def _fails_some_pin(impl):
    failed = []
    for check in pins.ALL_SDPA_CHECKS + pins.ALL_MHA_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(check.__name__)
    return failed


def test_unmutated_copy_passes_every_pin():
    assert _fails_some_pin(_build()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failed = _fails_some_pin(MUTANTS[name]())
    assert failed, f"planted mistake {name!r} passed every pin"


# ------------------------------------------------------------ encoder layer mutants

def _ln(var_ddof=0, eps_on=True, affine_swap=False):
    def layer_norm(U, gamma, beta, eps):
        U = np.asarray(U, dtype=np.float64)
        mu = U.mean(axis=-1, keepdims=True)
        var = U.var(axis=-1, ddof=var_ddof, keepdims=True)
        z = (U - mu) / np.sqrt(var + (eps if eps_on else 0.0))
        return (z * beta + gamma) if affine_swap else (gamma * z + beta)
    return layer_norm


def _ffn(relu=True, bias_after_relu=False):
    def ffn(X, W1, b1, W2, b2):
        H = np.asarray(X, dtype=np.float64) @ W1
        if not bias_after_relu:
            H = H + b1
        if relu:
            H = np.maximum(0.0, H)
        if bias_after_relu:
            H = H + b1
        return H @ W2 + b2
    return ffn


def _build_layer(layer_norm=None, ffn=None, order="post", residual=True):
    layer_norm = layer_norm or oracle.layer_norm
    ffn = ffn or oracle.ffn

    def encoder_layer_ref(X, Wq, Wk, Wv, Wo, h, g1, be1, W1, b1, W2, b2, g2, be2, eps,
                          mask_kind=0, key_lengths=None):
        X = np.asarray(X, dtype=np.float64)
        r = 1.0 if residual else 0.0
        if order == "pre":  # x + Sublayer(LayerNorm(x))
            Xn = layer_norm(X, g1, be1, eps)
            x1 = X + oracle.mha_ref(Xn, Xn, Wq, Wk, Wv, Wo, h, mask_kind, key_lengths)
            return x1 + ffn(layer_norm(x1, g2, be2, eps), W1, b1, W2, b2)
        A = oracle.mha_ref(X, X, Wq, Wk, Wv, Wo, h, mask_kind, key_lengths)
        x1 = layer_norm(r * X + A, g1, be1, eps)
        return layer_norm(r * x1 + ffn(x1, W1, b1, W2, b2), g2, be2, eps)

    return types.SimpleNamespace(layer_norm=layer_norm, ffn=ffn, encoder_layer_ref=encoder_layer_ref)


LAYER_MUTANTS = {
    "ln_unbiased_variance": lambda: _build_layer(layer_norm=_ln(var_ddof=1)),
    "ln_eps_dropped": lambda: _build_layer(layer_norm=_ln(eps_on=False)),
    "ln_gamma_beta_swapped": lambda: _build_layer(layer_norm=_ln(affine_swap=True)),
    "ffn_no_relu": lambda: _build_layer(ffn=_ffn(relu=False)),
    "ffn_bias_after_relu": lambda: _build_layer(ffn=_ffn(bias_after_relu=True)),
    "layer_pre_ln": lambda: _build_layer(order="pre"),
    "layer_no_residual": lambda: _build_layer(residual=False),
}


def _fails_some_layer_pin(impl):
    failed = []
    for check in pins.ALL_LAYER_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(check.__name__)
    return failed


def test_unmutated_layer_copy_passes_every_pin():
    assert _fails_some_layer_pin(_build_layer()) == []


@pytest.mark.parametrize("name", sorted(LAYER_MUTANTS))
def test_layer_mutant_is_caught(name):
    failed = _fails_some_layer_pin(LAYER_MUTANTS[name]())
    assert failed, f"planted mistake {name!r} passed every pin"


# ------------------------------------------------------------ input embedding mutants

def _pe(swap=False, exponent="pair", origin=0):
    def positional_encoding(n, d_model, pos0=0):
        pos = np.arange(pos0 + origin, pos0 + origin + n, dtype=np.float64)[:, None]
        i = np.arange(d_model // 2, dtype=np.float64)[None, :]
        e = {"pair": 2.0 * i / d_model, "half": i / d_model, "coord": 4.0 * i / d_model}[exponent]
        ang = pos / np.power(10000.0, e)
        pe = np.empty((n, d_model))
        pe[:, 0::2] = np.cos(ang) if swap else np.sin(ang)
        pe[:, 1::2] = np.sin(ang) if swap else np.cos(ang)
        return pe
    return positional_encoding


def _build_embed(pe=None, scale=lambda d: math.sqrt(d)):
    pe = pe or oracle.positional_encoding

    def embed_positional_ref(tokens, E, pos0=0):
        E = np.asarray(E, dtype=np.float64)
        tokens = np.asarray(tokens)
        return E[tokens] * scale(E.shape[1]) + pe(tokens.shape[1], E.shape[1], pos0)[None]

    return types.SimpleNamespace(positional_encoding=pe, embed_positional_ref=embed_positional_ref)


EMBED_MUTANTS = {
    "pe_sin_cos_swapped": lambda: _build_embed(pe=_pe(swap=True)),
    "pe_exponent_i_over_d": lambda: _build_embed(pe=_pe(exponent="half")),
    "pe_exponent_by_coordinate": lambda: _build_embed(pe=_pe(exponent="coord")),
    "pe_positions_from_one": lambda: _build_embed(pe=_pe(origin=1)),
    "embedding_unscaled": lambda: _build_embed(scale=lambda d: 1.0),
    "embedding_scaled_by_d": lambda: _build_embed(scale=lambda d: float(d)),
}


def _fails_some_embed_pin(impl):
    failed = []
    for check in pins.ALL_EMBED_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(check.__name__)
    return failed


def test_unmutated_embed_copy_passes_every_pin():
    assert _fails_some_embed_pin(_build_embed()) == []


@pytest.mark.parametrize("name", sorted(EMBED_MUTANTS))
def test_embed_mutant_is_caught(name):
    failed = _fails_some_embed_pin(EMBED_MUTANTS[name]())
    assert failed, f"planted mistake {name!r} passed every pin"


# ------------------------------------------------------------ backward mutants

def _bwd(variant):
    def sdpa_backward_ref(Q, K, V, dO, scale, mask_kind=0, key_lengths=None):
        P = oracle.attention_weights(Q, K, scale, mask_kind, key_lengths)
        Pt = np.swapaxes(P, -1, -2)
        dV = (P if variant == "dv_untransposed" else Pt) @ dO
        dP = dO @ np.swapaxes(V, -1, -2)
        if variant == "ds_no_centering":
            dS = P * dP
        elif variant == "ds_centered_by_mean":
            dS = P * (dP - dP.mean(axis=-1, keepdims=True))
        else:
            dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
        sq = 1.0 if variant == "dq_unscaled" else scale
        dQ = sq * (dS @ K)
        dK = scale * ((dS if variant == "dk_untransposed" else np.swapaxes(dS, -1, -2)) @ Q)
        return dQ, dK, dV

    def row_logsumexp(Q, K, scale, mask_kind=0, key_lengths=None):
        lse = oracle.row_logsumexp(Q, K, scale, mask_kind, key_lengths)
        return lse / scale if variant == "lse_unscaled" else lse

    def mha_backward_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, dY, mask_kind=0, key_lengths=None):
        g = list(oracle.mha_backward_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, dY, mask_kind, key_lengths))
        if variant == "dwo_transposed" and g[5].shape[0] == g[5].shape[1]:
            g[5] = g[5].T.copy()
        if variant == "dx_kv_missing_value_path":
            from oracle.attention import concat_heads, mha_ref, split_heads
            _, it = mha_ref(X_q, X_kv, Wq, Wk, Wv, Wo, h, mask_kind, key_lengths, return_intermediates=True)
            dO = split_heads(dY @ Wo.T, h)
            d = Wq.shape[1] // h
            _, dK, _ = oracle.sdpa_backward_ref(it["Q"], it["K"], it["V"], dO, 1.0 / np.sqrt(d), mask_kind,
                                                key_lengths)
            g[1] = concat_heads(dK) @ Wk.T
        return tuple(g)

    return types.SimpleNamespace(sdpa_backward_ref=sdpa_backward_ref, row_logsumexp=row_logsumexp,
                                 mha_backward_ref=mha_backward_ref)


BWD_MUTANTS = {v: (lambda v=v: _bwd(v)) for v in
               ("dv_untransposed", "ds_no_centering", "ds_centered_by_mean", "dq_unscaled",
                "dk_untransposed", "lse_unscaled", "dwo_transposed", "dx_kv_missing_value_path")}


def _fails_some_bwd_pin(impl):
    failed = []
    for check in pins.ALL_BWD_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(check.__name__)
    return failed


def test_unmutated_bwd_copy_passes_every_pin():
    assert _fails_some_bwd_pin(_bwd("none")) == []


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(name):
    failed = _fails_some_bwd_pin(BWD_MUTANTS[name]())
    assert failed, f"planted mistake {name!r} passed every pin"
