"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: fp32 inputs max-abs <= 1e-5; bf16 inputs (fp32 accumulation)
max-abs <= 2e-2 and relative L2 <= 5e-3, with identical masking patterns
(masked keys get weight exactly 0 on both sides; checked directly by the
perturbation tests, which must be bit-exact).

Each GPU step prints the case it runs (flushed) before launching it."""

import math

import numpy as np
import pytest
import torch

import oracle
import head_attention_forward_amd as hafa
from head_attention_forward_amd.workloads import WORKLOADS, generate, to_f64

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_MAX_ABS = 1e-5


def announce(*what):
    print("[gpu case]", *what, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda")


def assert_bf16_close(got, want, what=""):
    g = to_f64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = g - want
    max_abs = float(np.abs(err).max())
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300))
    print(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= BF16_MAX_ABS, f"{what}: max-abs {max_abs}"
    assert rel <= BF16_REL_L2, f"{what}: rel-L2 {rel}"


def assert_f32_close(got, want, what=""):
    g = to_f64(got)
    assert np.all(np.isfinite(g))
    max_abs = float(np.abs(g - want).max())
    print(f"  {what}: max_abs={max_abs:.3e}", flush=True)
    assert max_abs <= F32_MAX_ABS, f"{what}: max-abs {max_abs}"


def sdpa_inputs(B, h, n_q, n_k, dtype, seed, q_scale=1.0):
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    Q = (torch.randn((B, h, n_q, 64), generator=g) * q_scale).to(dtype)
    K = torch.randn((B, h, n_k, 64), generator=g).to(dtype)
    V = torch.randn((B, h, n_k, 64), generator=g).to(dtype)
    return Q, K, V


def run_sdpa(dev, Q, K, V, scale, mask, kl):
    return hafa.sdpa_forward(Q.to(dev), K.to(dev), V.to(dev), scale, mask, kl)


def ref_sdpa(Q, K, V, scale, mask, kl):
    return oracle.sdpa_ref(to_f64(Q), to_f64(K), to_f64(V), scale, mask,
                           None if kl is None else np.asarray(kl))


# ------------------------------------------------------------------ the five workloads

def test_sdpa_f32_tiny(dev):
    w = WORKLOADS["sdpa_f32_tiny"]
    x = generate(w, seed=0)
    announce("sdpa_forward f32", w.description)
    O = run_sdpa(dev, x["Q"], x["K"], x["V"], x["scale"], w.mask, None)
    torch.cuda.synchronize()
    assert_f32_close(O, ref_sdpa(x["Q"], x["K"], x["V"], x["scale"], w.mask, None), w.name)


def _mha_case(dev, w, seed=0):
    x = generate(w, seed=seed)
    Xq = x["X_q"].to(dev)
    Xkv = Xq if w.self_attn else x["X_kv"].to(dev)
    Ws = [x[k].to(dev) for k in ("Wq", "Wk", "Wv", "Wo")]
    kl = x["key_lengths"]
    announce("mha_forward bf16", w.description, "seed", seed)
    Y = hafa.mha_forward(Xq, Xkv, *Ws, w.h, w.mask, kl)
    torch.cuda.synchronize()
    want, inter = oracle.mha_ref(to_f64(x["X_q"]), to_f64(x["X_kv"]),
                                 *[to_f64(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")], w.h, w.mask,
                                 None if kl is None else kl.numpy(), return_intermediates=True)
    assert_bf16_close(Y, want, w.name)
    return x, Xq, Xkv, Ws, kl, Y, inter


@pytest.mark.parametrize("name", ["encoder_self_base", "decoder_causal_base", "cross_padded_big"])
def test_mha_workloads(dev, name):
    _mha_case(dev, WORKLOADS[name])


def test_mha_ragged_rows_on_256_row_projection_tiles(dev):
    """B = 5, n = 1631: 8155 rows x 1536 columns of the stacked projection
    take 256 x 256 tiles (192 of them), the last row tile 219 rows deep."""
    w = WORKLOADS["decoder_causal_base"].replace(name="ragged256", B=5, n_q=1631, n_k=1631,
                                                 description="B=5 n=1631 causal, 256-row tiles")
    _mha_case(dev, w, seed=5)


def test_mha_stages_equal_forward_and_intermediates(dev):
    """The three stage calls reproduce mha_forward bit for bit, and the
    workspace intermediates match the oracle's projections and concat."""
    w = WORKLOADS["cross_padded_big"]
    x, Xq, Xkv, Ws, kl, Y, inter = _mha_case(dev, w)
    ws = hafa.alloc_workspace(w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v, dev)
    announce("mha stages", w.name)
    hafa.mha_project_in(Xq, Xkv, Ws[0], Ws[1], Ws[2], w.h, ws)
    hafa.mha_attend(w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v, ws, w.mask, kl)
    Y2 = torch.empty_like(Y)
    hafa.mha_project_out(Ws[3], Y2, w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    q, k, v, o = hafa.workspace_views(ws, w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v)
    assert_bf16_close(q, inter["Q"], "Q projection")
    assert_bf16_close(k, inter["K"], "K projection")
    assert_bf16_close(v, inter["V"], "V projection")
    assert_bf16_close(o, inter["concat"], "concatenated heads")


def test_sdpa_long_causal_sampled(dev):
    """Full size, in the launch configuration the bench times; the oracle
    evaluates sampled rows one by one (every boundary row included)."""
    w = WORKLOADS["long_causal_sdpa"]
    x = generate(w, seed=0)
    announce("sdpa_forward bf16", w.description)
    O = run_sdpa(dev, x["Q"], x["K"], x["V"], x["scale"], w.mask, None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    special = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 2047, 2048, 4094, 4095]
    idx = [(b, hh, q) for b in range(w.B) for hh in (0, w.h - 1) for q in special]
    idx += [(int(rng.integers(w.B)), int(rng.integers(w.h)), int(rng.integers(w.n_q)))
            for _ in range(400)]
    idx = np.array(idx)
    want = oracle.sdpa_ref_rows(to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"]), x["scale"],
                                w.mask, None, idx)
    got = O[idx[:, 0], idx[:, 1], idx[:, 2]]
    assert_bf16_close(got, want, w.name + " sampled rows")
    # Two whole heads, every query tile: every row of the first and of the
    # last (batch, head) against the oracle, element by element.
    Q64, K64, V64 = to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"])
    for b, hh in ((0, 0), (w.B - 1, w.h - 1)):
        sl = lambda t: t[b:b + 1, hh:hh + 1]  # noqa: E731
        want_h = oracle.sdpa_ref(sl(Q64), sl(K64), sl(V64), x["scale"], w.mask, None)
        assert_bf16_close(O[b:b + 1, hh:hh + 1], want_h, f"{w.name} whole head ({b}, {hh})")
    # Causal row 0 sees only key 0: exactly value row 0.
    assert torch.equal(O[:, :, 0].cpu(), x["V"][:, :, 0])
    # Every output row is a convex combination of V rows: coordinates within the
    # per-(batch, head) range of V (checked on the whole output).
    Vd = x["V"].to(dev).float()
    lo = Vd.amin(dim=2, keepdim=True)
    hi = Vd.amax(dim=2, keepdim=True)
    Of = O.float()
    assert bool(((Of >= lo - 1e-2) & (Of <= hi + 1e-2)).all())


def test_sdpa_unmasked_eight_wave_workgroups(dev):
    """Unmasked attention large enough for 8-wave workgroups (B=4, h=16,
    n=2048: 512 of them): sampled rows (every tile boundary included) and two
    whole heads against the oracle; the forward with lse returns the same
    output and, on those heads, the oracle's row log-sum-exp (to 2^-8, the
    bound the backward tests use)."""
    B, h, n = 4, 16, 2048
    Q, K, V = sdpa_inputs(B, h, n, n, torch.bfloat16, seed=2048)
    announce("sdpa_forward bf16 unmasked, 8-wave workgroups", dict(B=B, h=h, n=n))
    Qd, Kd, Vd = (t.to(dev) for t in (Q, K, V))
    O = hafa.sdpa_forward(Qd, Kd, Vd, 0.125, 0)
    O2, lse = hafa.sdpa_forward_lse(Qd, Kd, Vd, 0.125, 0)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    rng = np.random.default_rng(1)
    special = [0, 1, 127, 128, 255, 256, 1023, 1024, 2046, 2047]
    idx = [(b, hh, q) for b in range(B) for hh in (0, h - 1) for q in special]
    idx += [(int(rng.integers(B)), int(rng.integers(h)), int(rng.integers(n))) for _ in range(300)]
    idx = np.array(idx)
    Q64, K64, V64 = to_f64(Q), to_f64(K), to_f64(V)
    want = oracle.sdpa_ref_rows(Q64, K64, V64, 0.125, 0, None, idx)
    assert_bf16_close(O[idx[:, 0], idx[:, 1], idx[:, 2]], want, "unmasked 4x16x2048 sampled rows")
    for b, hh in ((0, 0), (B - 1, h - 1)):
        sl = lambda t: t[b:b + 1, hh:hh + 1]  # noqa: E731
        want_h = oracle.sdpa_ref(sl(Q64), sl(K64), sl(V64), 0.125, 0, None)
        assert_bf16_close(O[b:b + 1, hh:hh + 1], want_h, f"unmasked whole head ({b}, {hh})")
        want_l = oracle.row_logsumexp(sl(Q64), sl(K64), 0.125, 0, None)
        lerr = float(np.abs(to_f64(lse[b:b + 1, hh:hh + 1]) - want_l).max())
        print(f"  lse ({b}, {hh}) max_abs={lerr:.2e}", flush=True)
        assert lerr <= 2.0 ** -8 + 1e-6


KEY_SPLIT = [
    # (B, h, n_q, n_k, mask, key_lengths): at most one 4-wave workgroup per
    # compute unit over at least 1024 keys, where the launch takes two key
    # groups per workgroup (four from 2048 keys on)
    (1, 2, 300, 1500, 0, None),            # ragged query and key tiles
    (1, 3, 1100, 1100, 1, None),           # causal: the second group sees part or none of a tile
    (2, 2, 200, 2000, 2, [1, 1500]),       # one visible key: the second group sees nothing
    (2, 1, 1030, 1030, 3, [1030, 700]),    # causal + padding
    (1, 1, 33, 4096, 0, None),             # four groups; one wave of queries has 1 query
    (1, 8, 128, 1024, 2, [1024]),          # exactly 16 key tiles, 8 per group
    # from 2048 keys on, four key groups
    (1, 2, 300, 2500, 0, None),            # ragged: 40 tiles, 10 per group
    (1, 2, 2100, 2100, 1, None),           # causal: early query tiles leave groups 1-3 idle
    (2, 1, 100, 3000, 2, [1, 2999]),       # one visible key: groups 1-3 see nothing
    (1, 3, 64, 2048, 2, [2048]),           # exactly 32 tiles, 8 per group
]


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl", KEY_SPLIT)
def test_sdpa_key_split(dev, B, h, n_q, n_k, mask, kl):
    """The two- and four-key-group workgroups against the oracle on every
    row, and their row log-sum-exp (the backward pass's input) to 2^-8."""
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=7 * n_q + n_k)
    announce("sdpa_forward bf16 key split", dict(B=B, h=h, n_q=n_q, n_k=n_k, mask=mask, kl=kl))
    Qd, Kd, Vd = (t.to(dev) for t in (Q, K, V))
    O = hafa.sdpa_forward(Qd, Kd, Vd, 0.125, mask, kl)
    O2, lse = hafa.sdpa_forward_lse(Qd, Kd, Vd, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    kla = None if kl is None else np.array(kl)
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"key split {B}x{h}x{n_q}x{n_k} m{mask}")
    want_l = oracle.row_logsumexp(to_f64(Q), to_f64(K), 0.125, mask, kla)
    lerr = float(np.abs(to_f64(lse) - want_l).max())
    print(f"  lse max_abs={lerr:.2e}", flush=True)
    assert lerr <= 2.0 ** -8 + 1e-6


def test_sdpa_key_split_padded_chunks(dev):
    """A padded batch beyond one launch (256 batches per launch) over more
    than 1024 keys: both chunks take the two-key-group workgroups; every
    batch's length is honoured (one of them a single key)."""
    B, h, n_q, n_k = 300, 1, 40, 1100
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=300)
    g = torch.Generator("cpu")
    g.manual_seed(301)
    kl = torch.randint(1, n_k + 1, (B,), generator=g).tolist()
    kl[0], kl[257], kl[-1] = 1, n_k, 700
    announce("sdpa_forward bf16 key split, padded, two launches", dict(B=B, n_q=n_q, n_k=n_k))
    O = run_sdpa(dev, Q, K, V, 0.125, 2, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, 2, kl), "key split padded chunks")


# ------------------------------------------------------------------ edge shapes

EDGE = [
    # (B, h, n_q, n_k, mask, key_lengths)
    (1, 1, 1, 1, 0, None),
    (1, 1, 1, 300, 0, None),          # single query, many keys
    (2, 3, 63, 63, 1, None),
    (1, 2, 64, 64, 1, None),
    (2, 1, 65, 65, 1, None),
    (3, 2, 100, 100, 0, None),
    (1, 1, 127, 127, 1, None),
    (2, 2, 128, 128, 0, None),
    (1, 3, 129, 129, 1, None),
    (2, 2, 200, 77, 0, None),         # n_q != n_k, ragged keys
    (2, 2, 33, 250, 0, None),
    (4, 2, 96, 128, 2, [1, 64, 127, 128]),
    (3, 1, 130, 130, 3, [1, 65, 130]),
    (2, 2, 257, 257, 3, [200, 257]),
    # key ranges of at most 128 (at most two key tiles)
    (2, 2, 300, 96, 0, None),         # three query tiles over 96 keys
    (3, 2, 40, 33, 0, None),          # the second key group holds one key
    (1, 2, 129, 1, 0, None),          # one key, two query tiles
    (2, 2, 130, 128, 2, [128, 31]),
    (2, 1, 100, 100, 3, [1, 100]),    # causal + padding, one visible key in batch 0
]


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl", EDGE)
def test_sdpa_bf16_edges(dev, B, h, n_q, n_k, mask, kl):
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=n_q * 1000 + n_k)
    announce("sdpa_forward bf16 edge", dict(B=B, h=h, n_q=n_q, n_k=n_k, mask=mask, kl=kl))
    O = run_sdpa(dev, Q, K, V, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"edge {B}x{h}x{n_q}x{n_k} m{mask}")


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl", [(2, 64, 1000, 1000, 3, [1000, 777]),
                                                 (2, 64, 1000, 1300, 0, None),
                                                 (1, 128, 777, 777, 1, None)])
def test_sdpa_bf16_large_ragged_sampled(dev, B, h, n_q, n_k, mask, kl):
    """Shapes large enough for the 256-query workgroup configuration, with
    ragged query and key counts; sampled rows against the oracle."""
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=n_q + n_k)
    announce("sdpa_forward bf16 large", dict(B=B, h=h, n_q=n_q, n_k=n_k, mask=mask, kl=kl))
    O = run_sdpa(dev, Q, K, V, 0.125, mask, kl)
    torch.cuda.synchronize()
    rng = np.random.default_rng(n_q)
    idx = [(b, hh, q) for b in range(B) for hh in (0, h - 1) for q in (0, 255, 256, n_q - 1)]
    idx += [(int(rng.integers(B)), int(rng.integers(h)), int(rng.integers(n_q))) for _ in range(300)]
    idx = np.array(idx)
    want = oracle.sdpa_ref_rows(to_f64(Q), to_f64(K), to_f64(V), 0.125, mask,
                                None if kl is None else np.array(kl), idx)
    assert_bf16_close(O[idx[:, 0], idx[:, 1], idx[:, 2]], want, f"large {B}x{h}x{n_q}x{n_k} m{mask}")


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl", [(1, 1, 1, 1, 0, None), (2, 2, 100, 100, 1, None),
                                                 (2, 1, 70, 129, 2, [5, 129]),
                                                 (1, 2, 200, 200, 3, [150]),
                                                 (3, 2, 33, 1000, 2, [1, 999, 1000])])
def test_sdpa_f32_edges(dev, B, h, n_q, n_k, mask, kl):
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.float32, seed=7 + n_q)
    announce("sdpa_forward f32 edge", dict(B=B, h=h, n_q=n_q, n_k=n_k, mask=mask, kl=kl))
    O = run_sdpa(dev, Q, K, V, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert_f32_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"f32 edge {n_q}x{n_k} m{mask}")


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl", [(4, 16, 300, 300, 1, None),
                                                 (2, 64, 100, 129, 2, [5, 129]),
                                                 (8, 32, 33, 70, 0, None)])
def test_sdpa_f32_eight_lane_kernel(dev, B, h, n_q, n_k, mask, kl):
    """Launches with at least one 32-query workgroup per compute unit take
    the eight-lanes-per-query fp32 kernel (the smaller ones above take the
    wave-per-query kernel); every output element against the oracle."""
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.float32, seed=11 + n_q)
    announce("sdpa_forward f32 eight-lane kernel", dict(B=B, h=h, n_q=n_q, n_k=n_k, mask=mask, kl=kl))
    O = run_sdpa(dev, Q, K, V, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert_f32_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"f32 {B}x{h}x{n_q}x{n_k} m{mask}")


def test_sdpa_f32_padded_chunks(dev):
    """fp32 over a padded batch beyond one launch: the first 256 batches fill
    the compute units (eight lanes per query), the other 44 do not (one wave
    per query); every batch's length is honoured."""
    B, h, n_q, n_k = 300, 1, 5, 70
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.float32, seed=302)
    g = torch.Generator("cpu")
    g.manual_seed(303)
    kl = torch.randint(1, n_k + 1, (B,), generator=g).tolist()
    kl[0], kl[256], kl[-1] = 1, n_k, 1
    announce("sdpa_forward f32 padded, two launches", dict(B=B, n_q=n_q, n_k=n_k))
    O = run_sdpa(dev, Q, K, V, 0.125, 2, kl)
    torch.cuda.synchronize()
    assert_f32_close(O, ref_sdpa(Q, K, V, 0.125, 2, kl), "f32 padded chunks")


@pytest.mark.parametrize("B,mask", [(256, 2), (256, 3), (257, 3), (1024, 2), (1024, 3)])
def test_sdpa_bf16_max_padded_batch(dev, B, mask):
    """Per-batch key lengths up to the largest padded batch (1024; they
    travel in the kernel arguments, 256 batches per launch, so 257 and 1024
    take two and four launches): every batch's lengths are honoured."""
    h, n = 1, 24
    Q, K, V = sdpa_inputs(B, h, n, n, torch.bfloat16, seed=31)
    g = torch.Generator("cpu")
    g.manual_seed(32)
    kl = torch.randint(1, n + 1, (B,), generator=g).tolist()
    kl[0], kl[-1] = 1, n
    announce("sdpa max padded batch", B, mask)
    O = run_sdpa(dev, Q, K, V, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"B={B} mask {mask}")


def test_sdpa_decode_padded_batch_1024(dev):
    """One query per sequence over a 300-key cache for 1024 sequences with
    their own cache lengths (the few-query kernel, four launches of 256)."""
    B, h, n_k = 1024, 2, 300
    Q, K, V = sdpa_inputs(B, h, 1, n_k, torch.bfloat16, seed=47)
    g = torch.Generator("cpu").manual_seed(48)
    kl = torch.randint(1, n_k + 1, (B,), generator=g).tolist()
    kl[0], kl[255], kl[256], kl[-1] = 1, n_k, 2, n_k
    announce("sdpa decode padded B=1024")
    O = run_sdpa(dev, Q, K, V, 0.125, 2, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, 2, kl), "decode B=1024")


def test_mha_max_padded_batch_and_fused_boundary(dev):
    """The whole block at the largest padded batch (fused path), and just past
    the fused kernel's 128-row limit (n = 129: the staged path)."""
    cases = [
        dict(B=256, n_q=16, n_k=16, d_model=64, h=1, mask=3, self_attn=True, key_len_range=(1, 16)),
        dict(B=1024, n_q=16, n_k=24, d_model=64, h=1, mask=2, self_attn=False, key_len_range=(1, 24)),
        dict(B=300, n_q=136, n_k=136, d_model=64, h=1, mask=3, self_attn=True, key_len_range=(1, 136)),
        dict(B=2, n_q=129, n_k=129, d_model=128, h=2, mask=1, self_attn=True),
        dict(B=2, n_q=128, n_k=129, d_model=128, h=2, mask=2, self_attn=False, key_len_range=(1, 129)),
    ]
    for c in cases:
        w = WORKLOADS["cross_padded_big"].replace(
            name="limits", B=c["B"], n_q=c["n_q"], n_k=c["n_k"], d_model=c["d_model"], h=c["h"],
            mask=c["mask"], self_attn=c["self_attn"], key_len_range=c.get("key_len_range"),
            description=str(c))
        fused = max(w.n_q, w.n_k) <= 128
        assert hafa.lib().mha_forward_launches(w.n_q, w.n_k, w.d_model, 1 if w.self_attn else 0) == \
            (2 if fused else (3 if w.self_attn else 4))
        _mha_case(dev, w, seed=3)


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl", [
    (2, 3, 1, 129, 0, None), (3, 2, 1, 300, 2, [300, 1, 191]), (2, 2, 5, 1000, 2, [1000, 650]),
    (1, 4, 32, 777, 0, None), (4, 2, 1, 4096, 2, [4096, 2049, 1, 3000]), (1, 2, 17, 8193, 0, None),
    # more (batch, head) pairs than compute units (a second wave of workgroups)
    (9, 32, 3, 513, 0, None), (65, 4, 1, 1000, 2, [1 + (i * 397) % 1000 for i in range(65)]),
])
def test_sdpa_decode_shapes(dev, B, h, n_q, n_k, mask, kl):
    """Few queries over long key ranges (one new query per sequence against
    cached keys, with per-sequence cache lengths): the keys are split over
    waves and the partial softmaxes merged."""
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=41)
    announce("sdpa decode", B, h, n_q, n_k, mask, kl)
    O = run_sdpa(dev, Q, K, V, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"decode {B}x{h} {n_q}x{n_k}")
    if kl is not None:  # keys past a sequence's length have exactly zero weight
        K2, V2 = K.clone(), V.clone()
        for b, L in enumerate(kl):
            K2[b, :, L:] = 40.0
            V2[b, :, L:] = -9.0
        O2 = run_sdpa(dev, Q, K2, V2, 0.125, mask, kl)
        torch.cuda.synchronize()
        assert torch.equal(O2.cpu(), O.cpu())


def test_decode_step_full_size(dev):
    """The decode workload at its full size (B=32, h=16: 512 heads of one
    query against cache lengths drawn from [1024, 4096]), every output
    against the oracle."""
    w = WORKLOADS["decode_step_sdpa"]
    g = torch.Generator().manual_seed(9)
    kl = torch.randint(w.key_len_range[0], w.key_len_range[1] + 1, (w.B,), generator=g).tolist()
    Q, K, V = sdpa_inputs(w.B, w.h, w.n_q, w.n_k, torch.bfloat16, seed=43)
    announce("sdpa decode full size", w.B, w.h, w.n_q, w.n_k, kl)
    O = run_sdpa(dev, Q, K, V, 0.125, w.mask, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, w.mask, kl), "decode_step_sdpa")


def test_saturated_and_uniform(dev):
    """Large-magnitude scores (softmax saturation) stay finite and accurate;
    Q = 0 gives uniform weights: outputs are means of the visible V rows."""
    Q, K, V = sdpa_inputs(2, 2, 150, 150, torch.bfloat16, seed=3, q_scale=30.0)
    announce("sdpa saturated")
    O = run_sdpa(dev, Q, K, V, 0.125, 1, None)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, 1, None), "saturated causal")
    Z = torch.zeros_like(Q)
    announce("sdpa zero queries")
    for mask, kl in ((0, None), (1, None), (2, [7, 150])):
        O = run_sdpa(dev, Z, K, V, 0.125, mask, kl)
        torch.cuda.synchronize()
        Vd = to_f64(V)
        want = np.empty(O.shape)
        for b in range(2):
            for q in range(150):
                n_vis = q + 1 if mask == 1 else (kl[b] if mask == 2 else 150)
                want[b, :, q] = Vd[b, :, :n_vis].mean(axis=1)
        assert_bf16_close(O, want, f"zero Q mask {mask}")


@pytest.mark.parametrize("mask,kl", [(0, None), (1, None), (2, [300, 170])])
def test_rising_scores_move_the_reference_every_half_tile(dev, mask, kl):
    """Scores that climb by about 11 (log2 units) every 32 keys force the
    streaming softmax to move its reference value in every half tile,
    including a half whose scores were already taken against the old one."""
    B, h, n = 2, 2, 300
    g = torch.Generator("cpu")
    g.manual_seed(21)
    Q = torch.randn((B, h, n, 64), generator=g) * 0.05
    K = torch.randn((B, h, n, 64), generator=g) * 0.05
    V = torch.randn((B, h, n, 64), generator=g)
    Q[..., 0] = 4.0
    K[..., 0] = 0.5 * torch.arange(n, dtype=torch.float32)  # score ~ 2 j, x 0.125 x log2(e)
    Q, K, V = Q.to(torch.bfloat16), K.to(torch.bfloat16), V.to(torch.bfloat16)
    announce("rising scores", mask, kl)
    O = run_sdpa(dev, Q, K, V, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"rising scores mask {mask}")


def test_masked_keys_have_exactly_zero_weight(dev):
    """Changing keys/values a query may not see leaves its output bit-exact:
    future rows under the causal mask, padded rows under key padding."""
    B, h, n = 2, 2, 200
    Q, K, V = sdpa_inputs(B, h, n, n, torch.bfloat16, seed=11)
    announce("causal perturbation")
    O = run_sdpa(dev, Q, K, V, 0.125, 1, None).cpu()
    for i in (0, 63, 64, 130, 198):
        K2, V2 = K.clone(), V.clone()
        K2[:, :, i + 1:] = K2[:, :, i + 1:] * -7
        V2[:, :, i + 1:] = V2[:, :, i + 1:] * 5 + 3
        O2 = run_sdpa(dev, Q, K2, V2, 0.125, 1, None).cpu()
        assert torch.equal(O2[:, :, : i + 1], O[:, :, : i + 1]), i
    announce("padding perturbation")
    kl = [37, 129]
    O = run_sdpa(dev, Q, K, V, 0.125, 2, kl).cpu()
    K2, V2 = K.clone(), V.clone()
    for b, L in enumerate(kl):
        K2[b, :, L:] = 50.0
        V2[b, :, L:] = -80.0
    O2 = run_sdpa(dev, Q, K2, V2, 0.125, 2, kl).cpu()
    assert torch.equal(O, O2)


def test_deterministic_and_in_bounds(dev):
    """Two runs agree bit for bit, and nothing is written past the output
    (canary bytes around the output stay intact)."""
    B, h, n_q, n_k = 3, 2, 131, 131
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=5)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    numel = B * h * n_q * 64
    pad = 4096
    buf = torch.full((numel + 2 * pad,), -12345.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + numel].view(B, h, n_q, 64)
    announce("determinism + canary")
    hafa.sdpa_forward(Qd, Kd, Vd, 0.125, 3, [131, 17, 64], out=out)
    first = out.clone()
    hafa.sdpa_forward(Qd, Kd, Vd, 0.125, 3, [131, 17, 64], out=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool((buf[:pad] == -12345.0).all()) and bool((buf[pad + numel:] == -12345.0).all())


def test_short_key_ranges_masking_saturation_canary(dev):
    """Key ranges of at most 128 keys (at most two key tiles):
    hidden keys have exactly zero weight, large scores stay accurate, two
    runs agree bit for bit and nothing is written past the output."""
    B, h, n = 2, 2, 100
    Q, K, V = sdpa_inputs(B, h, n, n, torch.bfloat16, seed=12)
    announce("short causal perturbation")
    O = run_sdpa(dev, Q, K, V, 0.125, 1, None).cpu()
    for i in (0, 31, 32, 63, 95):
        K2, V2 = K.clone(), V.clone()
        K2[:, :, i + 1:] = K2[:, :, i + 1:] * -7
        V2[:, :, i + 1:] = V2[:, :, i + 1:] * 5 + 3
        O2 = run_sdpa(dev, Q, K2, V2, 0.125, 1, None).cpu()
        assert torch.equal(O2[:, :, : i + 1], O[:, :, : i + 1]), i
    announce("short padding perturbation")
    kl = [37, 100]
    O = run_sdpa(dev, Q, K, V, 0.125, 2, kl).cpu()
    K2, V2 = K.clone(), V.clone()
    K2[0, :, 37:] = 50.0
    V2[0, :, 37:] = -80.0
    assert torch.equal(O, run_sdpa(dev, Q, K2, V2, 0.125, 2, kl).cpu())
    announce("short saturated")
    Qs, Ks, Vs = sdpa_inputs(2, 2, 120, 120, torch.bfloat16, seed=4, q_scale=30.0)
    for mask in (0, 1):
        Os = run_sdpa(dev, Qs, Ks, Vs, 0.125, mask, None)
        torch.cuda.synchronize()
        assert_bf16_close(Os, ref_sdpa(Qs, Ks, Vs, 0.125, mask, None), f"short saturated mask {mask}")
    announce("short determinism + canary")
    B, h, n_q, n_k = 3, 2, 131, 100
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=6)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    numel = B * h * n_q * 64
    pad = 4096
    buf = torch.full((numel + 2 * pad,), -12345.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + numel].view(B, h, n_q, 64)
    hafa.sdpa_forward(Qd, Kd, Vd, 0.125, 2, [100, 17, 64], out=out)
    first = out.clone()
    hafa.sdpa_forward(Qd, Kd, Vd, 0.125, 2, [100, 17, 64], out=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool((buf[:pad] == -12345.0).all()) and bool((buf[pad + numel:] == -12345.0).all())
    assert_bf16_close(out, ref_sdpa(Q, K, V, 0.125, 2, [100, 17, 64]), "short padding, two query tiles")


def test_mha_small_shapes(dev):
    """The whole block on small odd shapes: h = 1, odd batch, ragged rows,
    cross-attention without padding, padding with causal self-attention, and
    model widths that are not a multiple of the GEMM's 64-wide K stage or
    128-wide column tile (d_model = 200, 72)."""
    cases = [
        dict(B=1, n_q=1, n_k=1, d_model=64, h=1, mask=0, self_attn=True),
        dict(B=3, n_q=37, n_k=37, d_model=128, h=2, mask=1, self_attn=True),
        dict(B=2, n_q=50, n_k=130, d_model=192, h=3, mask=0, self_attn=False),
        dict(B=2, n_q=70, n_k=70, d_model=256, h=4, mask=3, self_attn=True, key_len_range=(1, 70)),
        dict(B=3, n_q=45, n_k=45, d_model=200, h=3, mask=1, self_attn=True),
        dict(B=2, n_q=33, n_k=66, d_model=72, h=2, mask=2, self_attn=False, key_len_range=(1, 66)),
    ]
    for c in cases:
        w = WORKLOADS["cross_padded_big"].replace(
            name="small", B=c["B"], n_q=c["n_q"], n_k=c["n_k"], d_model=c["d_model"], h=c["h"],
            mask=c["mask"], self_attn=c["self_attn"], key_len_range=c.get("key_len_range"),
            description=str(c))
        _mha_case(dev, w, seed=1)


@pytest.mark.parametrize("case", [
    dict(B=3, n_q=100, n_k=100, d_model=512, h=8, mask=0, self_attn=True),
    dict(B=2, n_q=96, n_k=128, d_model=1024, h=16, mask=2, self_attn=False, key_len_range=(1, 128)),
    # more (batch, head) units than compute units: two heads per workgroup
    dict(B=40, n_q=100, n_k=100, d_model=512, h=8, mask=1, self_attn=True),
    dict(B=20, n_q=96, n_k=128, d_model=1024, h=16, mask=2, self_attn=False, key_len_range=(1, 128)),
    # ... query rows ending inside an 8-row copy block, units not a multiple of the XCDs
    dict(B=33, n_q=100, n_k=77, d_model=512, h=8, mask=2, self_attn=False, key_len_range=(1, 77)),
    # ... one 32-row query block (the other Q row blocks skipped)
    dict(B=130, n_q=20, n_k=128, d_model=128, h=2, mask=0, self_attn=False),
    # ... a single k stage, all 128 rows
    dict(B=130, n_q=128, n_k=128, d_model=64, h=2, mask=0, self_attn=True),
    # ... an odd head count: one head per workgroup, the one-stage ring
    dict(B=100, n_q=50, n_k=50, d_model=192, h=3, mask=0, self_attn=True),
    dict(B=2, n_q=128, n_k=128, d_model=128, h=2, mask=1, self_attn=True),
    dict(B=4, n_q=1, n_k=77, d_model=64, h=1, mask=0, self_attn=False),
    dict(B=2, n_q=65, n_k=65, d_model=192, h=3, mask=3, self_attn=True, key_len_range=(1, 65)),
])
def test_fused_plan_equals_staged(dev, case):
    """Short sequences take the fused projection + attention kernel; its
    result equals the three stage calls (standalone projection GEMM,
    attention, output projection) bit for bit, and the oracle within the
    bf16 tolerance."""
    w = WORKLOADS["cross_padded_big"].replace(
        name="fused", B=case["B"], n_q=case["n_q"], n_k=case["n_k"], d_model=case["d_model"],
        h=case["h"], mask=case["mask"], self_attn=case["self_attn"],
        key_len_range=case.get("key_len_range"), description=str(case))
    assert hafa.lib().mha_forward_launches(w.n_q, w.n_k, w.d_model, 1 if w.self_attn else 0) == 2
    x, Xq, Xkv, Ws, kl, Y, inter = _mha_case(dev, w, seed=2)
    ws = hafa.alloc_workspace(w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v, dev)
    announce("staged path", w.description)
    hafa.mha_project_in(Xq, Xkv, Ws[0], Ws[1], Ws[2], w.h, ws)
    hafa.mha_attend(w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v, ws, w.mask, kl)
    Y2 = torch.empty_like(Y)
    hafa.mha_project_out(Ws[3], Y2, w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("B,h,n_q,n_k,mask,kl", [
    (8, 16, 1, 4096, 0, None),                 # 128 (batch, head) pairs: two workgroups each
    (1, 2, 3, 1000, 2, [777]),                 # few pairs, short range: split bounded by the tiles
    (2, 4, 32, 8193, 0, None),                 # eight splits, ragged last tile
    (3, 1, 5, 2000, 2, [2000, 1, 1100]),       # a sequence with one visible key: empty splits
    (4, 2, 1, 300, 2, [1, 300, 64, 129]),      # too few tiles to split: the plain path
    (2, 2, 64, 640, 0, None),                  # more than 32 queries: the plain path
    (1, 2, 200, 200, 1, None),                 # causal: the plain path
    (300, 1, 1, 600, 2, [1 + (i * 37) % 600 for i in range(300)]),  # padded beyond one launch: plain, chunked
])
def test_sdpa_decode_split(dev, B, h, n_q, n_k, mask, kl):
    """sdpa_decode: with few (batch, head) pairs the key tiles of each pair
    are dealt to several workgroups and their partial softmax states merged
    by a second launch.  Every output against the oracle; keys past a
    sequence's length have exactly zero weight."""
    Q, K, V = sdpa_inputs(B, h, n_q, n_k, torch.bfloat16, seed=61 + n_k)
    L = hafa.lib()
    announce("sdpa_decode", B, h, n_q, n_k, mask, kl,
             "launches", L.sdpa_decode_launches(B, h, n_q, n_k, mask))
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    O = hafa.sdpa_decode(Qd, Kd, Vd, 0.125, mask, kl)
    torch.cuda.synchronize()
    assert_bf16_close(O, ref_sdpa(Q, K, V, 0.125, mask, kl), f"decode split {B}x{h} {n_q}x{n_k}")
    if kl is not None:
        K2, V2 = Kd.clone(), Vd.clone()
        for b, Lb in enumerate(kl):
            K2[b, :, Lb:] = 40.0
            V2[b, :, Lb:] = -9.0
        O2 = hafa.sdpa_decode(Qd, K2, V2, 0.125, mask, kl)
        torch.cuda.synchronize()
        assert torch.equal(O2, O)
