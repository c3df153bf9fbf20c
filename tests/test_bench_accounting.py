"""The bench's algorithmic flop and byte counts against closed forms (CPU)."""

import math

import pytest
import torch

import bench
from head_attention_forward_amd.workloads import WORKLOADS, generate


def test_attention_counts_unmasked_self():
    w = WORKLOADS["encoder_self_base"]
    f, b = bench.attention_accounting(w, None)
    assert f == 4 * 32 * 8 * 100 * 100 * 64            # dense = nominal when unmasked
    assert b == 2 * 32 * 8 * 100 * 64 * 4                # Q, K, V read once, O written once
    assert abs(b - 13.1e6) < 0.05e6


def test_attention_counts_causal():
    w = WORKLOADS["long_causal_sdpa"]
    f, b = bench.attention_accounting(w, None)
    n = 4096
    assert f == 2 * (n * (n + 1) / 2) * 128 * 64        # i + 1 visible keys for query i
    assert abs(f / 1e9 - 137.5) < 0.1
    assert abs(w.nominal_attention_flops() / 1e9 - 274.9) < 0.1


def test_attention_counts_padded():
    w = WORKLOADS["cross_padded_big"]
    kl = torch.tensor([64, 128] * 16, dtype=torch.int32)
    f, b = bench.attention_accounting(w, kl)
    assert f == 2 * 96 * (64 + 128) * 16 * 16 * 128
    assert b == 2 * 16 * (32 * 96 * 64 + (64 + 128) * 16 * 128 + 32 * 96 * 64)


def test_causal_with_padding_counts():
    w = WORKLOADS["decoder_causal_base"].replace(kind="sdpa", mask=3, B=2, n_q=10, n_k=10, h=1)
    f, _ = bench.attention_accounting(w, [4, 10])
    # batch 0: queries 0..3 see 1..4 keys, queries 4..9 see 4; batch 1: 1..10
    pairs = (1 + 2 + 3 + 4 + 6 * 4) + 55
    assert f == 2 * pairs * 128


def test_gemm_plan():
    plan, _ = bench.kernel_plan(WORKLOADS["encoder_self_base"], 3)
    assert [p["name"] for p in plan] == ["qkv_projection_gemm", "attention", "output_projection_gemm"]
    assert plan[0]["flops"] == 2 * 3200 * 512 * 1536
    assert plan[2]["flops"] == 2 * 3200 * 512 * 512
    plan, _ = bench.kernel_plan(WORKLOADS["cross_padded_big"], 4)
    assert [p["name"] for p in plan][:2] == ["q_projection_gemm", "kv_projection_gemm"]
    assert abs((plan[0]["flops"] + plan[1]["flops"]) / 1e9 - 23.6) < 0.1


def test_fused_plan():
    """Short sequences: projection + attention in one kernel, whose flops
    are the three projections (the attention's are added by the bench) and
    whose bytes are X, the three weights and the concatenated heads."""
    w = WORKLOADS["encoder_self_base"]
    plan, _ = bench.kernel_plan(w, 2)
    assert [p["name"] for p in plan] == ["qkv_projection_attention", "output_projection_gemm"]
    assert plan[0]["flops"] == 2 * 3200 * 512 * 1536
    assert plan[0]["bytes"] == 2 * (3200 * 512 + 512 * 1536 + 3200 * 512)
    assert plan[0]["has_attention"] and not plan[1]["has_attention"]
    w = WORKLOADS["cross_padded_big"]
    plan, _ = bench.kernel_plan(w, 2)
    assert plan[0]["flops"] == 2 * 32 * 96 * 1024 * 1024 + 2 * 32 * 128 * 1024 * 2048
    assert plan[0]["bytes"] == 2 * (32 * 96 * 1024 + 32 * 128 * 1024 + 1024 * 3072 + 32 * 96 * 1024)


def test_buffer_sets_exceed_infinity_cache():
    for name, w in WORKLOADS.items():
        sets = max(2, min(64, math.ceil(2 * bench.MALL_BYTES / bench.set_bytes(w))))
        if w.B * w.n_q > 64:
            assert sets * bench.set_bytes(w) >= 2 * bench.MALL_BYTES or sets == 64, name


def test_gpus_above_one_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_peak_fraction_uses_algorithmic_causal_flops():
    """The long causal attention does (n + 1) / (2n) of the nominal dense
    work; its peak fraction must count only that.  At 110 us, 137.5 GFLOP
    is 49.7% of 2516.6 TFLOP/s, while the nominal count would claim 99%."""
    w = WORKLOADS["long_causal_sdpa"]
    f, _ = bench.attention_accounting(w, None)
    pct = bench.peak_percent(f, 110.0)
    assert abs(pct - 100 * f / 110e-6 / 1e12 / 2516.6) < 1e-9
    assert 49.5 < pct < 50.0
    nominal = bench.peak_percent(w.nominal_attention_flops(), 110.0)
    assert abs(nominal / pct - 2 * 4096 / 4097) < 1e-9


def test_headline_workload_is_long_causal():
    assert bench.DEFAULT_WORKLOAD == "long_causal_sdpa"
    w = WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (w.B, w.h, w.n_q, w.n_k, w.d_k, w.mask) == (4, 16, 4096, 4096, 64, 1)


def test_oracle_threads_follow_host_cores():
    import os
    assert bench.HOST_CORES == len(os.sched_getaffinity(0))
    assert int(os.environ["OMP_NUM_THREADS"]) >= 1
