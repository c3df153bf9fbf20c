"""Benchmark of the multi-head attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch: for a multi-head block
the input projection(s), the fused attention and the output projection; for
bare attention the fused attention kernel; for an encoder layer the block,
residual + LayerNorm, the two FFN GEMMs and residual + LayerNorm; for the
input embedding the fused lookup x sqrt(d_model) + positional encoding; for
the backward pass its two kernels (dQ, then dK/dV) on resident Q, K, V, O,
dO and row log-sum-exp.  The embedding and backward lines carry their
roofline and a null forward-attention metric value.  Inputs are seeded synthetic
tensors of the workload's shapes, resident in GPU memory before timing, and
rotated through enough buffer sets that every step reads memory no earlier
step left in the 256 MB Infinity Cache.

Prints one JSON line: the metric (attention forward TFLOP/s counted as
4*B*h*n_q*n_k*d_k per step, and its fraction of the bf16 MFMA peak), the
per-kernel durations (HIP launch events recorded by the library around each
kernel of each timed step), the roofline of the dominant kernel (for an
MFMA-bound one also the rate the matrix cores sustain in the same run,
measured with the library's matrix-core probe), and the fp64 CPU oracle
timed on a bounded sample of the same workload on the host.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

# The CPU oracle runs on the host cores this process may use.  Its BLAS
# thread pools read these variables when numpy first loads (torch loads it
# too), so they are set here, before either import; a value the environment
# already holds is kept.
HOST_CORES = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(HOST_CORES))

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·h·n_q·n_k·d_k) + % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk (dense bf16 MFMA)
PEAK_FP32_TFLOPS = 157.3       # fp32 vector
PEAK_HBM_GBS = 8000.0          # HBM3E
MALL_BYTES = 256 << 20
# The headline configuration: the long causal attention (B=4, h=16,
# n=4096, d=64, bf16), the largest of the workloads and the one whose
# attention kernel is bound by the matrix units.
DEFAULT_WORKLOAD = "long_causal_sdpa"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0 = auto)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target length of the CPU oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-parity", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="time eager launches only")
    p.add_argument("--no-mfma-probe", action="store_true",
                   help="skip the sustained matrix-core rate measured beside MFMA-bound kernels")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


# ----------------------------------------------------------------------------- accounting

def mha_launches(w):
    """Kernels one multi-head step launches, as the library plans them."""
    from head_attention_forward_amd import _binding as bnd
    n = bnd.lib().mha_forward_launches(w.n_q, w.n_k, w.d_model, 1 if w.self_attn else 0)
    if n < 0:
        raise RuntimeError(f"mha_forward_launches failed with status {n}")
    return n


def layer_launches(w):
    from head_attention_forward_amd import _binding as bnd
    n = bnd.lib().encoder_layer_launches(w.n_q, w.d_model)
    if n < 0:
        raise RuntimeError(f"encoder_layer_launches failed with status {n}")
    return n


def step_launches(w):
    if w.kind in ("sdpa", "embed", "mfma"):
        return 1
    if w.kind == "floor":
        return 2
    if w.kind == "decode":
        from head_attention_forward_amd import _binding as bnd
        return int(bnd.lib().sdpa_decode_launches(w.B, w.h, w.n_q, w.n_k, w.mask))
    if w.kind == "bwd":
        return 2
    if w.kind == "mha_bwd":
        from head_attention_forward_amd import _binding as bnd
        return int(bnd.lib().mha_backward_launches(1 if w.self_attn else 0))
    return layer_launches(w) if w.kind == "layer" else mha_launches(w)


def kernel_plan(w, n_launches=None):
    """Launch order of one step with each kernel's algorithmic flops and bytes
    (bytes: every input element read once, every output written once).  The
    attention's own counts (attention_accounting) are added to the kernel
    named "attention", or to the fused projection + attention kernel."""
    e = 2 if w.dtype == "bf16" else 4
    B, h, nq, nk, dk, dv = w.B, w.h, w.n_q, w.n_k, w.d_k, w.d_v
    plan = []

    def gemm(name, M, K, N, bias=False):
        plan.append(dict(name=name, flops=2.0 * M * K * N,
                         bytes=float(e * (M * K + K * N + M * N + (N if bias else 0))),
                         peak_kind="mfma", has_attention=False))

    def layernorm(name, M, d):
        # read x and the sublayer output, gamma and beta; write the result
        plan.append(dict(name=name, flops=0.0, bytes=float(e * (3 * M * d + 2 * d)),
                         peak_kind="hbm", has_attention=False))

    if w.kind == "mfma":
        # the matrix-core probe: products only (4 waves x 4 chains per workgroup)
        plan.append(dict(name="mfma_probe", flops=float(B) * 16 * w.iters * 2 * 32 * 32 * 16, bytes=0.0,
                         peak_kind="mfma", has_attention=False))
        return plan, None
    if w.kind == "floor":
        # an empty kernel, then one that reads Q, K, V and writes an O-sized output
        plan.append(dict(name="empty_kernel", flops=0.0, bytes=0.0, peak_kind="hbm", has_attention=False))
        plan.append(dict(name="xor3_copy", flops=0.0,
                         bytes=float(e * B * h * (nq * dk + nk * (dk + dv) + nq * dv)),
                         peak_kind="hbm", has_attention=False))
        return plan, None
    if w.kind == "decode":
        plan.append(dict(name="attention", flops=0.0, bytes=0.0, peak_kind="mfma", has_attention=True))
        if (n_launches or step_launches(w)) == 2:
            # the partial states (m, l and 32 accumulators per lane, 64 lanes per
            # workgroup) of every split, read once; O written
            from head_attention_forward_amd import _binding as bnd
            nb = int(bnd.lib().sdpa_decode_workspace_bytes(B, h, nq, nk))
            plan.append(dict(name="decode_merge", flops=0.0, bytes=float(nb + e * B * h * nq * dv),
                             peak_kind="hbm", has_attention=False))
        return plan, None
    if w.kind == "sdpa":
        plan.append(dict(name="attention", flops=0.0, bytes=0.0,
                         peak_kind="mfma" if w.dtype == "bf16" else "fp32", has_attention=True))
        return plan, None
    if w.kind == "bwd":
        # per visible (query, key) pair the dQ kernel runs three 2-d flop
        # products (S, dP, dQ), the dK/dV kernel four (S, dP, dV, dK)
        pairs = bwd_pairs(w)
        rows_q, rows_k = B * h * nq, B * h * nk
        plan.append(dict(name="backward_dq", flops=6.0 * pairs * dk,
                         bytes=float(e * rows_q * dk * 4 + 4 * rows_q * 2 + e * rows_k * dk * 2),
                         peak_kind="mfma", has_attention=False))
        plan.append(dict(name="backward_dkdv", flops=8.0 * pairs * dk,
                         bytes=float(e * rows_k * dk * 4 + e * rows_q * dk * 2 + 4 * rows_q * 2),
                         peak_kind="mfma", has_attention=False))
        return plan, None
    if w.kind == "mha_bwd":
        if not w.self_attn:
            raise ValueError("the block-backward bench covers self-attention")
        M, dm, hd = B * nq, w.d_model, h * dk
        pairs = bwd_pairs(w)
        # one batched transpose: W^O, C, W^Q, W^K, W^V, X
        plan.append(dict(name="transposes", flops=0.0, bytes=float(2 * e * (4 * hd * dm + 2 * M * dm)),
                         peak_kind="hbm", has_attention=False))
        def splits(Mo, No, Ko):  # the library's split-K factor for a weight gradient
            return 8

        def reduce(name, Mo, No):  # read the fp32 partials, write the bf16 result
            plan.append(dict(name=name, flops=0.0, bytes=float(4 * splits(Mo, No, M) * Mo * No + e * Mo * No),
                             peak_kind="hbm", has_attention=False))

        def group(name, n):  # the last n entries run as one launch
            parts = plan[-n:]
            del plan[-n:]
            plan.append(dict(name=name, flops=sum(q["flops"] for q in parts),
                             bytes=sum(q["bytes"] for q in parts), peak_kind="mfma", has_attention=False))
        # one launch: dC = dY W^O^T and the split-K partials of dW^O = C^T dY
        gemm("do", M, dm, hd)
        gemm("dwo", hd, M, dm)
        group("do_dwo_gemm", 2)
        plan.append(dict(name="backward_dq", flops=6.0 * pairs * dk,
                         bytes=float(e * B * h * nq * dk * 4 + 8 * B * h * nq + e * B * h * nk * dk * 2),
                         peak_kind="mfma", has_attention=False))
        plan.append(dict(name="backward_dkdv", flops=8.0 * pairs * dk,
                         bytes=float(e * B * h * nk * dk * 4 + e * B * h * nq * dk * 2 + 8 * B * h * nq),
                         peak_kind="mfma", has_attention=False))
        # one launch: dX, the split-K partials of dW^Q|dW^K|dW^V, the reduction of dW^O
        gemm("dx", M, 3 * hd, dm)
        gemm("dw", dm, M, 3 * hd)
        reduce("dwo_reduce", hd, dm)
        group("dx_dw_gemm", 3)
        reduce("dw_reduce", dm, 3 * hd)
        return plan, None
    if w.kind == "embed":
        # gather one table row per token, write one row per token, read the ids
        plan.append(dict(name="embed_positional", flops=0.0,
                         bytes=float(2 * e * B * nq * w.d_model + 4 * B * nq),
                         peak_kind="hbm", has_attention=False))
        return plan, None
    n = step_launches(w) if n_launches is None else n_launches
    if w.kind == "layer":
        n -= 4  # the block's own launches
    if n == 2:
        dm = w.d_model
        flops = 2.0 * B * nq * dm * h * dk + 2.0 * B * nk * dm * h * (dk + dv)
        x_bytes = B * nq * dm + (0 if w.self_attn else B * nk * dm)
        byts = float(e * (x_bytes + dm * h * (2 * dk + dv) + B * nq * h * dv))
        plan.append(dict(name="qkv_projection_attention", flops=flops, bytes=byts,
                         peak_kind="mfma", has_attention=True))
    else:
        if n == 3:
            gemm("qkv_projection_gemm", B * nq, w.d_model, h * (2 * dk + dv))
        else:
            gemm("q_projection_gemm", B * nq, w.d_model, h * dk)
            gemm("kv_projection_gemm", B * nk, w.d_model, h * (dk + dv))
        plan.append(dict(name="attention", flops=0.0, bytes=0.0, peak_kind="mfma", has_attention=True))
    gemm("output_projection_gemm", B * nq, h * dv, w.d_model)
    if w.kind == "layer":
        M = B * nq
        layernorm("residual_layernorm_1", M, w.d_model)
        gemm("ffn_gemm_1", M, w.d_model, w.d_ff, bias=True)
        gemm("ffn_gemm_2", M, w.d_ff, w.d_model, bias=True)
        layernorm("residual_layernorm_2", M, w.d_model)
    return plan, None


def bwd_pairs(w, key_lengths=None):
    """Visible (query, key) pairs of all heads."""
    L = [w.n_k] * w.B if key_lengths is None else [int(x) for x in key_lengths]
    pairs = 0.0
    for b in range(w.B):
        if w.mask & 1:
            full = min(L[b], w.n_q)
            pairs += full * (full + 1) / 2.0 + max(0, w.n_q - full) * L[b]
        else:
            pairs += w.n_q * L[b]
    return pairs * w.h


def block_bwd_flops(w, key_lengths=None):
    """Algorithmic flops of the block's backward: two products per forward
    projection (dX and dW for each of W^Q, W^K, W^V, W^O) and five per
    visible pair of the attention."""
    M, dm, hd = w.B * w.n_q, w.d_model, w.h * w.d_k
    return 2.0 * (2.0 * M * dm * hd * 4) + 10.0 * bwd_pairs(w, key_lengths) * w.d_k


def attention_accounting(w, key_lengths):
    """Algorithmic flops (visible pairs x 2(d_k + d_v)) and bytes (read Q,
    the K/V rows some query can see, write O) of one attention launch."""
    e = 2 if w.dtype == "bf16" else 4
    B, h, nq, nk, dk, dv = w.B, w.h, w.n_q, w.n_k, w.d_k, w.d_v
    if w.mask & 2:
        L = [int(x) for x in key_lengths]
    else:
        L = [nk] * B
    pairs = 0.0
    kv_rows = 0
    for b in range(B):
        if w.mask & 1:
            Lb = L[b]
            # query i sees min(i + 1, L_b) keys
            full = min(Lb, nq)
            pairs += full * (full + 1) / 2.0 + max(0, nq - full) * Lb
        else:
            pairs += nq * L[b]
        kv_rows += L[b]
    flops = 2.0 * pairs * (dk + dv) * h
    bytes_ = e * h * (B * nq * dk + kv_rows * (dk + dv) + B * nq * dv)
    return flops, float(bytes_)


def peak_percent(flops, us, peak_tflops=None):
    """flops done in us microseconds, as a percent of a peak in TFLOP/s
    (the bf16 dense MFMA peak by default)."""
    peak = PEAK_BF16_TFLOPS if peak_tflops is None else peak_tflops
    return 100.0 * flops / (us * 1e-6) / 1e12 / peak


# ----------------------------------------------------------------------------- steps

class Step:
    """Pre-marshalled launches of one workload over rotating buffer sets."""

    def __init__(self, w, x, dev, sets):
        import torch
        from head_attention_forward_amd import _binding as bnd
        self.w = w
        self.lib = bnd.lib()
        self.sets = []
        self.keep = []
        kl = x["key_lengths"]
        if kl is not None:
            self.kl_arr = (ctypes.c_int32 * w.B)(*[int(v) for v in kl])
            self.kl = ctypes.cast(self.kl_arr, ctypes.c_void_p)
        else:
            self.kl = None
        P = ctypes.c_void_p
        for _ in range(sets):
            if w.kind == "mfma":
                sink = torch.empty((w.B, 256), dtype=torch.float32, device=dev)
                self.keep.append((None, None, None, sink))
                self.sets.append((1 if w.operands == "sparse" else 0, w.B, w.iters, P(sink.data_ptr())))
                continue
            if w.kind == "floor":
                Q, K, V = (x[k].to(dev) for k in ("Q", "K", "V"))
                O = torch.empty_like(Q)
                self.keep.append((Q, K, V, O))
                self.sets.append((P(Q.data_ptr()), P(K.data_ptr()), P(V.data_ptr()), P(O.data_ptr()),
                                  Q.numel() * Q.element_size(), floor_grid(w)))
            elif w.kind == "decode":
                Q, K, V = (x[k].to(dev) for k in ("Q", "K", "V"))
                O = torch.empty((w.B, w.h, w.n_q, w.d_v), dtype=Q.dtype, device=dev)
                nbytes = int(self.lib.sdpa_decode_workspace_bytes(w.B, w.h, w.n_q, w.n_k))
                ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
                self.keep.append((Q, K, V, O, ws))
                self.sets.append((P(Q.data_ptr()), P(K.data_ptr()), P(V.data_ptr()), P(O.data_ptr()),
                                  w.B, w.h, w.n_q, w.n_k, w.d_k, w.d_v, float(x["scale"]), w.mask,
                                  self.kl, bnd.DTYPE_BF16, P(ws.data_ptr()), nbytes))
            elif w.kind == "sdpa":
                Q, K, V = (x[k].to(dev) for k in ("Q", "K", "V"))
                O = torch.empty((w.B, w.h, w.n_q, w.d_v), dtype=Q.dtype, device=dev)
                self.keep.append((Q, K, V, O))
                code = bnd.DTYPE_BF16 if w.dtype == "bf16" else bnd.DTYPE_F32
                self.sets.append((P(Q.data_ptr()), P(K.data_ptr()), P(V.data_ptr()), P(O.data_ptr()),
                                  w.B, w.h, w.n_q, w.n_k, w.d_k, w.d_v, float(x["scale"]), w.mask,
                                  self.kl, code))
            elif w.kind == "bwd":
                Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
                O = torch.empty_like(Q)
                lse = torch.empty((w.B, w.h, w.n_q), dtype=torch.float32, device=dev)
                st = self.lib.sdpa_forward_lse(P(Q.data_ptr()), P(K.data_ptr()), P(V.data_ptr()),
                                               P(O.data_ptr()), P(lse.data_ptr()), w.B, w.h, w.n_q,
                                               w.n_k, w.d_k, w.d_v, float(x["scale"]), w.mask, self.kl,
                                               bnd.DTYPE_BF16, P(torch.cuda.current_stream().cuda_stream))
                if st != 0:
                    raise RuntimeError(f"sdpa_forward_lse failed with status {st}")
                dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
                nbytes = int(self.lib.sdpa_backward_workspace_bytes(w.B, w.h, w.n_q))
                ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
                self.keep.append((Q, K, V, dQ, dK, dV, O, lse, dO, ws))
                self.sets.append((P(Q.data_ptr()), P(K.data_ptr()), P(V.data_ptr()), P(O.data_ptr()),
                                  P(dO.data_ptr()), P(lse.data_ptr()), P(dQ.data_ptr()),
                                  P(dK.data_ptr()), P(dV.data_ptr()), w.B, w.h, w.n_q, w.n_k, w.d_k,
                                  w.d_v, float(x["scale"]), w.mask, self.kl, bnd.DTYPE_BF16,
                                  P(ws.data_ptr()), nbytes))
            elif w.kind == "mha_bwd":
                Xq = x["X_q"].to(dev)
                Ws = [x[k].to(dev) for k in ("Wq", "Wk", "Wv", "Wo")]
                dY = x["dY"].to(dev)
                Y = torch.empty((w.B, w.n_q, w.d_model), dtype=Xq.dtype, device=dev)
                tb = int(self.lib.mha_train_workspace_bytes(w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v,
                                                            bnd.DTYPE_BF16))
                state = torch.empty(tb, dtype=torch.uint8, device=dev)
                sp0 = P(torch.cuda.current_stream().cuda_stream)
                st = self.lib.mha_forward_train(P(Xq.data_ptr()), P(Xq.data_ptr()),
                                                *[P(t.data_ptr()) for t in Ws], P(Y.data_ptr()), w.B,
                                                w.n_q, w.n_k, w.d_model, w.h, w.d_k, w.d_v, w.mask,
                                                self.kl, bnd.DTYPE_BF16, P(state.data_ptr()), tb, sp0)
                if st != 0:
                    raise RuntimeError(f"mha_forward_train failed with status {st}")
                dX = torch.empty_like(Xq)
                dW = [torch.empty_like(t) for t in Ws]
                bb = int(self.lib.mha_backward_workspace_bytes(w.B, w.n_q, w.n_k, w.d_model, w.h,
                                                               w.d_k, w.d_v, 1, bnd.DTYPE_BF16))
                ws = torch.empty(bb, dtype=torch.uint8, device=dev)
                self.keep.append((Xq, Ws, dY, dX, *dW, state, ws, Y))
                self.sets.append((P(Xq.data_ptr()), P(Xq.data_ptr()), *[P(t.data_ptr()) for t in Ws],
                                  P(dY.data_ptr()), P(dX.data_ptr()), None,
                                  *[P(t.data_ptr()) for t in dW], w.B, w.n_q, w.n_k, w.d_model, w.h,
                                  w.d_k, w.d_v, w.mask, self.kl, bnd.DTYPE_BF16, P(state.data_ptr()),
                                  tb, P(ws.data_ptr()), bb))
            elif w.kind == "embed":
                T = x["tokens"].to(dev)
                E = x["E"].to(dev)
                O = torch.empty((w.B, w.n_q, w.d_model), dtype=E.dtype, device=dev)
                self.keep.append((T, E, None, O))
                code = bnd.DTYPE_BF16 if w.dtype == "bf16" else bnd.DTYPE_F32
                self.sets.append((P(T.data_ptr()), P(E.data_ptr()), P(O.data_ptr()), w.B, w.n_q,
                                  w.vocab, w.d_model, int(x["pos0"]), code))
            elif w.kind == "layer":
                X = x["X"].to(dev)
                ps = [x[k].to(dev) for k in bnd.LAYER_PARAMS]
                Y = torch.empty_like(X)
                nbytes = bnd.encoder_layer_workspace_bytes(w.B, w.n_q, w.d_model, w.h, w.d_k,
                                                           w.d_v, w.d_ff)
                ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
                self.keep.append((X, ps, ws, Y))
                self.sets.append((P(X.data_ptr()), *[P(t.data_ptr()) for t in ps], P(Y.data_ptr()),
                                  w.B, w.n_q, w.d_model, w.h, w.d_k, w.d_v, w.d_ff, float(w.eps),
                                  w.mask, self.kl, bnd.DTYPE_BF16, P(ws.data_ptr()), nbytes))
            else:
                Xq = x["X_q"].to(dev)
                Xkv = Xq if w.self_attn else x["X_kv"].to(dev)
                Ws = [x[k].to(dev) for k in ("Wq", "Wk", "Wv", "Wo")]
                Y = torch.empty((w.B, w.n_q, w.d_model), dtype=Xq.dtype, device=dev)
                ws = bnd.alloc_workspace(w.B, w.n_q, w.n_k, w.h, w.d_k, w.d_v, dev)
                self.keep.append((Xq, Xkv, Ws, Y, ws))
                self.sets.append((P(Xq.data_ptr()), P(Xkv.data_ptr()),
                                  *[P(t.data_ptr()) for t in Ws], P(Y.data_ptr()),
                                  w.B, w.n_q, w.n_k, w.d_model, w.h, w.d_k, w.d_v, w.mask, self.kl,
                                  bnd.DTYPE_BF16, P(ws.data_ptr()), ws.numel()))
        self.n_launches = step_launches(w)
        names = {"floor": "mha_floor_probe", "mfma": "mha_mfma_probe", "decode": "sdpa_decode",
                 "sdpa": "sdpa_forward", "mha": "mha_forward", "layer": "encoder_layer_forward",
                 "embed": "embed_positional_forward", "bwd": "sdpa_backward",
                 "mha_bwd": "mha_backward"}
        self.entry = names[w.kind]

    def output(self, i):
        return self.keep[i][3]

    def parity_output(self, i):
        if self.w.kind == "bwd":
            return self.keep[i][3:6]
        if self.w.kind == "mha_bwd":
            return self.keep[i][3:8]  # dX, dWq, dWk, dWv, dWo
        return self.keep[i][3]

    def run(self, i, stream):
        if self.w.kind == "floor":  # the empty kernel, then the byte mover
            q, k, v, o, nbytes, grid = self.sets[i]
            for kind in (0, 1):
                st = self.lib.mha_floor_probe(kind, q, k, v, o, nbytes, grid, stream)
                if st != 0:
                    raise RuntimeError(f"launch failed with status {st}")
            return
        st = getattr(self.lib, self.entry)(*self.sets[i], stream)
        if st != 0:
            raise RuntimeError(f"launch failed with status {st}")

    def run_timed(self, i, stream, events_ptr, cap):
        if self.w.kind == "floor":
            q, k, v, o, nbytes, grid = self.sets[i]
            n = ctypes.c_int()
            for kind in (0, 1):
                ev = ctypes.c_void_p(events_ptr.value + kind * 2 * ctypes.sizeof(ctypes.c_void_p))
                st = self.lib.mha_floor_probe_timed(kind, q, k, v, o, nbytes, grid, stream, ev, 2,
                                                    ctypes.byref(n))
                if st != 0 or n.value != 1:
                    raise RuntimeError(f"timed launch failed with status {st}")
            return
        f = getattr(self.lib, self.entry + "_timed")
        n = ctypes.c_int()
        st = f(*self.sets[i], stream, events_ptr, cap, ctypes.byref(n))
        if st != 0 or n.value != self.n_launches:
            raise RuntimeError(f"timed launch failed with status {st} ({n.value} launches)")


def floor_grid(w):
    """Workgroups of the attention launch at w's shape: one per (batch, head)
    and block of 128 queries."""
    return w.B * w.h * ((w.n_q + 127) // 128)


def set_bytes(w):
    e = 2 if w.dtype == "bf16" else 4
    if w.kind == "mfma":
        return 4 * w.B * 256
    if w.kind == "mha_bwd":
        M, dm, hd = w.B * w.n_q, w.d_model, w.h * w.d_k
        return e * (3 * M * dm + 8 * dm * hd + 4 * M * hd + 2 * M * 3 * hd + 3 * M * hd + hd * M +
                    3 * hd * dm + dm * M)
    if w.kind == "bwd":
        return e * w.B * w.h * (w.n_q * 64 * 4 + w.n_k * 64 * 4) + 8 * w.B * w.h * w.n_q
    if w.kind == "embed":
        return e * (w.vocab * w.d_model + w.B * w.n_q * w.d_model) + 4 * w.B * w.n_q
    if w.kind in ("sdpa", "decode", "floor"):
        return e * w.B * w.h * (w.n_q * (w.d_k + w.d_v) + w.n_k * (w.d_k + w.d_v))
    xs = w.B * w.n_q * w.d_model * (1 if w.self_attn else 1) + (0 if w.self_attn else w.B * w.n_k * w.d_model)
    ws = w.B * w.h * (w.n_q * w.d_k + w.n_k * (w.d_k + w.d_v) + w.n_q * w.d_v)
    weights = w.d_model * w.h * (2 * w.d_k + w.d_v) + w.h * w.d_v * w.d_model
    total = xs + ws + weights + w.B * w.n_q * w.d_model
    if w.kind == "layer":
        M, D, F = w.B * w.n_q, w.d_model, w.d_ff
        total += 2 * M * D + M * F + 2 * D * F + F + 5 * D  # S, x1, H; FFN and LayerNorm parameters
    return e * total


def layer_flops(w):
    """All matrix-product flops of one encoder-layer step (projections,
    attention at nominal dense count, FFN)."""
    M, D, F = w.B * w.n_q, w.d_model, w.d_ff
    proj = 2.0 * M * D * w.h * (2 * w.d_k + w.d_v) + 2.0 * M * w.h * w.d_v * D
    return proj + w.nominal_attention_flops() + 4.0 * M * D * F


# ----------------------------------------------------------------------------- parity

def parity_check(w, x, out):
    """One step's output against the fp64 oracle (sampled rows for shapes too
    large to evaluate whole)."""
    import numpy as np
    import oracle
    from head_attention_forward_amd.workloads import to_f64
    kl = None if x["key_lengths"] is None else x["key_lengths"].numpy()
    rows = "all"
    if w.kind == "mfma":  # every workgroup of the probe writes the same 256 finite values
        import torch
        o = out.cpu()
        ok = bool(torch.isfinite(o).all()) and bool((o == o[0:1]).all())
        return dict(max_abs=0.0 if ok else None, rel_l2=0.0 if ok else None, ok=ok,
                    rows="all (equal across workgroups, finite)")
    if w.kind == "floor":  # the byte mover's output, bit for bit (no attention arithmetic)
        import torch
        want = x["Q"].view(torch.int16) ^ x["K"].view(torch.int16) ^ x["V"].view(torch.int16)
        ok = bool(torch.equal(out.cpu().view(torch.int16), want))
        return dict(max_abs=0.0 if ok else None, rel_l2=0.0 if ok else None, ok=ok,
                    rows="all (xor of Q, K, V, bit for bit)")
    if w.kind == "mha_bwd":
        # whole gradients; bar of the block-gradient tests: rel-L2 <= 4u and
        # every element within 8u max|want|, u = 2^-8
        u = 2.0 ** -8
        want = oracle.mha_backward_ref(to_f64(x["X_q"]), to_f64(x["X_q"]),
                                       *[to_f64(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")], w.h,
                                       to_f64(x["dY"]), w.mask, kl)
        wants = [want[0] + want[1]] + list(want[2:])
        worst, rel_max, max_abs = 0.0, 0.0, 0.0
        for got_t, want_t in zip(out, wants):
            got = to_f64(got_t)
            err = np.abs(got - want_t)
            worst = max(worst, float(err.max()) / (8 * u * float(np.abs(want_t).max())))
            rel_max = max(rel_max, float(np.linalg.norm(got - want_t) / np.linalg.norm(want_t)))
            max_abs = max(max_abs, float(err.max()))
        return dict(max_abs=max_abs, rel_l2=rel_max, worst_over_bound=worst,
                    ok=bool(worst <= 1.0 and rel_max <= 4 * u), rows="all (dX, dWq, dWk, dWv, dWo)")
    if w.kind == "bwd":
        # two sampled (batch, head) pairs, whole gradients; the test bar:
        # rel-L2 <= 2u and every element within 4u max(max|want|, 1), u = 2^-8
        u = 2.0 ** -8
        worst, rel_max, max_abs = 0.0, 0.0, 0.0
        picks = [(0, 0), (w.B - 1, w.h - 1)]
        for b, hh in picks:
            sl = lambda t: to_f64(t[b:b + 1, hh:hh + 1])  # noqa: E731
            want = oracle.sdpa_backward_ref(sl(x["Q"]), sl(x["K"]), sl(x["V"]), sl(x["dO"]),
                                            x["scale"], w.mask, None if kl is None else kl[b:b + 1])
            for got_t, want_t in zip(out, want):
                got = to_f64(got_t[b:b + 1, hh:hh + 1])
                err = np.abs(got - want_t)
                worst = max(worst, float(err.max()) / (4 * u * max(float(np.abs(want_t).max()), 1.0)))
                rel_max = max(rel_max, float(np.linalg.norm(got - want_t) / np.linalg.norm(want_t)))
                max_abs = max(max_abs, float(err.max()))
        return dict(max_abs=max_abs, rel_l2=rel_max, worst_over_bound=worst,
                    ok=bool(worst <= 1.0 and rel_max <= 2 * u), rows="2 sampled (batch, head) pairs")
    if w.kind == "embed":
        want = oracle.embed_positional_ref(x["tokens"].numpy(), to_f64(x["E"]), x["pos0"])
        got = to_f64(out)
        err = np.abs(got - want)
        # one rounding of the exact value (double-precision encoding, fp32 sum)
        u = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -24
        worst = float((err / (u * np.abs(want) + 1e-5)).max())
        rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        return dict(max_abs=float(err.max()), rel_l2=rel, worst_over_bound=worst,
                    ok=bool(worst <= 1.0), rows=rows)
    if w.kind == "layer":
        from head_attention_forward_amd._binding import LAYER_PARAMS
        p = [to_f64(x[k]) for k in LAYER_PARAMS]
        want = oracle.encoder_layer_ref(to_f64(x["X"]), *p[:4], w.h, *p[4:], w.eps, w.mask, kl)
        got = to_f64(out)
        err = got - want
        # elementwise 2e-2 + 2u|want| (u = 2^-8, bf16): LayerNorm outputs reach
        # magnitude ~5, where the output's own rounding is already u * 5
        worst = float((np.abs(err) / (2e-2 + 2 * 2.0 ** -8 * np.abs(want))).max())
        rel = float(np.linalg.norm(err) / np.linalg.norm(want))
        return dict(max_abs=float(np.abs(err).max()), rel_l2=rel, worst_over_bound=worst,
                    ok=bool(worst <= 1.0 and rel <= 5e-3), rows=rows)
    if w.kind == "mha":
        want = oracle.mha_ref(to_f64(x["X_q"]), to_f64(x["X_kv"]),
                              *[to_f64(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")], w.h, w.mask, kl)
        got = to_f64(out)
    elif w.B * w.h * w.n_q * w.n_k <= (1 << 24):
        want = oracle.sdpa_ref(to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"]), x["scale"], w.mask, kl)
        got = to_f64(out)
    else:
        rng = np.random.default_rng(1)
        idx = np.stack([rng.integers(0, w.B, 256), rng.integers(0, w.h, 256),
                        rng.integers(0, w.n_q, 256)], axis=1)
        idx[0] = (0, 0, w.n_q - 1)
        rows = "256 sampled"
        want = oracle.sdpa_ref_rows(to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"]), x["scale"],
                                    w.mask, kl, idx)
        got = to_f64(out[idx[:, 0], idx[:, 1], idx[:, 2]])
    err = got - want
    max_abs = float(np.abs(err).max())
    rel = float(np.linalg.norm(err) / np.linalg.norm(want))
    if w.dtype == "bf16":
        ok = max_abs <= 2e-2 and rel <= 5e-3
    else:
        ok = max_abs <= 1e-5
    return dict(max_abs=max_abs, rel_l2=rel, ok=bool(ok), rows=rows)


# ----------------------------------------------------------------------------- cpu baseline

def blas_threads():
    """Threads of numpy's BLAS pool as it actually runs (threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(w, x, target_s):
    """The oracle, as it is, on a bounded sample of the workload, sized to
    roughly target_s seconds: whole multi-head blocks (the first b
    sequences, or the whole batch repeated) or (batch, head) pairs of bare
    attention in order (the whole set repeated when it is shorter)."""
    import numpy as np
    import oracle
    from head_attention_forward_amd.workloads import to_f64
    threads = blas_threads()
    kl = None if x["key_lengths"] is None else x["key_lengths"].numpy()

    if w.kind == "mha_bwd":
        Xq = to_f64(x["X_q"])
        Ws = [to_f64(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")]
        dY = to_f64(x["dY"])

        def run(b):
            oracle.mha_backward_ref(Xq[:b], Xq[:b], *Ws, w.h, dY[:b], w.mask,
                                    None if kl is None else kl[:b])
        run(1)
        t0 = time.perf_counter()
        run(1)
        t1 = max(time.perf_counter() - t0, 1e-6)
        n = int(max(1, min(w.B, target_s / t1)))
        t0 = time.perf_counter()
        run(n)
        t = time.perf_counter() - t0
        flops = block_bwd_flops(w) / w.B * n
        return dict(value=flops / t / 1e12, unit="TFLOP/s", cores=int(threads), host_cores=HOST_CORES, kind="oracle",
                    sample=f"{n} of {w.B} sequences, block backward; {t:.2f} s, numpy float64"
                           " (algorithmic flops of the block's backward)", seconds=round(t, 3))
    if w.kind == "bwd":
        Q, K, V, dO = (to_f64(x[k]) for k in ("Q", "K", "V", "dO"))

        def run_pairs(n):  # the first n (batch, head) pairs
            done = 0
            for b in range(w.B):
                for hh in range(w.h):
                    if done >= n:
                        return
                    oracle.sdpa_backward_ref(Q[b:b + 1, hh:hh + 1], K[b:b + 1, hh:hh + 1],
                                             V[b:b + 1, hh:hh + 1], dO[b:b + 1, hh:hh + 1], x["scale"],
                                             w.mask, None if kl is None else kl[b:b + 1])
                    done += 1
        t0 = time.perf_counter()
        run_pairs(1)
        t1 = max(time.perf_counter() - t0, 1e-6)
        n = int(max(1, min(w.B * w.h, target_s / t1)))
        t0 = time.perf_counter()
        run_pairs(n)
        t = time.perf_counter() - t0
        flops = 10.0 * bwd_pairs(w) / (w.B * w.h) * w.d_k * n
        return dict(value=flops / t / 1e12, unit="TFLOP/s", cores=int(threads), host_cores=HOST_CORES, kind="oracle",
                    sample=f"{n} of {w.B * w.h} (batch, head) pairs, backward; {t:.2f} s, numpy float64"
                           " (algorithmic backward flops: 5 products per visible pair)",
                    seconds=round(t, 3))
    if w.kind == "embed":
        tokens, E = x["tokens"].numpy(), to_f64(x["E"])
        e = 2 if w.dtype == "bf16" else 4

        def run(b):
            oracle.embed_positional_ref(tokens[:b], E, x["pos0"])
        # in the unit of this workload's roofline: algorithmic GB/s
        run(1)
        t0 = time.perf_counter()
        run(w.B)
        t1 = max(time.perf_counter() - t0, 1e-6)
        reps = int(max(1, min(10000, target_s / t1)))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(w.B)
        t = time.perf_counter() - t0
        byts = float(2 * e * w.B * w.n_q * w.d_model + 4 * w.B * w.n_q) * reps
        return dict(value=byts / t / 1e9, unit="GB/s", cores=int(threads), host_cores=HOST_CORES, kind="oracle",
                    sample=f"{w.B} of {w.B} sequences, {reps} passes; {t:.2f} s, numpy float64",
                    seconds=round(t, 3))
    if w.kind == "layer":
        from head_attention_forward_amd._binding import LAYER_PARAMS
        X = to_f64(x["X"])
        p = [to_f64(x[k]) for k in LAYER_PARAMS]

        def run(b):
            oracle.encoder_layer_ref(X[:b], *p[:4], w.h, *p[4:], w.eps, w.mask,
                                     None if kl is None else kl[:b])
        unit_flops = 4.0 * w.h * w.n_q * w.n_k * w.d_k  # per sequence, the metric's count
        n_units, what = w.B, "sequences (whole encoder layers)"
    elif w.kind == "mha":
        Xq, Xkv = to_f64(x["X_q"]), to_f64(x["X_kv"])
        Ws = [to_f64(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")]

        def run(b):
            oracle.mha_ref(Xq[:b], Xkv[:b], *Ws, w.h, w.mask, None if kl is None else kl[:b])
        unit_flops = 4.0 * w.h * w.n_q * w.n_k * w.d_k  # per sequence
        n_units, what = w.B, "sequences"
    else:
        Q, K, V = to_f64(x["Q"]), to_f64(x["K"]), to_f64(x["V"])

        def run(n):  # the first n (batch, head) pairs, batch by batch
            done = 0
            for b in range(w.B):
                if done >= n:
                    break
                k = min(w.h, n - done)
                oracle.sdpa_ref(Q[b:b + 1, :k], K[b:b + 1, :k], V[b:b + 1, :k], x["scale"], w.mask,
                                None if kl is None else kl[b:b + 1])
                done += k
        unit_flops = 4.0 * w.n_q * w.n_k * w.d_k  # per (batch, head) pair
        n_units, what = w.B * w.h, "(batch, head) pairs"

    run(1)  # warm-up (thread pools, first-touch)
    t0 = time.perf_counter()
    run(1)
    t1 = max(time.perf_counter() - t0, 1e-6)
    units = int(max(1, min(n_units, target_s / t1)))
    # whole passes until target_s has elapsed (a batched pass runs faster
    # per unit than the single unit timed above)
    reps = 0
    t0 = time.perf_counter()
    while True:
        run(units)
        reps += 1
        t = time.perf_counter() - t0
        if units < n_units or t >= target_s or reps >= 1000:
            break
    flops = unit_flops * units * reps
    sample = f"{units} of {n_units} {what}" + (f", {reps} passes" if reps > 1 else "")
    return dict(value=flops / t / 1e12, unit="TFLOP/s", cores=int(threads), host_cores=HOST_CORES, kind="oracle",
                sample=sample + f"; {t:.2f} s, numpy float64", seconds=round(t, 3))


# ----------------------------------------------------------------------------- traffic

# HIP sources that determine a timed kernel's code and launch shape, by kernel
# name (the name recorded with each counter entry).
_COMMON_SOURCES = ("device.h", "kernels.h")
KERNEL_SOURCES = {
    "attn_fwd_bf16_d64_kernel": ("attn_bf16.hip", "attn_decode_bf16.hip", "wave_attention.h", "device_info.hip"),
    "attn_decode_bf16_d64_kernel": ("attn_decode_bf16.hip", "attn_bf16.hip", "wave_attention.h",
                                    "mha_api.hip", "device_info.hip"),
    "attn_decode_merge_kernel": ("attn_decode_bf16.hip", "wave_attention.h", "mha_api.hip",
                                 "device_info.hip"),
    "attn_fwd_f32_d64_kernel": ("attn_f32.hip", "device_info.hip"),
    "attn_fwd_f32_d64_wave_kernel": ("attn_f32.hip", "device_info.hip"),
    "proj_attn_bf16_kernel": ("proj_attn_bf16.hip", "wave_attention.h", "mha_api.hip", "device_info.hip"),
    "proj_attn2_bf16_kernel": ("proj_attn_bf16.hip", "wave_attention.h", "mha_api.hip", "device_info.hip"),
    "gemm_bf16_kernel": ("gemm_bf16.hip", "mha_api.hip"),
    "add_layernorm_bf16_kernel": ("add_layernorm_bf16.hip", "mha_api.hip"),
    "embed_positional_kernel": ("embed_positional.hip", "mha_api.hip"),
    "attn_bwd_dq_kernel": ("attn_bwd_bf16.hip", "wave_attention.h", "mha_api.hip"),
    "attn_bwd_dkdv_kernel": ("attn_bwd_bf16.hip", "wave_attention.h", "mha_api.hip"),
    "transpose_bf16_kernel": ("transpose_bf16.hip", "mha_api.hip"),
    "gemm_splitk_reduce_kernel": ("gemm_bf16.hip", "mha_api.hip"),
    "gemm_group_kernel": ("gemm_bf16.hip", "mha_api.hip"),
    "floor_empty_kernel": ("floor_probe.hip",),
    "floor_xor3_kernel": ("floor_probe.hip",),
    "probe_mfma_kernel": ("floor_probe.hip",),
}


def sources_of(kernel_name):
    return KERNEL_SOURCES.get(kernel_name.split("<", 1)[0].strip())


def kernel_source_sha(names=None):
    """Hash of the named HIP sources (all of them when names is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "head_attention_forward_amd", "csrc")
    if names is None:
        files = sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".h")))
    else:
        files = sorted(set(names) | set(_COMMON_SOURCES))
    for name in files:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current sources of that kernel; otherwise None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except Exception:
        return None
    ent = rec.get("entries", {}).get(f"{workload}/{kernel}")
    if ent is None:
        return None
    files = sources_of(ent.get("kernel", ""))
    if files is None or ent.get("source_sha") != kernel_source_sha(files):
        return None
    return float(ent["bytes_per_launch"])


# ----------------------------------------------------------------------------- main

PROBE_ITERS = 16384  # products per chain of the matrix-core probe (a launch of a few ms)


def sustained_mfma_tflops(lib, sp, dev, launches=3):
    """The dense bf16 rate the matrix cores sustain on this device now: the
    matrix-core probe (mha_mfma_probe, random-bit operands, four waves of
    four independent product chains per workgroup, four workgroups per
    compute unit, no memory traffic) timed with launch events on the bench
    stream, one untimed launch first.  Returns TFLOP/s."""
    import numpy as np
    import torch
    from head_attention_forward_amd import _hip
    grid = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty((grid, 256), dtype=torch.float32, device=dev)
    P = ctypes.c_void_p(sink.data_ptr())
    if lib.mha_mfma_probe(0, grid, PROBE_ITERS, P, sp) != 0:
        raise RuntimeError("matrix-core probe launch failed")
    pool = _hip.EventPool(2 * launches)
    n = ctypes.c_int()
    for i in range(launches):
        st = lib.mha_mfma_probe_timed(0, grid, PROBE_ITERS, P, sp, pool.ptr(2 * i), 2, ctypes.byref(n))
        if st != 0 or n.value != 1:
            raise RuntimeError(f"timed matrix-core probe failed with status {st}")
    torch.cuda.synchronize()
    ms = float(np.mean([pool.elapsed_ms(2 * i, 2 * i + 1) for i in range(launches)]))
    pool.close()
    flops = float(grid) * 16 * PROBE_ITERS * 2 * 32 * 32 * 16
    return flops / (ms * 1e-3) / 1e12


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by (batch, head) with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from head_attention_forward_amd import _hip
    from head_attention_forward_amd.workloads import WORKLOADS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload not in WORKLOADS:
        print(f"unknown workload {args.workload}; choose from {sorted(WORKLOADS)}", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    x = generate(w, seed=args.seed)
    sets = args.sets or max(2, min(64, math.ceil(2 * MALL_BYTES / set_bytes(w))))
    log(f"workload {w.name}: {w.description}; {sets} buffer sets of {set_bytes(w) / 2**20:.1f} MiB")
    step = Step(w, x, dev, sets)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    parity = None
    if not args.no_parity:
        step.run(0, sp)
        torch.cuda.synchronize()
        parity = parity_check(w, x, step.parity_output(0))
        log(f"parity vs oracle: {parity}")
        if not parity["ok"]:
            print(json.dumps(dict(metric=METRIC, value=None, error="parity failed", parity=parity)))
            sys.exit(1)

    for i in range(args.warmup):
        step.run(i % sets, sp)
    torch.cuda.synchronize()
    K = args.steps

    # Timed region for the metric: K steps of plain launches, replayed from a
    # captured HIP graph when capture works (launch overhead off the host),
    # otherwise issued eagerly.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for k in range(K):
        step.run(k % sets, sp)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_eager = t_start.elapsed_time(t_end) / K
    ref_out = step.output(0).clone()

    ms_graph = None
    graph_note = None
    if not args.no_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for k in range(K):
                    step.run(k % sets, cs)
            for rep in range(3):
                step.output(0).zero_()
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                if not torch.equal(step.output(0), ref_out):
                    raise RuntimeError(f"graph replay {rep} differs from the eager result")
            t_start.record(stream)
            graph.replay()
            t_end.record(stream)
            torch.cuda.synchronize()
            ms_graph = t_start.elapsed_time(t_end) / K
            del graph
        except Exception as ex:  # capture unsupported: keep the eager figure
            graph_note = f"graph capture not used: {ex}"
            log(graph_note)
    ms_step = ms_graph if ms_graph is not None else ms_eager

    # Per-kernel durations: K more steps through the instrumented entry point,
    # whose launch events bracket each kernel's own execution.
    nl = step.n_launches
    pool = _hip.EventPool(2 * nl * K)
    for k in range(K):
        step.run_timed(k % sets, sp, pool.ptr(2 * nl * k), 2 * nl)
    torch.cuda.synchronize()

    plan, _ = kernel_plan(w, nl)
    a_flops, a_bytes = attention_accounting(w, x["key_lengths"])
    kernels = []
    for j, kp in enumerate(plan):
        durs = [pool.elapsed_ms(2 * (nl * k + j), 2 * (nl * k + j) + 1) for k in range(K)]
        avg_us = 1e3 * float(np.mean(durs))
        flops, byts = kp["flops"], kp["bytes"]
        if kp["has_attention"]:
            flops += a_flops
            # a standalone attention kernel moves Q, K, V and O through HBM;
            # the fused kernel's bytes are its own inputs and output
            if kp["name"] == "attention":
                byts += a_bytes
        kernels.append(dict(name=kp["name"], has_attention=kp["has_attention"], avg_us=round(avg_us, 3),
                            min_us=round(1e3 * float(np.min(durs)), 3),
                            tflops=round(flops / (avg_us * 1e-6) / 1e12, 2),
                            gbs=round(byts / (avg_us * 1e-6) / 1e9, 1),
                            flops=flops, bytes=byts, peak_kind=kp["peak_kind"]))
    pool.close()
    log("kernels: " + ", ".join(f"{k['name']} {k['avg_us']:.2f} us" for k in kernels))

    # the dominant kernel: the longest one that does algorithmic work (the
    # floor probe's empty kernel does none)
    working = [k for k in kernels if k["flops"] > 0 or k["bytes"] > 0] or kernels
    dom = max(working, key=lambda k: k["avg_us"])
    peak_flops = PEAK_BF16_TFLOPS if dom["peak_kind"] == "mfma" else PEAK_FP32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    ai = dom["flops"] / dom["bytes"] if dom["bytes"] > 0 else (math.inf if dom["flops"] > 0 else 0.0)
    traffic = recorded_traffic(w.name, dom["name"])
    if ai < ridge:
        roof = dict(bound="hbm", achieved=dom["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(dom["gbs"] / PEAK_HBM_GBS, 4))
    else:
        roof = dict(bound="mfma" if dom["peak_kind"] == "mfma" else "alu", achieved=dom["tflops"],
                    peak=peak_flops, unit="TFLOP/s", frac=round(dom["tflops"] / peak_flops, 4))
    roof.update(traffic=traffic, kernel=dom["name"], avg_us=dom["avg_us"],
                algorithmic_flops=dom["flops"], algorithmic_bytes=dom["bytes"])
    # Beside an MFMA-bound kernel, the rate the matrix cores sustain on this
    # box in the same run (the shader clock under dense products is below the
    # 2.4 GHz of the nominal peak): context for `frac`, which stays nominal.
    if roof["bound"] == "mfma" and w.dtype == "bf16" and w.kind != "mfma" and not args.no_mfma_probe:
        probe = sustained_mfma_tflops(step.lib, sp, dev)
        roof["sustained"] = dict(probe_tflops=round(probe, 1), frac=round(dom["tflops"] / probe, 4),
                                 probe="mha_mfma_probe: random-bit bf16 operands, 4 workgroups of "
                                       "4 waves per compute unit, 4 chains of %d "
                                       "v_mfma_f32_32x32x16_bf16 per wave" % PROBE_ITERS)
        log(f"sustained matrix-core rate: {probe:.1f} TFLOP/s; {dom['name']} at "
            f"{100 * dom['tflops'] / probe:.1f}% of it")

    nominal = w.nominal_attention_flops()
    att = next((k for k in kernels if k["has_attention"]), None)
    value = nominal / (ms_step * 1e-3) / 1e12 if att is not None else None
    pct_alg = (peak_percent(att["flops"], att["avg_us"])
               if att is not None and w.dtype == "bf16" else None)

    cpu = None
    if not args.no_cpu_baseline and w.kind not in ("floor", "mfma"):  # the probes run no oracle arithmetic
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, x, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")

    kinds = {"floor": "launch floor: an empty kernel and a kernel moving the attention's bytes",
             "mfma": "matrix-core probe: dense bf16 products only, no memory traffic",
             "mha": "multi-head block (projections + attention + output projection)",
             "sdpa": "bare attention",
             "decode": "bare attention, few queries over long caches (sdpa_decode)",
             "embed": "token embedding x sqrt(d_model) + sinusoidal positional encoding",
             "bwd": "attention backward (dQ, dK, dV from dO, O and the row log-sum-exp)",
             "mha_bwd": "multi-head block backward (dX, dW^Q, dW^K, dW^V, dW^O)",
             "layer": "encoder layer, Post-LN (block, residual + LayerNorm, FFN, residual + LayerNorm)"}
    cfg = dict(workload=w.name, B=w.B, n_q=w.n_q, n_k=w.n_k, h=w.h, d_k=w.d_k, d_v=w.d_v,
               mask={0: "none", 1: "causal", 2: "key_padding", 3: "causal+key_padding"}[w.mask],
               kind=kinds[w.kind], buffer_sets=sets)
    if w.kind in ("mha", "layer", "mha_bwd"):
        cfg.update(d_model=w.d_model, self_attention=w.self_attn)
    if w.kind == "layer":
        cfg.update(d_ff=w.d_ff, eps=w.eps)
    if w.kind == "embed":
        cfg = dict(workload=w.name, B=w.B, n=w.n_q, d_model=w.d_model, vocab=w.vocab, pos0=0,
                   kind=kinds[w.kind], buffer_sets=sets)
    if w.kind == "mfma":
        cfg = dict(workload=w.name, workgroups=w.B, waves_per_workgroup=4, chains_per_wave=4,
                   products_per_chain=w.iters, instruction="v_mfma_f32_32x32x16_bf16", operands=w.operands,
                   kind=kinds[w.kind], buffer_sets=sets)
    if x["key_lengths"] is not None:
        cfg["key_lengths_mean"] = float(x["key_lengths"].float().mean())
    out = {
        "metric": METRIC,
        "value": None if value is None else round(value, 3),
        "unit": "TFLOP/s",
        # The peak fraction counts the work the method does: the attention
        # kernel's algorithmic flops (visible (query, key) pairs x 2(d_k + d_v),
        # plus the fused projections when the kernel also projects) over that
        # kernel's own average launch time.  The nominal dense count of the
        # metric's formula doubles a causal attention's work, so its step-level
        # fraction is given separately and labelled.
        "pct_of_bf16_mfma_peak": None if pct_alg is None else round(pct_alg, 3),
        "pct_of_bf16_mfma_peak_basis": None if pct_alg is None else
            "algorithmic flops of the attention kernel over its average launch time",
        "nominal_pct_of_bf16_mfma_peak_step": None if value is None else round(100 * value / PEAK_BF16_TFLOPS, 3),
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "timing": dict(launch="hip graph" if ms_graph is not None else "eager",
                       ms_per_step_graph=None if ms_graph is None else round(ms_graph, 5),
                       ms_per_step_eager=round(ms_eager, 5),
                       kernel_sum_ms=round(sum(k["avg_us"] for k in kernels) / 1e3, 5),
                       note=graph_note),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/d_model) weights)",
        "config": cfg,
        # the kernel that runs the attention (fused with the input
        # projections for short sequences); algorithmic_flops counts all its flops
        "attention_kernel": None if att is None else dict(
            kernel=att["name"], avg_us=att["avg_us"],
            algorithmic_flops=att["flops"],
            algorithmic_tflops=att["tflops"],
            nominal_attention_tflops=round(nominal / (att["avg_us"] * 1e-6) / 1e12, 2),
            gbs=att["gbs"]),
        "kernels": [{k: v for k, v in kk.items() if k not in ("peak_kind", "has_attention")} for kk in kernels],
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "kernel_source_sha": kernel_source_sha(),
    }
    if w.kind == "embed":
        out["data"] = "synthetic (seeded uniform token ids, N(0,1/d_model) embedding table)"
    if w.kind == "mha_bwd":
        out["data"] = "synthetic (seeded N(0,1) X and dY, N(0,1/d_model) weights)"
        bf = block_bwd_flops(w, x["key_lengths"])
        out["backward"] = dict(algorithmic_flops_per_step=bf,
                               algorithmic_tflops=round(bf / (ms_step * 1e-3) / 1e12, 2),
                               pct_of_bf16_mfma_peak=round(100 * bf / (ms_step * 1e-3) / 1e12 /
                                                           PEAK_BF16_TFLOPS, 2),
                               note="dX and dW of the four projections, five products per visible "
                                    "attention pair; the transposes are copies")
    if w.kind == "bwd":
        out["data"] = "synthetic (seeded N(0,1) Q, K, V and upstream gradient dO)"
        bf = 10.0 * bwd_pairs(w, x["key_lengths"]) * w.d_k
        out["backward"] = dict(algorithmic_flops_per_step=bf,
                               algorithmic_tflops=round(bf / (ms_step * 1e-3) / 1e12, 2),
                               pct_of_bf16_mfma_peak=round(100 * bf / (ms_step * 1e-3) / 1e12 /
                                                           PEAK_BF16_TFLOPS, 2),
                               note="5 products (S, dP, dV, dK, dQ) of 2 d flops per visible pair; "
                                    "the kernels also recompute S and dP in both kernels")
    if w.kind == "layer":
        lf = layer_flops(w)
        out["layer"] = dict(matmul_flops_per_step=lf,
                            tflops=round(lf / (ms_step * 1e-3) / 1e12, 2),
                            tokens_per_s=round(w.B * w.n_q / (ms_step * 1e-3), 1))
        out["data"] = ("synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights, "
                       "0.1*N(0,1) biases and LayerNorm shifts, 1+0.1*N(0,1) LayerNorm scales)")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
