"""The C ABI's host code under AddressSanitizer (CPU only).

libmha_asan.so is libmha built with the host pass instrumented
(build(asan=True)); a child process with the sanitizer runtime preloaded
loads it through ctypes (no torch) and drives every host-side path that
needs no GPU: status strings, workspace sizes, launch counts and every
argument check, including key-length arrays read to their last element
(B = 1024) and the split-count paths.  Any invalid memory access in that
code aborts the child with an AddressSanitizer report."""

import os
import subprocess
import sys
import textwrap

import pytest

from head_attention_forward_amd import build as hbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = textwrap.dedent(r'''
    import ctypes, importlib.util, sys
    spec = importlib.util.spec_from_file_location("abi", sys.argv[1])
    abi = importlib.util.module_from_spec(spec); spec.loader.exec_module(abi)
    L = ctypes.CDLL(sys.argv[2])
    for name, (res, args) in abi.SIG.items():
        f = getattr(L, name); f.restype = res; f.argtypes = args
    P = ctypes.c_void_p
    F, F2, MIS = P(0x10000), P(0x20000), P(0x10008)
    def kl(*v):
        a = (ctypes.c_int32 * len(v))(*v)
        return ctypes.cast(a, P), a
    keep = []
    for c in list(range(-12, 3)) + [12345]:
        assert L.mha_status_str(c)
    for args in [(2, 8, 8, 2, 64, 64, 0), (0, 8, 8, 2, 64, 64, 0), (3, 100, 77, 8, 64, 64, 1)]:
        L.mha_workspace_bytes(*args)
    L.sdpa_backward_workspace_bytes(4, 16, 4096); L.sdpa_backward_workspace_bytes(0, 1, 1)
    L.mha_train_workspace_bytes(2, 8, 8, 2, 64, 64, 0)
    L.mha_backward_workspace_bytes(2, 8, 8, 64, 2, 64, 64, 1, 0)
    L.ffn_workspace_bytes(3, 512, 2048, 0); L.encoder_layer_workspace_bytes(2, 8, 64, 2, 64, 64, 128, 0)
    L.mha_forward_launches(100, 100, 512, 1); L.mha_forward_launches(512, 512, 512, 1)
    L.mha_backward_launches(1); L.encoder_layer_launches(100, 512)
    L.sdpa_decode_workspace_bytes(0, 1, 1, 1); L.sdpa_decode_launches(0, 1, 1, 1, 0)
    def sdpa(Q=F, B=2, h=2, nq=8, nk=8, dk=64, sc=0.125, m=0, k=None, dt=0):
        return L.sdpa_forward(Q, F, F, F2, B, h, nq, nk, dk, 64, sc, m, k, dt, None)
    codes = [sdpa(Q=None), sdpa(B=0), sdpa(dk=32), sdpa(sc=0.0), sdpa(m=4), sdpa(m=1, nq=8, nk=9),
             sdpa(m=2), sdpa(dt=5), sdpa(Q=MIS)]
    p, a = kl(*([4] * 1023 + [0])); keep.append(a)
    codes += [sdpa(m=2, k=p, B=1024, h=1), sdpa(m=3, k=p, B=1024, h=1)]
    p, a = kl(*([4] * 1025)); keep.append(a)
    codes += [sdpa(m=2, k=p, B=1025, h=1)]
    p, a = kl(*([9] * 7 + [3])); keep.append(a)
    codes += [sdpa(m=2, k=p, B=8, nk=8)]
    def mha(B=2, k=None, m=0, ws_bytes=None, Xq=F):
        wb = L.mha_workspace_bytes(B, 8, 8, 2, 64, 64, 0) if ws_bytes is None else ws_bytes
        return L.mha_forward(Xq, F, F, F, F, F, F2, B, 8, 8, 64, 2, 64, 64, m, k, 0, F, wb, None)
    p, a = kl(*([4] * 1023 + [0])); keep.append(a)
    codes += [mha(Xq=None), mha(B=0), mha(ws_bytes=16), mha(m=2, k=p, B=1024), mha(m=2, k=p, B=1025)]
    def dec(Q=F, B=2, m=0, k=None):
        return L.sdpa_decode(Q, F, F, F2, B, 2, 1, 1000, 64, 64, 0.125, m, k, 0, F, 1 << 20, None)
    codes += [dec(Q=None), dec(B=0), dec(m=2)]
    def bwd(Q=F, B=2, k=None, m=0, nq=8):
        return L.sdpa_backward_noalloc(Q, F, F, F, F, F, F2, F2, F2, B, 2, nq, 8, 64, 64, 0.125, m, k,
                                       0, None)
    p, a = kl(0, 5); keep.append(a)
    codes += [bwd(Q=None), bwd(B=0), bwd(m=2), bwd(m=2, k=p), bwd(B=1, nq=(1 << 19) + 1)]
    codes += [L.mha_floor_probe(7, F, F, F, F2, 4096, 16, None),
              L.mha_floor_probe(1, F, F, F, F2, 4100, 16, None)]
    assert all(c < 0 for c in codes), codes
    print("ASAN-CHECK-OK", len(codes))
''')


def test_host_paths_under_address_sanitizer(tmp_path):
    runtime = hbuild.asan_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc's clang")
    lib = hbuild.ASAN_LIB_PATH
    if not os.path.exists(lib):
        hbuild.build(asan=True)
    script = tmp_path / "asan_abi.py"
    script.write_text(SCRIPT)
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    p = subprocess.run([sys.executable, str(script),
                        os.path.join(ROOT, "head_attention_forward_amd", "_abi.py"), lib],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    assert p.returncode == 0, p.stderr[-4000:]
    assert "ASAN-CHECK-OK" in p.stdout


CANARY = textwrap.dedent(r'''
    import ctypes, importlib.util, sys
    spec = importlib.util.spec_from_file_location("abi", sys.argv[1])
    abi = importlib.util.module_from_spec(spec); spec.loader.exec_module(abi)
    L = ctypes.CDLL(sys.argv[2])
    for name, (res, args) in abi.SIG.items():
        f = getattr(L, name); f.restype = res; f.argtypes = args
    P = ctypes.c_void_p
    a = (ctypes.c_int32 * 300)(*([4] * 300))
    # a caller that breaks the contract: 301 batches, 300 lengths
    L.sdpa_forward(P(0x10000), P(0x10000), P(0x10000), P(0x20000), 301, 1, 8, 8, 64, 64, 0.125, 2,
                   ctypes.cast(a, P), 0, None)
''')


def test_sanitizer_reports_a_short_length_array(tmp_path):
    """The instrumentation is live: the argument check reads one length per
    batch, so a 300-entry array for 301 batches is reported."""
    runtime = hbuild.asan_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc's clang")
    if not os.path.exists(hbuild.ASAN_LIB_PATH):
        hbuild.build(asan=True)
    script = tmp_path / "canary.py"
    script.write_text(CANARY)
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    p = subprocess.run([sys.executable, str(script),
                        os.path.join(ROOT, "head_attention_forward_amd", "_abi.py"), hbuild.ASAN_LIB_PATH],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env, timeout=300)
    assert p.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in p.stderr
