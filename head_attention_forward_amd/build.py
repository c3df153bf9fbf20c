"""Build libmha.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m head_attention_forward_amd.build [--asan | --fault]

Compiles every ``csrc/*.hip`` with hipcc (one process per file, in
parallel) into ``_build/`` and links ``libmha.so`` next to this file.  Always
rebuilds.  ``--asan`` (or build(asan=True)) builds ``libmha_asan.so`` instead:
the host code instrumented with AddressSanitizer (device code unchanged), for
the CPU check of the C ABI's host paths; it needs the sanitizer runtime
preloaded into the process that loads it.  ``--fault`` builds
``libmha_fault.so``, whose launches can be made to fail on demand
(mha_fault_inject), for tests of the error path.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmha.so")
ASAN_BUILD_DIR = os.path.join(HERE, "_build_asan")
ASAN_LIB_PATH = os.path.join(HERE, "libmha_asan.so")
# Host-side AddressSanitizer only (each option applies to the host pass).
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
# The fault-injection test build (launch failures on demand, mha_fault_inject).
FAULT_BUILD_DIR = os.path.join(HERE, "_build_fault")
FAULT_LIB_PATH = os.path.join(HERE, "libmha_fault.so")
FAULT_FLAGS = ["-DMHA_FAULT_INJECTION"]

ARCH = "gfx950"
# Packed fp32 VALU instructions are switched off for all device code.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]
# Per-file additions.  The bf16 attention kernel never sees a NaN by
# contract (finite inputs; masked scores are -inf), so its float max needs no
# NaN canonicalization: this lets v_max3_f32 take raw scores.  Host-side
# argument checks (which do test for NaN) live in other files.
EXTRA = {"attn_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
         "attn_decode_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
         "proj_attn_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmha)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note.
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    return p.returncode, out


def asan_runtime():
    """Path of the AddressSanitizer runtime matching hipcc's clang, or None."""
    try:
        out = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                             stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True).stdout.strip()
    except Exception:
        return None
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def build(verbose=False, asan=False, fault=False):
    hipcc = _hipcc()
    build_dir = ASAN_BUILD_DIR if asan else (FAULT_BUILD_DIR if fault else BUILD_DIR)
    lib_path = ASAN_LIB_PATH if asan else (FAULT_LIB_PATH if fault else LIB_PATH)
    extra_all = (ASAN_FLAGS if asan else []) + (FAULT_FLAGS if fault else [])
    os.makedirs(build_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(build_dir, os.path.basename(s)[:-4] + ".o") for s in sources]

    def compile_one(src_obj):
        src, obj = src_obj
        cmd = ([hipcc] + COMMON + extra_all + EXTRA.get(os.path.basename(src), []) +
               ["-c", src, "-o", obj])
        rc, out = _run(cmd)
        return src, rc, out, cmd

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        results = list(ex.map(compile_one, zip(sources, objs)))
    failed = False
    for src, rc, out, cmd in results:
        if out.strip() and (verbose or rc):
            sys.stderr.write(f"--- {os.path.basename(src)}\n{out}\n")
        if rc:
            sys.stderr.write("command: " + " ".join(cmd) + "\n")
            failed = True
    if failed:
        raise RuntimeError("libmha: compilation failed")
    tmp = lib_path + ".tmp"
    # (the sanitizer runtime is not linked in: the loading process preloads it)
    rc, out = _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    if rc:
        sys.stderr.write(out + "\n")
        raise RuntimeError("libmha: link failed")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv, fault="--fault" in sys.argv))
