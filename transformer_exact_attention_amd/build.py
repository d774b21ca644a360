"""Build libgqa_attn.so in place (hipcc, gfx950).

Usage: ``python -m transformer_exact_attention_amd.build`` or ``build()``.
Objects go to ``_build/`` at the repository root; the library lands next to
this file, where the Python binding loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libgqa_attn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("GQA_ATTN_ARCH", "gfx950")

DEVICE_SOURCES = ["prefill_f32.hip", "prefill_bf16.hip", "decode.hip", "kv_cache.hip", "backward.hip"]
HOST_SOURCES = ["gqa_attn.cpp", "kv_cache.cpp"]

# Packed-fp32 VALU forms are disabled on purpose (-packed-fp32-ops); the host
# pass warns that it does not know the feature, which is harmless.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-ffp-contract=fast"]
# Per-source extras.  The bf16 prefill kernel keeps its output accumulators in
# AGPRs through inline asm and needs every compiler-generated MFMA (the score
# product, read by the softmax) in the VGPR form.
SOURCE_FLAGS = {"prefill_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
# Sources whose generated assembly must pass asm_check (MFMAs in inline asm).
ASM_CHECKED = ["prefill_bf16.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def hip_runtime_dir() -> str:
    """Directory whose libamdhip64.so the library links against.

    When torch (ROCm build) is installed, its bundled HIP runtime is the one a
    Python process has loaded; linking against it records the dependency as
    ``libamdhip64.so`` so the loader reuses that copy (one runtime per process,
    so torch streams and pointers are valid here).  Without torch the system
    copy under /opt/rocm/lib is found by the same name.
    """
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec and spec.origin:
        d = os.path.join(os.path.dirname(spec.origin), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    return "/opt/rocm/lib"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, [cc, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                           "-o", obj]))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, [cc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c",
                           os.path.join(CSRC, src), "-o", obj]))
    # Assembly of the sources with inline-asm MFMAs, for the hazard check.
    asm_jobs = []
    for src in ASM_CHECKED:
        out = os.path.join(BUILD_DIR, src + ".s")
        asm_jobs.append((out, [cc, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
                               os.path.join(CSRC, src), "-o", out]))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs) + len(asm_jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs + asm_jobs))[:len(jobs)]
    try:
        from . import asm_check
    except ImportError:          # run as a script: this directory is on sys.path
        import asm_check
    for out, _ in asm_jobs:
        problems = asm_check.check_all(open(out).read())
        if problems:
            raise RuntimeError(f"MFMA wait-state check failed for {out}:\n" + "\n".join(problems))
    if verbose:
        for (obj, cmd), out in zip(jobs, outs):
            print(" ".join(cmd))
            if out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run(["g++", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs], "-L" + hip_runtime_dir(),
          "-lamdhip64", "-Wl,--no-undefined"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
