"""Build libkvq.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m quantized_decode_attention_02_amd.build

Flags that matter for correctness:
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32
    instructions are generated;
  * ``-fno-gpu-flush-denormals-to-zero`` and
    ``-fhip-fp32-correctly-rounded-divide-sqrt``: IEEE fp32 division and
    denormals, which the bit-exact quantizer relies on;
  * no fast-math of any kind;
  * ``-mllvm -amdgpu-atomic-optimizer-strategy=None``: the decode kernels'
    chunk claims are one lane's atomic whose result is read a tile later;
    the atomic optimizer would rewrite it into a wave-wide form that reads
    the result back at once, stalling the wave on the atomic's round trip
    and on every load issued before it.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libkvq.so")
SOURCES = ["kvq.cpp", "append.hip", "append_block.hip", "append_kivi.hip", "decode.hip", "decode_mfma.hip", "decode_rope.hip", "dequant.hip"]
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libkvq)")


def command(out=LIB, defines=()):
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            *[f"-D{d}" for d in defines],
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-fno-fast-math", "-Wall", "-Wno-unused-function",
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", out] + \
           [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose=False, out=LIB, defines=()):
    """Compile every source into ``out`` (default _lib/libkvq.so; always
    recompiles).  ``defines``: tuning macros such as KVQ_DECODE_PREFETCH=1."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = command(tmp, defines)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkvq.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
