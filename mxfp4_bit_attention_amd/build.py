"""Build libmxattn.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python mxfp4_bit_attention_amd/build.py

(run as a script: importing the package itself loads the library, which may not
exist yet or may be stale).

Every HIP translation unit is compiled with IEEE-exact fp32 settings (no
contraction into FMA, denormals kept) because the quantiser must reproduce
the fp32 Hadamard butterflies bit for bit, and with packed-fp32 instructions
disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmxattn.so")
# the microbenchmarks behind the benchmark's measured roofline denominators, kept out of
# the attention library itself
PROBES_LIB = os.path.join(HERE, "libmxattn_probes.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["quantize.hip", "attention.hip", "api.cpp", "noalloc.hip"]
PROBE_SOURCES = ["probes.hip"]
# Per-source flags beyond the common ones (none at present: every kernel honours NaN,
# since a non-finite block must turn the outputs it reaches into NaN).
EXTRA_FLAGS: dict[str, list[str]] = {}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxattn)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _link(cc: str, objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc, *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    _link(cc, objs[: len(SOURCES)], LIB)
    _link(cc, objs[len(SOURCES):], PROBES_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
