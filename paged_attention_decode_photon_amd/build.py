"""Build libphoton_decode.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m paged_attention_decode_photon_amd.build [--jobs N]

Each HIP source is compiled to an object in parallel, then linked into a
shared library next to this file.  Code objects use version 5, which every
ROCm 7 runtime loads (the library runs inside the HIP runtime that PyTorch
ships, which may be older than this hipcc).  Packed-fp32 VALU forms are disabled for
all device code (-packed-fp32-ops): the kernels rely on scalar fp32 FMA only.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libphoton_decode.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["photon_abi.hip", "kv_cache_write.hip", "paged_decode.hip", "rope_kv_write.hip",
           "paged_multi_query.hip", "bandwidth_probe.hip"]
HOST_SOURCES = ["scheduler.cpp"]  # host-only C++ (the block manager and scheduler)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-fvisibility=hidden"]
COMMON = [
    f"--offload-arch={ARCH}", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax reads them with no AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source device flags.  The decode kernel's first two arguments (context
# lengths, batch size) are preloaded into SGPRs at dispatch (gfx950 kernel
# argument preloading; older firmware runs the compiler's fallback prologue).
SOURCE_FLAGS = {"paged_decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=2"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if src in HOST_SOURCES:
        cmd = [CXX, *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed for {src}:\n{r.stderr}")
    # the host pass does not know the device-only feature; drop that line
    noise = "is not a recognized feature for this target"
    rest = [ln for ln in r.stderr.splitlines() if noise not in ln and ln.strip()]
    if rest:
        sys.stderr.write("\n".join(rest) + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 (and the host C++ sources), link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = SOURCES + HOST_SOURCES
    jobs = jobs or min(len(sources), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    print(build(args.jobs))


if __name__ == "__main__":
    main()
