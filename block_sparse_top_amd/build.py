"""Build libbsattn.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m block_sparse_top_amd.build        # or __graft_entry__.build()

Objects go to block_sparse_top_amd/_build/, the library to block_sparse_top_amd/libbsattn.so.
Every call recompiles.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbsattn.so")
SOURCES = ["api.hip", "pool.hip", "select.hip", "select_large.hip", "attn_bf16.hip",
           "attn_bf16_page.hip", "attn_f32.hip", "attn_fp8.hip", "validate.hip", "attn_bwd.hip",
           "decode.hip"]
# flags of single sources: the (D = 64, block = 64) attention kernels take the iterative ILP
# machine scheduler (faster on that shape; the other kernels were slower with it)
SOURCE_FLAGS = {"attn_bf16_page.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}
# achievable-peak probes (measurement support, include/bsattn_probe.h): a library of their own
PROBE_LIB = os.path.join(PKG, "libbsattn_probe.so")
PROBE_SOURCES = ["probe.hip"]

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results and accumulators in ordinary VGPRs: no AGPR <-> VGPR copies in the loops
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


# host AddressSanitizer for a test build of the C-ABI layer (device code is built as usual;
# every -fsanitize= sits after -Xarch_host so that it applies to the host pass only)
ASAN_CFLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LDFLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libasan"]


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, extra=()):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, extra_flags=(), build_dir: str = BUILD, lib: str = LIB,
          probes: bool = True, asan: bool = False) -> str:
    """Compiles and links libbsattn.so (and libbsattn_probe.so). build_dir/lib/probes/asan give
    a separate test build: host AddressSanitizer, no probe library, elsewhere than the product."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = SOURCES + (PROBE_SOURCES if probes else [])
    flags = list(extra_flags) + (ASAN_CFLAGS if asan else [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, flags, build_dir), srcs)))
    _link([objs[s] for s in SOURCES], lib, ASAN_LDFLAGS if asan else ())
    if probes:
        _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {lib}" + (f" and {PROBE_LIB}" if probes else ""))
    return lib


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
