"""The C-ABI layer's argument checks under host AddressSanitizer (CPU): a separate build of
libbsattn.so with the host pass sanitized runs every ABI test of tests/test_abi.py (all of
them fail their checks on the host before any launch) in a child process with the sanitizer
runtime preloaded; any invalid read or write in the host code aborts that process."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.skipif(_asan_runtime() is None, reason="no host AddressSanitizer runtime")
def test_abi_checks_under_host_asan(tmp_path):
    from block_sparse_top_amd.build import build
    lib = str(tmp_path / "libbsattn_asan.so")
    build(build_dir=str(tmp_path / "obj"), lib=lib, probes=False, asan=True)
    env = dict(os.environ, BSATTN_LIB=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
