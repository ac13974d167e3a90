"""The achievable-peak probes (include/bsattn_probe.h) run and the copy probe copies."""
import ctypes
import sys

import pytest
import torch


pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_probes_run_and_copy_is_exact():
    print("[probes]", flush=True)
    sys.stdout.flush()
    from bench import probe_lib
    L = probe_lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    groups = 64
    sink = torch.full((L.bsattn_probe_sink_floats(groups),), float("nan"), device=DEV)
    fl = ctypes.c_double(0.0)
    assert L.bsattn_probe_mfma_bf16(100, groups, P(sink), ctypes.byref(fl), sp) == 0
    torch.cuda.synchronize()
    assert fl.value == 2.0 * 32 * 32 * 16 * 8 * 4 * groups * 100
    assert torch.isfinite(sink).all()
    assert L.bsattn_probe_mfma_fp8(100, groups, P(sink), ctypes.byref(fl), sp) == 0
    torch.cuda.synchronize()
    assert fl.value == 2.0 * 32 * 32 * 64 * 8 * 4 * groups * 100
    assert torch.isfinite(sink).all()
    g = torch.Generator(device=DEV).manual_seed(5)
    src = torch.randint(0, 256, (3 << 20,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros_like(src)
    assert L.bsattn_probe_copy(P(src), P(dst), src.numel(), groups, sp) == 0
    assert L.bsattn_probe_read(P(src), src.numel(), groups, P(sink), sp) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.isfinite(sink).all()
