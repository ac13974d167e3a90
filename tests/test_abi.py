"""The C-ABI library loads and exports what include/bsattn.h declares; host-side argument
checks reject bad calls before any launch (no GPU needed: every call here fails its
checks on the host)."""
import ctypes
import os
import re

import pytest

import block_sparse_top_amd as bst
from block_sparse_top_amd import bsattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails first


def declared_functions(header=None):
    names = set()
    for h in HEADERS:
        if header and os.path.basename(h) != header:
            continue
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(bsattn_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    """libbsattn.so exports every function of bsattn.h, libbsattn_probe.so those of
    bsattn_probe.h; the method's library holds no probe."""
    from bench import probe_lib
    L = bst.lib()
    names = declared_functions("bsattn.h")
    assert {"bsattn_select", "bsattn_forward", "bsattn_select_workspace_bytes",
            "bsattn_abi_version", "bsattn_status_str", "bsattn_last_error",
            "bsattn_select_ex", "bsattn_forward_ex", "bsattn_key_blocks",
            "bsattn_select_workspace_bytes_ex", "bsattn_decode_ex",
            "bsattn_select_noalloc", "bsattn_select_noalloc_max_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    pnames = declared_functions("bsattn_probe.h")
    assert {"bsattn_probe_mfma_bf16", "bsattn_probe_read", "bsattn_probe_copy",
            "bsattn_probe_sink_floats", "bsattn_probe_mfma_fp8",
            "bsattn_probe_last_error"} <= set(pnames)
    P = probe_lib()
    for n in pnames:
        assert hasattr(P, n), n
        assert not hasattr(L, n), f"{n} is exported by the method's library"
    assert set(names).isdisjoint(pnames)


def test_version_and_status_strings():
    L = bst.lib()
    assert L.bsattn_abi_version() == 5
    for s in range(5):
        assert L.bsattn_status_str(s).decode() == bsattn.STATUS[s]
    assert L.bsattn_status_str(99).decode() == "unknown status"


def sel(dtype=1, B=1, N=512, Hq=2, Hkv=2, D=64, block=64, topk=2, q=FAKE, k=FAKE, idx=FAKE,
        ws=FAKE, wsb=1 << 30):
    return bst.lib().bsattn_select(dtype, B, N, Hq, Hkv, D, block, topk, q, k, idx, ws, wsb, None)


def fwd(dtype=1, B=1, N=512, Hq=2, Hkv=2, D=64, block=64, topk=2, q=FAKE, k=FAKE, v=FAKE,
        idx=FAKE, scale=0.125, descale=None, out=FAKE):
    return bst.lib().bsattn_forward(dtype, B, N, Hq, Hkv, D, block, topk, q, k, v, idx, scale,
                                    descale, out, None)


def last():
    return bst.lib().bsattn_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=7), 1, "dtype"),
    (dict(N=500), 1, "multiple of block"),
    (dict(topk=0), 1, "topk"),
    (dict(topk=9), 1, "topk"),
    (dict(Hq=3, Hkv=2), 1, "multiple of Hkv"),
    (dict(Hkv=0), 1, "Hkv"),
    (dict(B=-1), 1, "negative"),
    (dict(D=96), 2, "D=96"),
    (dict(block=32, N=512), 2, "block=32"),
    (dict(q=None), 1, "null"),
    (dict(k=ctypes.c_void_p(0x10008)), 1, "aligned"),
    (dict(ws=None), 3, "workspace"),
    (dict(wsb=16), 3, "workspace"),
    (dict(ws=ctypes.c_void_p(0x10010)), 3, "aligned"),
    (dict(N=64 * 2048 + 64, topk=3), 2, "nb=2049"),
    (dict(N=64 * 16384, topk=3), 2, "nb=16384"),
])
def test_select_rejects(kw, status, msg):
    assert sel(**kw) == status
    assert msg in last()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(scale=float("nan")), 1, "scale"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(dtype=2), 1, "descale"),
    (dict(dtype=2, descale=(ctypes.c_float * 3)(1.0, 0.0, 1.0)), 1, "descale_qkv[1]"),
    (dict(out=None), 1, "null"),
    (dict(v=ctypes.c_void_p(0x10004)), 1, "aligned"),
    (dict(topk=10), 1, "topk"),
    (dict(N=96), 1, "multiple of block"),
    (dict(D=32), 2, "D=32"),
])
def test_forward_rejects(kw, status, msg):
    assert fwd(**kw) == status
    assert msg in last()


def sel_ex(flags, **kw):
    a = dict(dtype=1, B=1, N=512, Hq=2, Hkv=2, D=64, block=64, topk=2, q=FAKE, k=FAKE,
             idx=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return bst.lib().bsattn_select_ex(a["dtype"], a["B"], a["N"], a["Hq"], a["Hkv"], a["D"],
                                      a["block"], a["topk"], flags, a.get("nrand", 0), 0,
                                      a.get("ks", 0), a["q"], a["k"], a["idx"], a["ws"], a["wsb"],
                                      None)


def test_extended_entry_points_reject():
    assert sel_ex(8) == 1 and "flags" in last()                   # unknown bit
    assert sel_ex(4, nrand=1, N=64 * 2048, topk=3) == 2 and "random" in last()  # fused only
    assert sel_ex(1, q=None) == 1 and "null" in last()           # checks as bsattn_select
    assert sel_ex(0, nrand=3) == 1 and "nrand" in last()         # nrand > topk
    assert sel_ex(1, nrand=1) == 2 and "causal" in last()
    assert sel_ex(0, nrand=1, N=64 * 2048, topk=3) == 2 and "random" in last()
    L = bst.lib()
    st = L.bsattn_forward_ex(1, 1, 512, 2, 2, 64, 64, 2, 16, 0, FAKE, FAKE, FAKE, FAKE, 0.125,
                             None, FAKE, None, None)
    assert st == 1 and "flags" in last()
    st = L.bsattn_forward_ex(1, 1, 512, 2, 2, 64, 64, 2, 1, 0, FAKE, FAKE, FAKE, FAKE,
                             float("inf"), None, FAKE, None, None)
    assert st == 1 and "scale" in last()
    st = L.bsattn_forward_ex(1, 1, 512, 2, 2, 64, 64, 2, 0, 0, FAKE, FAKE, FAKE, FAKE, 0.125,
                             None, FAKE, ctypes.c_void_p(0x10002), None)
    assert st == 1 and "lse" in last()


def test_key_blocks():
    L = bst.lib()
    # ceil((N - block) / stride) + 1 key blocks, the last one ending at token N
    for N, blk, ks, n in ((512, 64, 0, 8), (512, 64, 64, 8), (512, 64, 48, 11), (8192, 64, 48, 171),
                          (8192, 128, 96, 85), (256, 64, 32, 7), (0, 64, 48, 0), (64, 64, 48, 1)):
        assert L.bsattn_key_blocks(N, blk, ks) == n, (N, blk, ks)
        assert bst.key_blocks(N, blk, ks) == n
    for N, blk, ks in ((500, 64, 48), (512, 64, 31), (512, 64, 65), (-64, 64, 0)):
        assert L.bsattn_key_blocks(N, blk, ks) == -1 and last()
    with pytest.raises(bsattn.BsattnError):
        bst.key_blocks(512, 64, 20)
    n = L.bsattn_select_workspace_bytes_ex(2, 8192, 16, 4, 64, 64, 48)
    assert n == 2 * 16 * 128 * 64 * 4 + 2 * 4 * 171 * 64 * 4
    assert L.bsattn_select_workspace_bytes_ex(2, 8192, 16, 4, 64, 64, 0) == \
        L.bsattn_select_workspace_bytes(2, 8192, 16, 4, 64, 64)


def test_overlap_rejects():
    L = bst.lib()
    assert sel_ex(0, ks=31) == 1 and "key_stride" in last()
    assert sel_ex(0, ks=65) == 1 and "key_stride" in last()
    assert sel_ex(0, ks=48, topk=12) == 1 and "topk" in last()          # 11 key blocks
    assert sel_ex(1, ks=48) == 2 and "causal" in last()
    assert sel_ex(0, ks=48, N=64 * 800, topk=3) == 2 and "overlapping" in last()   # 1066 > 1024
    assert sel_ex(0, ks=48, topk=11, q=None) == 1 and "null" in last()  # topk 11 passes the checks
    assert sel_ex(0, ks=48, topk=11, wsb=16) == 3 and "workspace" in last()
    st = L.bsattn_forward_ex(1, 1, 512, 2, 2, 64, 64, 2, 1, 48, FAKE, FAKE, FAKE, FAKE, 0.125,
                             None, FAKE, None, None)
    assert st == 2 and "causal" in last()
    st = L.bsattn_forward_ex(1, 1, 64 * 11000, 2, 2, 64, 64, 2, 0, 48, FAKE, FAKE, FAKE, FAKE,
                             0.125, None, FAKE, None, None)
    assert st == 2 and "overlapping" in last()
    st = L.bsattn_forward_ex(1, 1, 512, 2, 2, 64, 64, 11, 0, 48, FAKE, FAKE, FAKE, None, 0.125,
                             None, FAKE, None, None)
    assert st == 1 and "null" in last()


def bwd(**kw):
    a = dict(dtype=1, B=1, N=512, Hq=2, Hkv=2, D=64, block=64, topk=2, flags=0, t=FAKE,
             scale=0.125, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    t = a["t"]
    return bst.lib().bsattn_backward(a["dtype"], a["B"], a["N"], a["Hq"], a["Hkv"], a["D"],
                                     a["block"], a["topk"], a["flags"], t, t, t, t, t, t, t,
                                     a["scale"], t, t, t, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=0), 2, "backward"),
    (dict(dtype=2, D=128), 2, "backward"),
    (dict(block=32, N=1024), 2, "block=32"),
    (dict(N=64 * 5000, topk=3), 2, "64-token blocks"),
    (dict(block=128, N=128 * 2100, topk=3), 2, "64-token blocks"),
    (dict(flags=8), 1, "flags"),
    (dict(scale=0.0), 1, "scale"),
    (dict(t=None), 1, "null"),
    (dict(ws=None), 3, "workspace"),
    (dict(wsb=8), 3, "workspace"),
])
def test_backward_rejects(kw, status, msg):
    assert bwd(**kw) == status
    assert msg in last()


def test_backward_workspace_bytes():
    L = bst.lib()
    n = L.bsattn_backward_workspace_bytes(2, 8192, 16, 4, 64, 64, 38)
    al = lambda x: (x + 255) // 256 * 256
    assert n == al(2 * 16 * 8192 * 4) + al(2 * 4 * 129 * 4) + al(2 * 16 * 128 * 38 * 4)
    # block 128: the 64-token form with 2 * topk places, then its index rows
    n = L.bsattn_backward_workspace_bytes(2, 8192, 16, 4, 64, 128, 19)
    assert n == (al(2 * 16 * 8192 * 4) + al(2 * 4 * 129 * 4) + al(2 * 16 * 128 * 38 * 4)
                 + al(2 * 16 * 128 * 38 * 4))


def test_empty_calls_launch_nothing():
    # B == 0 or N == 0: checked, then nothing to do (no pointer is touched)
    assert sel(B=0, q=None, k=None, idx=None, ws=None, wsb=0) == 0
    assert sel(N=0, topk=0, q=None, k=None, idx=None, ws=None, wsb=0) == 0
    assert fwd(B=0, q=None, k=None, v=None, idx=None, out=None) == 0
    assert sel(N=0, topk=1) == 1          # topk must be 0 when nb == 0


def test_workspace_bytes():
    L = bst.lib()
    n = L.bsattn_select_workspace_bytes(2, 8192, 16, 4, 64, 64)
    assert n == 2 * 16 * 128 * 64 * 4 + 2 * 4 * 128 * 64 * 4
    assert L.bsattn_select_workspace_bytes(0, 8192, 16, 4, 64, 64) == 0
    assert L.bsattn_select_workspace_bytes(1, 100, 1, 1, 64, 64) == 0
    assert "workspace" in last()


def test_python_binding_refuses_cpu_tensors():
    """Every entry point refuses host tensors before any call into the library (a host
    pointer handed to a kernel would fault the GPU)."""
    import torch
    x = torch.zeros(1, 128, 2, 64, dtype=torch.bfloat16)
    idx = torch.zeros(1, 2, 2, 1, dtype=torch.int32)
    lse = torch.zeros(1, 2, 128)
    with pytest.raises(ValueError, match="device"):
        bst.select(x, x, 64, 1)
    with pytest.raises(ValueError, match="device"):
        bst.forward(x, x, x, idx)
    with pytest.raises(ValueError, match="device"):
        bst.backward(x, x, x, idx, x, x, lse)
    with pytest.raises(ValueError, match="device"):
        bst.block_sparse_attention(x, x, x, 64, 0.5)
    kc = torch.zeros(2, 256, 1, 64, dtype=torch.bfloat16)
    lens = torch.tensor([200, 256], dtype=torch.int32)
    kbar = torch.zeros(2, 1, 64, 4)
    with pytest.raises(ValueError, match="device"):
        bst.decode_pool(kc, lens, kbar, 64)
    with pytest.raises(ValueError, match="device"):
        bst.decode(torch.zeros(2, 2, 64, dtype=torch.bfloat16), kc, kc, kbar, lens, 64, 2)


def test_device_tensor_checks():
    """The binding's argument check: device, contiguity, dtype, shape and size, each refused
    with a message naming the argument (host tensors stand in; the device test comes first)."""
    import torch
    chk = bst.bsattn._device_tensor
    with pytest.raises(TypeError, match="lens"):
        chk([1, 2], "lens", None)
    with pytest.raises(ValueError, match="out must be a device tensor"):
        chk(torch.zeros(4), "out", None)


class _FakeDeviceTensor:
    """Duck-typed stand-in for a device tensor, to reach the checks after the device test on a
    machine without a GPU (the binding never hands it to the library in these tests)."""

    def __init__(self, shape, dtype, contiguous=True, device="cuda:0", nbytes=None):
        import torch
        self.shape, self.dtype, self._c = tuple(shape), dtype, contiguous
        self.device = torch.device(device)
        self.is_cuda = True
        self._n = 1
        for d in shape:
            self._n *= d
        self._nbytes = nbytes

    def is_contiguous(self):
        return self._c

    def numel(self):
        return self._n

    def element_size(self):
        import torch
        return torch.empty((), dtype=self.dtype).element_size() if self._nbytes is None else 1


def test_device_tensor_checks_after_device(monkeypatch):
    import torch
    monkeypatch.setattr(bst.bsattn.torch, "Tensor", _FakeDeviceTensor)
    chk = bst.bsattn._device_tensor
    ok = _FakeDeviceTensor((2,), torch.int32)
    assert chk(ok, "lens", "cuda:0", torch.int32, (2,)) is ok
    with pytest.raises(ValueError, match="lens is on cuda:1"):
        chk(_FakeDeviceTensor((2,), torch.int32, device="cuda:1"), "lens", "cuda:0")
    with pytest.raises(ValueError, match="contiguous"):
        chk(_FakeDeviceTensor((2,), torch.int32, contiguous=False), "lens", "cuda:0")
    with pytest.raises(ValueError, match="lens must be torch.int32"):
        chk(_FakeDeviceTensor((2,), torch.int64), "lens", "cuda:0", torch.int32)
    with pytest.raises(ValueError, match="shape"):
        chk(_FakeDeviceTensor((3,), torch.int32), "lens", "cuda:0", torch.int32, (2,))
    with pytest.raises(ValueError, match="bytes"):
        chk(_FakeDeviceTensor((100,), torch.uint8, nbytes=100), "workspace", "cuda:0",
            min_bytes=101)


def test_probe_rejects():
    from bench import probe_lib
    L = probe_lib()

    def last():
        return L.bsattn_probe_last_error().decode()
    fl = ctypes.c_double(0.0)
    assert L.bsattn_probe_sink_floats(4) == 1024 and L.bsattn_probe_sink_floats(0) == 0
    assert L.bsattn_probe_mfma_bf16(0, 4, FAKE, ctypes.byref(fl), None) == 1
    assert L.bsattn_probe_mfma_bf16(10, 70000, FAKE, ctypes.byref(fl), None) == 1
    assert L.bsattn_probe_mfma_bf16(10, 4, None, ctypes.byref(fl), None) == 1 and "sink" in last()
    assert L.bsattn_probe_read(FAKE, 24, 4, FAKE, None) == 1
    assert L.bsattn_probe_read(None, 32, 4, FAKE, None) == 1
    assert L.bsattn_probe_copy(FAKE, ctypes.c_void_p(0x10010), 64, 4, None) == 1 and "overlap" in last()
    assert L.bsattn_probe_copy(FAKE, ctypes.c_void_p(0x20000), 0, 4, None) == 1


def test_decode_ex_rejects():
    L = bst.lib()
    st = L.bsattn_decode_ex(1, 1, 1024, 4, 2, 64, 64, 4, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125,
                            FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == 1 and "flags" in last()
    st = L.bsattn_decode_ex(0, 1, 1024, 4, 2, 64, 64, 4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125,
                            FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == 2 and "bf16" in last()
