"""bsattn_select_noalloc (static device scratch, no workspace argument) against
bsattn_select_ex with a caller workspace: identical indices on two calls in a row, the
second with a smaller input, and a call on the many-block path (score matrix in the scratch)."""
import ctypes
import sys

import pytest
import torch

import block_sparse_top_amd as bst
from block_sparse_top_amd import synthetic as syn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _both(shape, dtype, flags=0, nrand=0, seed=0, index=61):
    B, N, Hq, Hkv, D, blk, topk = shape
    L = bst.lib()
    q, k, _, _ = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=index, device=DEV)
    nb = N // blk
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dcode = bst.bsattn._DTYPES[q.dtype]
    ws = torch.empty(bst.select_workspace_bytes(B, N, Hq, Hkv, D, blk), dtype=torch.uint8,
                     device=DEV)
    ref = torch.full((B, Hq, nb, topk), -7, dtype=torch.int32, device=DEV)
    got = torch.full((B, Hq, nb, topk), -7, dtype=torch.int32, device=DEV)
    st = L.bsattn_select_ex(dcode, B, N, Hq, Hkv, D, blk, topk, flags, nrand, seed, 0, P(q),
                            P(k), P(ref), P(ws), ws.numel(), sp)
    assert st == 0, L.bsattn_last_error()
    st = L.bsattn_select_noalloc(dcode, B, N, Hq, Hkv, D, blk, topk, flags, nrand, seed, 0,
                                 P(q), P(k), P(got), sp)
    assert st == 0, L.bsattn_last_error()
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry_point():
    say("[noalloc] two calls in a row, the second smaller")
    r1, g1 = _both((2, 64 * 200, 8, 2, 64, 64, 60), "bf16")
    assert torch.equal(r1, g1)
    r2, g2 = _both((1, 64 * 37, 4, 2, 128, 64, 9), "f32", flags=bst.CAUSAL, index=62)
    assert torch.equal(r2, g2)
    say("[noalloc] many-block path and random places")
    r3, g3 = _both((1, 64 * 1088, 2, 1, 64, 64, 100), "bf16", index=63)
    assert torch.equal(r3, g3)
    r4, g4 = _both((2, 64 * 40, 4, 4, 64, 64, 8), "bf16", nrand=2, seed=99, index=64)
    assert torch.equal(r4, g4)


def test_noalloc_rejects_oversized():
    L = bst.lib()
    big = L.bsattn_select_noalloc(1, 8, 65536, 16, 16, 128, 64, 307, 0, 0, 0, 0, None, None,
                                  None, None)
    assert big == 3 and "static scratch" in L.bsattn_last_error().decode()
