"""Python binding of libbsattn.so (ctypes): argument marshalling only.

Every step of the method runs in the library's gfx950 kernels; torch supplies device
memory and the current HIP stream. There is no fallback: if the library is missing or
was built for another target, loading raises.

The method: SparseFormer page (qqiyuan.cn, "2026 新一代卷积与Transformer网络架构技术演进与性能
对比"), section "SparseFormer 注意力实现": block_sparse_attention(q, k, v, block_size=64,
topk_ratio=0.3) on q/k/v [B, N, H, D] -- pool q/k per block, score blocks, keep the top
int(topk_ratio * num_blocks) key blocks per query block and head, attend over them with
scale 1/sqrt(D). GQA head mapping per the MSA page (cloud.baidu.com, "从M2.7到M3：多模态
模型稀疏注意力架构设计与实现全解析", §3.1).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# BSATTN_LIB names another build of the same library (the tests' host-sanitizer build)
LIB_PATH = os.environ.get("BSATTN_LIB") or os.path.join(_PKG, "libbsattn.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported size or dtype",
          3: "workspace missing or too small", 4: "HIP runtime error"}


class BsattnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"bsattn: {STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with block_sparse_top_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.bsattn_abi_version.restype = i32
    L.bsattn_abi_version.argtypes = []
    L.bsattn_status_str.restype = ctypes.c_char_p
    L.bsattn_status_str.argtypes = [i32]
    L.bsattn_last_error.restype = ctypes.c_char_p
    L.bsattn_last_error.argtypes = []
    L.bsattn_select_workspace_bytes.restype = sz
    L.bsattn_select_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
    L.bsattn_select.restype = i32
    L.bsattn_select.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.bsattn_forward.restype = i32
    L.bsattn_forward.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                 ctypes.c_float, ctypes.POINTER(ctypes.c_float), vp, vp]
    u32 = ctypes.c_uint
    L.bsattn_select_ex.restype = i32
    L.bsattn_select_ex.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, u32, i32,
                                   ctypes.c_uint64, i32, vp, vp, vp, vp, sz, vp]
    L.bsattn_forward_ex.restype = i32
    L.bsattn_forward_ex.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, u32, i32, vp, vp, vp,
                                    vp, ctypes.c_float, ctypes.POINTER(ctypes.c_float), vp, vp, vp]
    L.bsattn_select_noalloc_max_bytes.restype = sz
    L.bsattn_select_noalloc_max_bytes.argtypes = []
    L.bsattn_select_noalloc.restype = i32
    L.bsattn_select_noalloc.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, u32, i32,
                                        ctypes.c_uint64, i32, vp, vp, vp, vp]
    L.bsattn_key_blocks.restype = i64
    L.bsattn_key_blocks.argtypes = [i64, i32, i32]
    L.bsattn_select_workspace_bytes_ex.restype = sz
    L.bsattn_select_workspace_bytes_ex.argtypes = [i64, i64, i32, i32, i32, i32, i32]
    L.bsattn_backward_workspace_bytes.restype = sz
    L.bsattn_backward_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32, i32]
    L.bsattn_backward.restype = i32
    L.bsattn_backward.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, u32, vp, vp, vp, vp, vp,
                                  vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    L.bsattn_decode_pool.restype = i32
    L.bsattn_decode_pool.argtypes = [i32, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp]
    L.bsattn_decode_workspace_bytes.restype = sz
    L.bsattn_decode_workspace_bytes.argtypes = [i64, i32, i32, i32]
    L.bsattn_decode.restype = i32
    L.bsattn_decode.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                ctypes.c_float, vp, vp, vp, sz, vp]
    L.bsattn_decode_ex.restype = i32
    L.bsattn_decode_ex.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, ctypes.c_uint, vp, vp,
                                   vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise BsattnError(status, lib().bsattn_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _device_tensor(t, name: str, device, dtype=None, shape=None, min_bytes: int | None = None):
    """Refuses anything the library must not receive as a device pointer: a tensor on the
    host or on another device than `device`, a non-contiguous one, a wrong dtype or shape, or
    one smaller than `min_bytes`. Every tensor argument of every entry point passes here."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got one on {t.device})")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {min_bytes} needed")
    return t


def _shapes(q, k, v=None):
    if not isinstance(q, torch.Tensor) or not isinstance(k, torch.Tensor):
        raise TypeError("q and k must be torch tensors")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, N, H, D]")
    B, N, Hq, D = q.shape
    if k.shape[0] != B or k.shape[1] != N or k.shape[3] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _device_tensor(q, "q", None)
    _device_tensor(k, "k", q.device, q.dtype)
    if v is not None:
        _device_tensor(v, "v", q.device, q.dtype, k.shape)
    return B, N, Hq, k.shape[2], D


# option bits of the extended entry points (include/bsattn.h)
CAUSAL, POOL_MAX, GROUP_SELECT = 1, 2, 4


def _flags(causal=False, pooling="mean", group=False) -> int:
    if pooling not in ("mean", "max"):
        raise ValueError("pooling must be 'mean' or 'max'")
    return (CAUSAL if causal else 0) | (POOL_MAX if pooling == "max" else 0) | \
        (GROUP_SELECT if group else 0)


def topk_count(topk_ratio: float, num_blocks: int) -> int:
    """k = int(topk_ratio * num_blocks), as the SparseFormer page's sketch computes it."""
    return int(topk_ratio * num_blocks)


def select_workspace_bytes(B, N, Hq, Hkv, D, block, key_stride: int = 0) -> int:
    return int(lib().bsattn_select_workspace_bytes_ex(B, N, Hq, Hkv, D, block, key_stride))


def key_blocks(N: int, block: int, key_stride: int = 0) -> int:
    """Key blocks of N tokens at key_stride (0: block): the plain N // block, or the
    overlapping blocks starting every key_stride tokens, the last one ending at token N."""
    n = int(lib().bsattn_key_blocks(N, block, key_stride))
    if n < 0:
        raise BsattnError(1, lib().bsattn_last_error().decode())
    return n


def select(q, k, block: int, topk: int, *, causal: bool = False, pooling: str = "mean",
           group: bool = False, nrand: int = 0, seed: int = 0, key_stride: int = 0,
           return_pooled: bool = False, workspace=None):
    """Top-k key blocks per (batch, query head, query block): int32 [B, Hq, nb, topk].

    causal: own block forced, earlier blocks only, unused places -1; pooling "max": in-block
    maximum instead of the mean; group: one selection per KV head for all its query heads;
    nrand, seed: nrand of the topk places drawn at random from the non-top blocks;
    key_stride: overlapping key blocks starting every key_stride tokens (0: block), the
    entries then index those key blocks (`key_blocks`).
    With return_pooled, also returns the pooled q and k (fp32 [B, Hq, nb, D] and
    [B, Hkv, key blocks, D]; for fp8 inputs without the per-tensor descale).
    """
    flags = _flags(causal, pooling, group)
    B, N, Hq, Hkv, D = _shapes(q, k)
    nb = N // block if block > 0 else 0
    idx = torch.empty((B, Hq, nb, max(topk, 0)), dtype=torch.int32, device=q.device)
    valid = block > 0 and N % block == 0 and (key_stride == 0 or block <= 2 * key_stride <= 2 * block)
    nbytes = select_workspace_bytes(B, N, Hq, Hkv, D, block, key_stride) if valid else 0
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _device_tensor(workspace, "workspace", q.device, min_bytes=nbytes)
    with torch.cuda.device(q.device):
        _check(lib().bsattn_select_ex(_DTYPES[q.dtype], B, N, Hq, Hkv, D, block, topk, flags,
                                      int(nrand), int(seed) & ((1 << 64) - 1), int(key_stride),
                                      _ptr(q), _ptr(k), _ptr(idx), _ptr(workspace),
                                      workspace.numel(), _stream(q.device)))
    if not return_pooled:
        return idx
    nkb = key_blocks(N, block, key_stride)
    qb_bytes = (B * Hq * nb * D * 4 + 255) // 256 * 256
    qbar = workspace[: B * Hq * nb * D * 4].view(torch.float32).view(B, Hq, nb, D)
    kbar = workspace[qb_bytes: qb_bytes + B * Hkv * nkb * D * 4].view(torch.float32).view(
        B, Hkv, nkb, D)
    return idx, qbar, kbar


def forward(q, k, v, idx, scale: float | None = None, descales=(1.0, 1.0, 1.0), out=None, *,
            causal: bool = False, key_stride: int = 0, return_lse: bool = False):
    """Attention of every query block over its selected key blocks: [B, N, Hq, D].

    Output dtype: fp32 for fp32 inputs, bf16 for bf16 and fp8 inputs. causal: rows in the
    form `select(..., causal=True)` writes; keys after the query are masked. key_stride: idx
    names overlapping key blocks (as `select(..., key_stride=...)` writes them) and each query
    block attends to the union of their tokens. return_lse: also the rows' natural
    log-sum-exp, fp32 [B, Hq, N] (the input `backward` needs).
    """
    B, N, Hq, Hkv, D = _shapes(q, k, v)
    _device_tensor(idx, "idx", q.device, torch.int32)
    if idx.dim() != 4:
        raise ValueError("idx must be a contiguous int32 device tensor [B, Hq, nb, topk]")
    nb, topk = idx.shape[2], idx.shape[3]
    if idx.shape[0] != B or idx.shape[1] != Hq or (nb and N % nb):
        raise ValueError(f"idx shape {tuple(idx.shape)} does not match q {tuple(q.shape)}")
    block = N // nb if nb else 0
    if block == 0:
        raise ValueError("cannot infer the block size from an empty idx")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    odt = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=odt, device=q.device)
    else:
        _device_tensor(out, "out", q.device, odt, (B, N, Hq, D))
    ds = (ctypes.c_float * 3)(*[float(x) for x in descales])
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if return_lse else None
    with torch.cuda.device(q.device):
        _check(lib().bsattn_forward_ex(_DTYPES[q.dtype], B, N, Hq, Hkv, D, block, topk,
                                       CAUSAL if causal else 0, int(key_stride), _ptr(q),
                                       _ptr(k), _ptr(v),
                                       _ptr(idx), scale, ds, _ptr(out), _ptr(lse),
                                       _stream(q.device)))
    return (out, lse) if return_lse else out


def backward(q, k, v, idx, out, dout, lse, scale: float | None = None, *, causal: bool = False,
             workspace=None):
    """Gradients (dq, dk, dv), fp32, of the attention with the selection `idx` held fixed.

    out and lse come from `forward(..., return_lse=True)`; dout is bf16 like out.
    """
    B, N, Hq, Hkv, D = _shapes(q, k, v)
    _device_tensor(idx, "idx", q.device, torch.int32)
    if idx.dim() != 4 or idx.shape[0] != B or idx.shape[1] != Hq:
        raise ValueError("idx must be int32 [B, Hq, nb, topk]")
    nb, topk = idx.shape[2], idx.shape[3]
    block = N // nb if nb else 0
    _device_tensor(out, "out", q.device, torch.bfloat16, q.shape)
    _device_tensor(dout, "dout", q.device, torch.bfloat16, q.shape)
    _device_tensor(lse, "lse", q.device, torch.float32, (B, Hq, N))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    L = lib()
    nbytes = int(L.bsattn_backward_workspace_bytes(B, N, Hq, Hkv, D, block, topk)) if block else 0
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _device_tensor(workspace, "workspace", q.device, min_bytes=nbytes)
    with torch.cuda.device(q.device):
        _check(L.bsattn_backward(_DTYPES[q.dtype], B, N, Hq, Hkv, D, block, topk,
                                 CAUSAL if causal else 0, _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                 _ptr(out), _ptr(dout), _ptr(lse), scale, _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(workspace), workspace.numel(),
                                 _stream(q.device)))
    return dq, dk, dv


def block_sparse_attention(q, k, v, block_size: int = 64, topk_ratio: float = 0.3,
                           descales=(1.0, 1.0, 1.0), return_idx: bool = False, *,
                           causal: bool = False, pooling: str = "mean", group: bool = False,
                           overlap_ratio: float = 0.0):
    """The whole method: select, then attend with scale 1/sqrt(D).

    overlap_ratio: neighbouring key blocks share round(overlap_ratio * block_size) tokens
    (the MSA page's §5.3 suggests 0.25); top-k then counts int(topk_ratio * key blocks).
    """
    B, N, Hq, Hkv, D = _shapes(q, k, v)
    ks = block_size - int(round(overlap_ratio * block_size))
    topk = topk_count(topk_ratio, key_blocks(N, block_size, ks) if N else 0)
    idx = select(q, k, block_size, topk, causal=causal, pooling=pooling, group=group,
                 key_stride=ks)
    out = forward(q, k, v, idx, 1.0 / math.sqrt(D), descales, causal=causal, key_stride=ks)
    return (out, idx) if return_idx else out


def decode_pool(k_cache, lens_new, kbar, block: int, lens_old=None):
    """Pools the key blocks completed between lens_old and lens_new (all complete blocks if
    lens_old is None) into kbar, fp32 [B, Hkv, D, Lmax // block] (transposed), in place."""
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Lmax, Hkv, D]")
    B, Lmax, Hkv, D = k_cache.shape
    if k_cache.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k_cache.dtype}")
    dev = k_cache.device
    _device_tensor(k_cache, "k_cache", None)
    _device_tensor(lens_new, "lens_new", dev, torch.int32, (B,))
    if lens_old is not None:
        _device_tensor(lens_old, "lens_old", dev, torch.int32, (B,))
    _device_tensor(kbar, "kbar", dev, torch.float32,
                   (B, Hkv, D, Lmax // block if block > 0 else 0))
    with torch.cuda.device(k_cache.device):
        _check(lib().bsattn_decode_pool(_DTYPES[k_cache.dtype], B, Lmax, Hkv, D, block,
                                        _ptr(k_cache), _ptr(lens_old), _ptr(lens_new),
                                        _ptr(kbar), _stream(k_cache.device)))
    return kbar


def decode(q, k_cache, v_cache, kbar, lens, block: int, topk: int, scale: float | None = None,
           workspace=None, *, group: bool = False):
    """One decode step: q bf16 [B, Hq, D] (the newest token of each sequence), caches bf16
    [B, Lmax, Hkv, D], kbar from `decode_pool`, lens int32 [B] on the device. group: one
    choice of blocks per KV head from its query heads' summed scores, shared by them.
    Returns (out bf16 [B, Hq, D], idx int32 [B, Hq, topk])."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Lmax, Hkv, D]")
    B, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _device_tensor(q, "q", None)
    _device_tensor(k_cache, "k_cache", q.device, q.dtype, (B, Lmax, Hkv, D))
    _device_tensor(v_cache, "v_cache", q.device, q.dtype, (B, Lmax, Hkv, D))
    _device_tensor(kbar, "kbar", q.device, torch.float32,
                   (B, Hkv, D, Lmax // block if block > 0 else 0))
    _device_tensor(lens, "lens", q.device, torch.int32, (B,))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    idx = torch.empty((B, Hq, topk), dtype=torch.int32, device=q.device)
    L = lib()
    n = int(L.bsattn_decode_workspace_bytes(B, Hq, D, max(topk, 1))) if B else 0
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _device_tensor(workspace, "workspace", q.device, min_bytes=n)
    with torch.cuda.device(q.device):
        _check(L.bsattn_decode_ex(_DTYPES[q.dtype], B, Lmax, Hq, Hkv, D, block, topk,
                                  GROUP_SELECT if group else 0, _ptr(q), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(kbar), _ptr(lens), scale, _ptr(out),
                                  _ptr(idx), _ptr(workspace), workspace.numel(),
                                  _stream(q.device)))
    return out, idx
