"""Seeded synthetic inputs for block-sparse top-k attention.

This module is the one piece shared by the GPU path's tests/bench and the fp64
oracle's tests: it only draws random tensors. It holds none of the method's
arithmetic (no pooling, scoring, selection or attention) and imports neither
the HIP binding nor the oracle.

Workloads follow the shapes the pages discuss:
  * SparseFormer page (qqiyuan.cn, "2026 新一代卷积与Transformer网络架构技术演进与性能对比"),
    table under "基准测试": sequence 8192, hidden 1024, batch 32; code sketch under
    "SparseFormer 注意力实现": q/k/v laid out [B, N, H, D], block_size 64, topk_ratio 0.3.
  * MSA page (cloud.baidu.com, "从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析"),
    §3.2 parameter table (block_size 64-256, topk_ratio 0.15-0.3), §3.2 1M-token
    context at block 128, §3.1 GQA-based attention block.
No page prints input data, so every tensor is i.i.d. normal (or the planted
structure described in `planted_inputs`), drawn in fp32 from a seeded torch
generator and then rounded to the storage dtype (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
import math

import torch

FP8_MAX = 448.0  # largest finite OCP e4m3 ("fn") magnitude


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    block: int
    ratio: float
    dtype: str            # "f32" | "bf16" | "fp8"
    structure: str = "iid"  # "iid" | "planted"
    index: int = 0        # seed family

    @property
    def nb(self) -> int:
        return self.N // self.block


# The five workloads, in seed-family order 1..5.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, N=512, Hq=2, Hkv=2, D=64, block=64,
                         ratio=0.25, dtype="f32", index=1),
    "sparseformer_n8192_bf16": Workload("sparseformer_n8192_bf16", B=32, N=8192, Hq=16, Hkv=16,
                                        D=64, block=64, ratio=0.3, dtype="bf16", index=2),
    "planted_n32768_bf16": Workload("planted_n32768_bf16", B=4, N=32768, Hq=16, Hkv=16, D=128,
                                    block=128, ratio=0.2, dtype="bf16", structure="planted",
                                    index=3),
    "longctx_gqa_n1m_bf16": Workload("longctx_gqa_n1m_bf16", B=1, N=1 << 20, Hq=32, Hkv=8,
                                     D=128, block=128, ratio=0.15, dtype="bf16", index=4),
    "fp8_n65536": Workload("fp8_n65536", B=8, N=65536, Hq=16, Hkv=16, D=128, block=64,
                           ratio=0.3, dtype="fp8", index=5),
}


# Decode workload (one new token per sequence against a full KV cache of N tokens).
DECODE_WORKLOADS = {
    "decode_gqa_l32768": Workload("decode_gqa_l32768", B=32, N=32768, Hq=32, Hkv=8, D=128,
                                  block=64, ratio=0.15, dtype="bf16", index=6),
}


def seeds(index: int) -> dict:
    """Seed family of a workload: q, k, v, sampling and planted-structure streams."""
    base = 1000 * index
    return {"q": base + 1, "k": base + 2, "v": base + 3, "sample": base + 4, "planted": base + 5}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed: int, device="cpu", chunk_elems: int = 1 << 28) -> torch.Tensor:
    """fp32 N(0,1) tensor from one seeded generator (drawn in chunks to bound memory)."""
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(flat.numel(), s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
    return out


def to_storage(x32: torch.Tensor, dtype: str):
    """Round an fp32 tensor to the storage dtype. Returns (tensor, descale).

    fp8: per-tensor amax scaling to the e4m3 range; the stored code times `descale`
    is the value the method sees. Other dtypes: descale 1.0.
    """
    if dtype == "f32":
        return x32.contiguous(), 1.0
    if dtype == "bf16":
        return x32.to(torch.bfloat16).contiguous(), 1.0
    if dtype == "fp8":
        amax = float(x32.abs().max())
        amax = amax if amax > 0 else 1.0
        x8 = (x32 * (FP8_MAX / amax)).to(torch.float8_e4m3fn).contiguous()
        return x8, amax / FP8_MAX
    raise ValueError(f"unknown dtype {dtype}")


def iid_inputs(B, N, Hq, Hkv, D, dtype="bf16", index=0, device="cpu"):
    """q [B,N,Hq,D], k/v [B,N,Hkv,D], i.i.d. N(0,1), rounded to `dtype`.

    Returns (q, k, v, descales) with descales = (dq, dk, dv).
    """
    s = seeds(index)
    out, ds = [], []
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        x32 = randn((B, N, H, D), s[name], device)
        x, d = to_storage(x32, dtype)
        del x32
        out.append(x)
        ds.append(d)
    return out[0], out[1], out[2], tuple(ds)


def decode_inputs(w: Workload, device="cpu"):
    """Decode inputs: the newest query token q [B, Hq, D] and caches k, v [B, N, Hkv, D],
    i.i.d. N(0,1) rounded to the workload's dtype (the q, k, v seeds of its family)."""
    s = seeds(w.index)
    q, _ = to_storage(randn((w.B, w.Hq, w.D), s["q"], device), w.dtype)
    k, _ = to_storage(randn((w.B, w.N, w.Hkv, w.D), s["k"], device), w.dtype)
    v, _ = to_storage(randn((w.B, w.N, w.Hkv, w.D), s["v"], device), w.dtype)
    return q, k, v


def planted_inputs(B, N, Hq, Hkv, D, block, planted_k, dtype="bf16", index=0, device="cpu",
                   mean_var=0.5):
    """Inputs with a planted block structure.

    Every key block j of KV head g gets a mean vector mu[b,g,j] ~ N(0, mean_var*I);
    its tokens are mu + N(0, I). For every (batch, query head, query block) a set of
    `planted_k` distinct key blocks is drawn; with u the sum of their means, the query
    tokens are sqrt(D)*u/|u| + N(0, I). Values are rounded to `dtype` at the end.
    Returns (q, k, v, descales, planted) with planted [B,Hq,nb,planted_k] (sorted).
    """
    s = seeds(index)
    nb = N // block
    G = Hq // Hkv
    gp = _gen(s["planted"], device)
    mu = torch.randn((B, Hkv, nb, D), generator=gp, device=device) * math.sqrt(mean_var)
    # planted key-block sets: the first planted_k entries of a random permutation
    keys = torch.rand((B, Hq, nb, nb), generator=gp, device=device)
    planted = keys.argsort(dim=-1)[..., :planted_k].sort(dim=-1).values
    del keys

    k32 = randn((B, N, Hkv, D), s["k"], device)
    k32.view(B, nb, block, Hkv, D).add_(mu.permute(0, 2, 1, 3).unsqueeze(2))

    q32 = randn((B, N, Hq, D), s["q"], device)
    kv_of_h = torch.arange(Hq, device=device) // G
    mu_h = mu[:, kv_of_h]                                   # [B,Hq,nb,D]
    u = torch.gather(mu_h, 2, planted.reshape(B, Hq, nb * planted_k, 1).expand(-1, -1, -1, D))
    u = u.view(B, Hq, nb, planted_k, D).sum(3)              # [B,Hq,nb,D]
    u = u * (math.sqrt(D) / u.norm(dim=-1, keepdim=True).clamp_min(1e-30))
    q32.view(B, nb, block, Hq, D).add_(u.permute(0, 2, 1, 3).unsqueeze(2))

    v32 = randn((B, N, Hkv, D), s["v"], device)
    q, dq = to_storage(q32, dtype)
    del q32
    k, dk = to_storage(k32, dtype)
    del k32
    v, dv = to_storage(v32, dtype)
    del v32
    return q, k, v, (dq, dk, dv), planted


def workload_inputs(w: Workload, device="cpu"):
    """Inputs of a named workload. Returns (q, k, v, descales, extra)."""
    if w.structure == "planted":
        planted_k = int(w.ratio * w.nb)
        q, k, v, ds, planted = planted_inputs(w.B, w.N, w.Hq, w.Hkv, w.D, w.block, planted_k,
                                              w.dtype, w.index, device)
        return q, k, v, ds, {"planted": planted}
    q, k, v, ds = iid_inputs(w.B, w.N, w.Hq, w.Hkv, w.D, w.dtype, w.index, device)
    return q, k, v, ds, {}


def sample_rows(count: int, population: int, index: int, salt: int = 0):
    """`count` distinct sorted row numbers out of `population`, from the sampling seed."""
    g = _gen(seeds(index)["sample"] + salt, "cpu")
    count = min(count, population)
    return torch.randperm(population, generator=g)[:count].sort().values.tolist()


def random_block_sets(B: int, H: int, nq: int, nkb: int, topk: int, index: int,
                      device="cpu") -> torch.Tensor:
    """int32 [B, H, nq, topk]: per row, topk distinct key blocks out of [0, nkb), seeded.

    Rows 3m are runs of consecutive blocks (neighbours share tokens when key blocks overlap),
    rows 3m+1 the run that ends at the last key block, rows 3m+2 random sets; rows are
    ascending except every fifth row, which is descending (attention takes a row's entries
    in any order).
    """
    g = _gen(seeds(index)["sample"] + 101, "cpu")
    rows = B * H * nq
    sets = torch.rand((rows, nkb), generator=g).argsort(dim=1)[:, :topk].sort(dim=1).values
    r = torch.arange(rows)[:, None]
    start = torch.randint(0, nkb - topk + 1, (rows, 1), generator=g)
    step = torch.arange(topk)[None, :]
    sets = torch.where(r % 3 == 0, start + step, sets)
    sets = torch.where(r % 3 == 1, nkb - topk + step, sets)
    sets = torch.where(r % 5 == 0, sets.flip(1), sets)
    return sets.to(torch.int32).reshape(B, H, nq, topk).to(device)
