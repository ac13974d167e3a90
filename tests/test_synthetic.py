"""Seeded input generators: determinism, shapes, fp8 scaling, planted structure."""
import math

import numpy as np
import torch

from block_sparse_top_amd import synthetic as syn
import oracle.bsattn_oracle as O


def test_iid_deterministic_and_shaped():
    a = syn.iid_inputs(1, 128, 4, 2, 16, "bf16", index=7)
    b = syn.iid_inputs(1, 128, 4, 2, 16, "bf16", index=7)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert a[0].shape == (1, 128, 4, 16) and a[1].shape == (1, 128, 2, 16)
    assert a[0].dtype == torch.bfloat16 and a[3] == (1.0, 1.0, 1.0)
    c = syn.iid_inputs(1, 128, 4, 2, 16, "bf16", index=8)
    assert not torch.equal(a[0], c[0])


def test_fp8_scaling():
    q, k, v, ds = syn.iid_inputs(1, 256, 2, 2, 32, "fp8", index=3)
    assert q.dtype == torch.float8_e4m3fn
    for x, d in zip((q, k, v), ds):
        vals = O.decode_e4m3(x.view(torch.uint8).numpy())
        assert np.nanmax(np.abs(vals)) == 448.0          # amax maps to the top code
        assert not np.isnan(vals).any()
        assert d > 0


def test_planted_structure_recovered_by_oracle():
    B, N, H, D, blk = 1, 2048, 2, 32, 32
    nb = N // blk
    kk = int(0.2 * nb)
    q, k, v, ds, planted = syn.planted_inputs(B, N, H, H, D, blk, kk, "f32", index=3)
    idx = O.select(q.double().numpy(), k.double().numpy(), blk, kk)
    # planted and other blocks differ by about 1.6 standard deviations of the score, so
    # recovery is statistical: well above the chance rate kk/nb = 0.19
    hits = np.mean([len(set(a) & set(b)) / kk for a, b in
                    zip(idx.reshape(-1, kk), planted.numpy().reshape(-1, kk))])
    assert hits > 0.45


def test_sample_rows():
    a = syn.sample_rows(10, 100, index=2)
    assert a == syn.sample_rows(10, 100, index=2)
    assert len(set(a)) == 10 and a == sorted(a)


def test_workload_table():
    w = syn.WORKLOADS["sparseformer_n8192_bf16"]
    assert (w.B, w.N, w.Hq, w.D, w.block, w.nb) == (32, 8192, 16, 64, 64, 128)
    assert O.topk_count(w.ratio, w.nb) == 38
    assert O.topk_count(syn.WORKLOADS["longctx_gqa_n1m_bf16"].ratio, 8192) == 1228
