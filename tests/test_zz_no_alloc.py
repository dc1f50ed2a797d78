"""msa_decode_tiled_noalloc (the decode over the tiled cache with the
library's static per-device workspace, for callers that cannot allocate)
against msa_decode_tiled with a caller workspace: the same kernels, so the
outputs and lse must be equal bit for bit.  Calls run back to back on the one
static workspace, larger batches first, then smaller ones, then a batch of
one workgroup per unit (no workspace) and a split batch again."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
from gpu_helpers import device_tensors, say, shape_of
from workloads import make_case

pytestmark = pytest.mark.gpu

# every sequence length a multiple of 64, so every sequence starts a tile
CALLS = [
    # 4 rows x 4 key heads = 16 units: the split kernel (4 partials per unit)
    dict(name="split16", seq_lens=[9024, 3008, 704], rows=[1, 2, 1], n_kv_heads=4, seed=901),
    # smaller: 1 row x 2 key heads at top_k 5 (2 partials per unit)
    dict(name="split2", seq_lens=[2560], rows=[1], n_kv_heads=2, seed=902, top_k=5),
    # 96 units: one workgroup per unit, no workspace touched
    dict(name="unit96", seq_lens=[1280, 640], rows=[16, 8], n_kv_heads=4, seed=903),
    # the split kernel again at top_k 32 (8 partials per unit), on the same array
    dict(name="split_top32", seq_lens=[4096, 1984], rows=[1, 1], n_kv_heads=3, seed=904, top_k=32),
]


def _one(kw):
    case = make_case(**kw)
    t = device_tensors(case)
    shape = shape_of(case)
    batch = msa.Batch(case.seq_lens, case.rows)
    kvt = msa.KVTiled.empty(t["k"].shape[0], case.n_kv_heads, "cuda", fill=float("nan"))
    msa.msa_pack_kv_tiled(shape, t["k"], t["v"], kvt)
    o = msa.run_path(shape, batch, t, "decode", kvt=kvt)        # selection + decode with a workspace
    out2 = torch.full_like(o["out"], float("nan"))
    lse2 = torch.full_like(o["lse"], float("nan"))
    msa.msa_decode_tiled_noalloc(shape, batch, t["q"], kvt, o["block_idx"], out2, lse2)
    torch.cuda.synchronize()
    return o["out"].cpu(), o["lse"].cpu(), out2.cpu(), lse2.cpu()


def test_noalloc_equals_workspace_decode_in_a_row():
    for rep in range(2):
        for kw in CALLS:
            say(f"[gpu] noalloc {kw['name']} rep {rep}")
            out, lse, out2, lse2 = _one(kw)
            assert torch.isfinite(out.float()).all()
            assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), kw["name"]
            assert np.array_equal(lse.numpy().view(np.uint32), lse2.numpy().view(np.uint32)), kw["name"]
