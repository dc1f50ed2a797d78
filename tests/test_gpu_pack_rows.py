"""GPU parity of msa_index_select_pack_rows: the batch's own keys written into
the tiled cache and steps 1-3, in one call.  Its tiles, selection and scores
must equal msa_pack_kv_tiled_rows followed by msa_index_select bit for bit
(every tile element, NaN patterns included), on every path the selection takes:
one-row batches (the writer's workgroups ride in the fused launch), windows of
up to 16 rows (they ride in the scores launch), key heads in fours or not, and
prompt chunks (a launch of their own first), over contiguous and paged caches;
and the decode attention after it must equal the two-call step's."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
from gpu_helpers import device_tensors, say, shape_of
from test_gpu_tiled import aligned_copy, u16
from workloads import make_case, to_pages

pytestmark = pytest.mark.gpu

CASES = {
    "one_row": dict(seq_lens=[40000, 7000, 300], rows=[1, 1, 1], n_kv_heads=4, seed=231),
    "one_row_h3": dict(seq_lens=[9000, 65, 1], rows=[1, 1, 1], n_kv_heads=3, seed=232),
    "windows": dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[16, 1, 16, 7, 3], n_kv_heads=4, seed=233),
    "windows_h2": dict(seq_lens=[3000, 900], rows=[16, 5], n_kv_heads=2, seed=234),
    "chunk": dict(seq_lens=[3000, 900], rows=[300, 1], n_kv_heads=2, seed=235),
}


def _setup(name, layout):
    """The case's tensors, batch, and the cache token of key j of sequence s."""
    case = make_case(name, **CASES[name])
    t = device_tensors(case)
    if layout == "paged":
        pool, pt = to_pages(case, seed=17, extra_pages=2)
        t.update({n: x.cuda() for n, x in pool.items()})
        batch = msa.Batch(case.seq_lens, case.rows, page_table=pt)
        tok = lambda s, j: int(pt[s, j // 64]) * 64 + j % 64
    else:
        t, starts = aligned_copy(case, t)
        batch = msa.Batch(case.seq_lens, case.rows, kv_start=starts)
        tok = lambda s, j: starts[s] + j
    return case, t, batch, tok


def _tiles_without_rows(case, t, tok):
    """A tiled cache holding every key but the batch's own, which stay NaN
    (packed from a copy of the cache with those keys set to NaN)."""
    kz, vz = t["k"].clone(), t["v"].clone()
    for s, (L, n) in enumerate(zip(case.seq_lens, case.rows)):
        for j in range(L - n, L):
            kz[tok(s, j)] = float("nan")
            vz[tok(s, j)] = float("nan")
    kvt = msa.KVTiled.empty(t["k"].shape[0], case.n_kv_heads, "cuda", fill=float("nan"))
    msa.msa_pack_kv_tiled(shape_of(case), kz, vz, kvt)
    return kvt


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
@pytest.mark.parametrize("name", list(CASES))
def test_pack_rows_in_the_selection_launch(name, layout):
    case, t, batch, tok = _setup(name, layout)
    shape = shape_of(case)
    say(f"[gpu] index_select_pack_rows {name} {layout}: seqs={case.seq_lens} rows={case.rows}")
    base = _tiles_without_rows(case, t, tok)
    want_t = msa.KVTiled(base.k.clone(), base.v.clone())
    got_t = msa.KVTiled(base.k.clone(), base.v.clone())
    n_blk = batch.n_blocks
    R, H, K = batch.total_rows, case.n_kv_heads, case.top_k
    with_scores = [True] + ([False] if name == "chunk" else [])
    for keep_scores in with_scores:
        s_w = torch.full((R, H, n_blk), -7.0, device="cuda") if keep_scores else None
        s_g = torch.full((R, H, n_blk), -7.0, device="cuda") if keep_scores else None
        i_w = torch.full((R, H, K), -7, dtype=torch.int32, device="cuda")
        i_g = torch.full((R, H, K), -7, dtype=torch.int32, device="cuda")
        ws_w = msa.index_select_workspace(shape, batch)
        ws_g = msa.index_select_workspace(shape, batch)
        msa.msa_pack_kv_tiled_rows(shape, batch, t["k"], t["v"], want_t)
        msa.msa_index_select(shape, batch, t["iq"], t["ik"], s_w, i_w, ws_w)
        msa.msa_index_select_pack_rows(shape, batch, t["iq"], t["ik"], s_g, i_g, t["k"], t["v"], got_t, ws_g)
        torch.cuda.synchronize()
        assert np.array_equal(u16(got_t.k), u16(want_t.k)), "K tiles differ"
        assert np.array_equal(u16(got_t.v), u16(want_t.v)), "V tiles differ"
        assert torch.equal(i_g, i_w), "selection differs"
        if keep_scores:
            assert torch.equal(s_g.view(torch.int32), s_w.view(torch.int32)), "scores differ"
        # the workspace counters are back at zero for the next call
        assert int(ws_g[:256 * 1024].view(torch.int32).abs().sum().item()) == 0
    # the step's attention over the tiles it wrote
    o_w, o_g = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    l_w = torch.empty(R, H * 16, device="cuda")
    l_g = torch.empty(R, H * 16, device="cuda")
    if max(case.rows) <= 16:
        msa.msa_decode_tiled(shape, batch, t["q"], want_t, i_w, o_w, l_w, msa.decode_workspace(shape, R))
        msa.msa_decode_tiled(shape, batch, t["q"], got_t, i_g, o_g, l_g, msa.decode_workspace(shape, R))
    else:
        msa.msa_prefill_tiled(shape, batch, t["q"], want_t, i_w, o_w, l_w)
        msa.msa_prefill_tiled(shape, batch, t["q"], got_t, i_g, o_g, l_g)
    torch.cuda.synchronize()
    assert not torch.isnan(o_g.float()).any(), "the attention read a key left unwritten"
    assert torch.equal(o_g.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(l_g.view(torch.int32), l_w.view(torch.int32))
