"""GPU parity of the paged key layout (pages of 64 tokens = one sparse block,
a page table per sequence): the same inputs scattered into a page pool in a
random page order must give bit for bit the results of the contiguous layout
(same arithmetic, only the addressing differs), pass the oracle checks, and
let sequences share the pages of a common prefix."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
import oracle
from gpu_helpers import (check_lse, check_out, check_scores, check_selection, device_tensors, say,
                         shape_of)
from workloads import make_case, to_pages

pytestmark = pytest.mark.gpu
B = 64


def page_pool(case, seed, extra_pages=5, shared=None):
    pool, pt = to_pages(case, seed, extra_pages, shared)
    return {n: x.cuda() for n, x in pool.items()}, pt


def run(case, t, batch, mode, fused=False):
    out = msa.run_path(shape_of(case), batch, t, mode, fused=fused)
    torch.cuda.synchronize()
    return {n: x.cpu() for n, x in out.items() if n not in ("workspace", "select_workspace")}


CASES = {
    # > 16 rows: the LDS-tiled indexer and the merged-walk prefill
    "tiled": (dict(seq_lens=[700, 1500, 300, 64], rows=[300, 5, 300, 64], n_kv_heads=2, seed=301), "prefill"),
    # <= 16 rows: the streaming indexer, decode and the fused selection
    "window": (dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[16, 1, 16, 7, 3], n_kv_heads=3, seed=302), "decode"),
    "shared_ik": (dict(seq_lens=[4000, 900], rows=[40, 8], n_kv_heads=4, seed=303, ik_shared=True), "prefill"),
    # enough rows for the prefill to put four rows in each wave
    "walk4": (dict(seq_lens=[2600, 700], rows=[2000, 100], n_kv_heads=4, seed=306), "prefill"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_paged_equals_contiguous(name):
    kw, mode = CASES[name]
    case = make_case(name, **kw)
    dense = run(case, device_tensors(case), msa.Batch(case.seq_lens, case.rows), mode)
    pool, pt = page_pool(case, seed=kw["seed"])
    t = dict(device_tensors(case), **pool)
    paged_batch = msa.Batch(case.seq_lens, case.rows, page_table=pt)
    for fused in ([False, True] if mode == "decode" else [False]):
        paged = run(case, t, paged_batch, mode, fused=fused)
        say(f"[gpu] paged {name} {mode} fused={fused}")
        for n in ("block_scores", "block_idx", "out", "lse"):
            assert torch.equal(dense[n], paged[n]), n
    if mode == "prefill":   # the other attention entry point on the same pages
        d2 = run(case, device_tensors(case), msa.Batch(case.seq_lens, case.rows), "decode")
        p2 = run(case, t, paged_batch, "decode")
        assert torch.equal(d2["out"], p2["out"])


def test_paged_against_oracle():
    case = make_case("paged_oracle", [6000, 2500, 130], [24, 16, 3], 2, seed=304)
    ref = oracle.run(case)
    pool, pt = page_pool(case, seed=304)
    t = dict(device_tensors(case), **pool)
    batch = msa.Batch(case.seq_lens, case.rows, page_table=pt)
    rows = np.arange(case.total_rows)
    for mode in ("prefill", "decode"):
        g = run(case, t, batch, mode)
        check_scores(case, g, rows, ref)
        clear = check_selection(case, g, rows, ref, case.top_k)
        own_out, own_lse = oracle.attention(case, g["block_idx"].numpy(), rows)
        check_out(g["out"], own_out, f"paged/{mode}/own-selection")
        check_lse(g["lse"], own_lse, f"paged/{mode}/own-selection")
        ok = clear.all(axis=1)
        check_out(g["out"][ok], ref["out"][ok], f"paged/{mode}/e2e")


def test_shared_prefix_pages_and_chunk_resume():
    """Sequence 1 resumes a 300-row prompt chunk on top of sequence 0's
    cached 4,096-key prefix (64 pages referenced, not copied); sequence 0 is
    a one-row step on the prefix alone.  Equal to the contiguous layout with
    the prefix duplicated."""
    P = 4096
    case = make_case("prefix", [P, P + 300], [1, 300], 2, seed=305)
    s1 = case.kv_start[1]
    for n in ("k", "v", "ik"):
        getattr(case, n)[s1:s1 + P] = getattr(case, n)[:P]
    dense = run(case, device_tensors(case), msa.Batch(case.seq_lens, case.rows), "prefill")
    pool, pt = page_pool(case, seed=305, shared=(0, 1, P // B))
    assert (pt[1, :P // B] == pt[0, :P // B]).all()
    t = dict(device_tensors(case), **pool)
    paged = run(case, t, msa.Batch(case.seq_lens, case.rows, page_table=pt), "prefill")
    for n in ("block_scores", "block_idx", "out", "lse"):
        assert torch.equal(dense[n], paged[n]), n


def test_shared_pages_across_sequences_in_one_walk():
    """Two 1,050-row chunks resumed on one shared 2,048-key prefix, with enough
    rows (x 4 key heads) for four rows per prefill wave: the wave holding rows
    1,048-1,051 mixes the two sequences, and a prefix page both kept is one
    group of the walk (loaded once, folded into rows of both sequences).
    Equal to the contiguous layout with the prefix duplicated."""
    P, n = 2048, 1050
    case = make_case("xprefix", [P + n, P + n], [n, n], 4, seed=306)
    s1 = case.kv_start[1]
    for name in ("k", "v", "ik"):
        getattr(case, name)[s1:s1 + P] = getattr(case, name)[:P]
    dense = run(case, device_tensors(case), msa.Batch(case.seq_lens, case.rows), "prefill")
    pool, pt = page_pool(case, seed=306, shared=(0, 1, P // B))
    t = dict(device_tensors(case), **pool)
    paged = run(case, t, msa.Batch(case.seq_lens, case.rows, page_table=pt), "prefill")
    for name in ("block_scores", "block_idx", "out", "lse"):
        assert torch.equal(dense[name], paged[name]), name
    # the boundary wave's rows of the two sequences keep common prefix pages
    idx = paged["block_idx"].numpy()
    common = 0
    for h in range(case.n_kv_heads):
        a = {int(pt[0, b]) for r in (n - 2, n - 1) for b in idx[r, h] if 0 <= b < P // B}
        c = {int(pt[1, b]) for r in (n, n + 1) for b in idx[r, h] if 0 <= b < P // B}
        common += len(a & c)
    say(f"[gpu] prefix pages kept by both sequences in the boundary wave: {common}")
    assert common > 0
