"""GPU parity of msa_index_select (index scores, max-pool and selection in one
call: one launch when every sequence has one row, else the two launches of
msa_index_scores + msa_select_blocks): its block_idx and block_scores must
equal msa_index_scores + msa_select_blocks bit for bit, and the whole path
through it must pass the same oracle checks."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
from gpu_helpers import device_tensors, full_check, gpu_run, say, shape_of
from workloads import config, make_case

pytestmark = pytest.mark.gpu

CASES = {
    # ragged, a 1-key sequence, 1..16 rows per sequence, 3 key heads
    "ragged": dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[16, 1, 16, 7, 3], n_kv_heads=3, seed=201),
    "shared_ik": dict(seq_lens=[4000, 900], rows=[16, 5], n_kv_heads=4, seed=202, ik_shared=True),
    "top1": dict(seq_lens=[1200, 800], rows=[4, 3], n_kv_heads=2, seed=203, top_k=1),
    "top5": dict(seq_lens=[3000, 1500], rows=[16, 3], n_kv_heads=2, seed=204, top_k=5),
    "top32": dict(seq_lens=[5000, 2100], rows=[16, 2], n_kv_heads=2, seed=205, top_k=32),
    "one_row": dict(seq_lens=[40000, 7000, 300], rows=[1, 1, 1], n_kv_heads=2, seed=206),
    # one row per sequence (the one-launch path), ragged, with 1-, 64- and 65-key sequences
    "one_row_ragged": dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[1] * 5, n_kv_heads=3, seed=212),
    "one_row_shared_ik": dict(seq_lens=[4000, 900], rows=[1, 1], n_kv_heads=4, seed=213, ik_shared=True),
    "one_row_top1": dict(seq_lens=[1200, 800], rows=[1, 1], n_kv_heads=2, seed=214, top_k=1),
    "one_row_top5": dict(seq_lens=[3000, 1500], rows=[1, 1], n_kv_heads=2, seed=215, top_k=5),
    "one_row_top32": dict(seq_lens=[5000, 2100], rows=[1, 1], n_kv_heads=2, seed=216, top_k=32),
}


def _both(case, t=None, top_k=None):
    t = t or device_tensors(case)
    a = gpu_run(case, "decode", t=t, top_k=top_k)
    b = gpu_run(case, "decode", t=t, top_k=top_k, fused=True)
    return a, b


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_two_step_and_oracle(name):
    case = make_case(name, **CASES[name])
    a, b = _both(case)
    assert torch.equal(a["block_scores"], b["block_scores"])
    assert torch.equal(a["block_idx"], b["block_idx"])
    assert torch.equal(a["out"], b["out"])
    full_check(case, "decode", fused=True)


@pytest.mark.parametrize("name", ["decode", "long", "windows"])
def test_fused_full_configs(name):
    case = config(name)
    a, b = _both(case)
    assert torch.equal(a["block_scores"], b["block_scores"])
    assert torch.equal(a["block_idx"], b["block_idx"])
    if name == "windows":
        idx = b["block_idx"].numpy()
        for s in range(case.n_seqs):
            for r in range(case.cu_rows[s], case.cu_rows[s + 1]):
                for h in range(case.n_kv_heads):
                    assert set(case.needles[s]) <= set(idx[r, h].tolist())
    else:
        full_check(case, "decode", fused=True)


def test_fused_workspace_reuse_and_counters():
    case = make_case("ws", [9000, 3000, 70], [1, 1, 1], 2, seed=207)
    shape = shape_of(case)
    batch = msa.Batch(case.seq_lens, case.rows)
    t = device_tensors(case)
    ws = msa.index_select_workspace(shape, batch)
    res = []
    for _ in range(3):
        s = torch.empty(batch.total_rows, 2, batch.n_blocks, dtype=torch.float32, device="cuda")
        i = torch.empty(batch.total_rows, 2, case.top_k, dtype=torch.int32, device="cuda")
        msa.msa_index_select(shape, batch, t["iq"], t["ik"], s, i, ws)
        res.append(i)
    torch.cuda.synchronize()
    assert torch.equal(res[0], res[1]) and torch.equal(res[0], res[2])
    # the counters (the first 256 KiB) are left at zero; the range maxima after them are scratch
    assert int(ws[:256 * 1024].view(torch.int32).abs().sum().item()) == 0


def test_prompt_chunk_with_scores_takes_two_launches():
    """More than 16 rows in a sequence with block_scores given: the two
    separate steps' launches, scores written as msa_index_scores writes them."""
    case = make_case("chunk", [3000, 900], [300, 1], 2, seed=208)
    shape = shape_of(case)
    batch = msa.Batch(case.seq_lens, case.rows)
    t = device_tensors(case)
    a = gpu_run(case, "decode", t=t)
    s = torch.empty(batch.total_rows, 2, batch.n_blocks, dtype=torch.float32, device="cuda")
    i = torch.empty(batch.total_rows, 2, case.top_k, dtype=torch.int32, device="cuda")
    msa.msa_index_select(shape, batch, t["iq"], t["ik"], s, i)
    torch.cuda.synchronize()
    assert torch.equal(a["block_scores"], s.cpu())
    assert torch.equal(a["block_idx"], i.cpu())


def test_max_context_one_row():
    """The largest context the selection stages (16,384 blocks = 1,048,576
    keys): both selection paths and the decode attention against the oracle."""
    case = make_case("max", [1 << 20], [1], 1, seed=209)
    a, b = _both(case)
    assert torch.equal(a["block_scores"], b["block_scores"])
    assert torch.equal(a["block_idx"], b["block_idx"])
    m = full_check(case, "decode", fused=True)
    say(f"[gpu] max context: {m}")


def test_fused_reused_buffers_see_new_scores():
    """The same block_scores / block_idx / workspace buffers across calls on
    different inputs: every call's selection must come from its own scores
    (the last workgroup reads what the others stored in this launch)."""
    kw = dict(seq_lens=[40000, 9000, 2000], rows=[1, 1, 1], n_kv_heads=2)
    cases = [make_case("reuseA", seed=210, **kw), make_case("reuseB", seed=211, **kw)]
    shape = shape_of(cases[0])
    batch = msa.Batch(cases[0].seq_lens, cases[0].rows)
    ts = [device_tensors(c) for c in cases]
    want = [gpu_run(c, "decode", t=t)["block_idx"] for c, t in zip(cases, ts)]
    assert not torch.equal(want[0], want[1])
    s = torch.empty(batch.total_rows, 2, batch.n_blocks, dtype=torch.float32, device="cuda")
    i = torch.empty(batch.total_rows, 2, cases[0].top_k, dtype=torch.int32, device="cuda")
    ws = msa.index_select_workspace(shape, batch)
    for it in range(6):
        k = it % 2
        msa.msa_index_select(shape, batch, ts[k]["iq"], ts[k]["ik"], s, i, ws)
        torch.cuda.synchronize()
        assert torch.equal(i.cpu(), want[k]), f"call {it}"


@pytest.mark.parametrize("heads", [4, 3])
def test_fused_one_row_exact_ties(heads):
    """Small-integer indexer inputs on one-row sequences: exact scores with
    mass ties at the cut (the range-maximum filter then keeps many ranges, or
    gives way to the exact search over every score); the selection must equal
    the oracle's and the two launches' bit for bit."""
    import oracle
    case = make_case("ties1", [40000, 9000, 2000], [1, 1, 1], heads, seed=217)
    gen = torch.Generator().manual_seed(7)
    case.iq = torch.randint(-1, 2, case.iq.shape, generator=gen).to(torch.bfloat16)
    case.ik = torch.randint(-1, 2, case.ik.shape, generator=gen).to(torch.bfloat16)
    a, b = _both(case)
    assert torch.equal(a["block_scores"], b["block_scores"])
    assert torch.equal(a["block_idx"], b["block_idx"])
    ref = oracle.run(case)
    assert np.array_equal(b["block_idx"].numpy(), ref["block_idx"])
