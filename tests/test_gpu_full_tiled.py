"""The benchmarked path at full size: the five named workloads through exactly
the calls the benchmark times over the tiled bf16 cache -- the step's new
keys written into the tiles (msa_pack_kv_tiled over one token range for the
prompt chunk; for decode batches and the 2,048-token prefill the write rides
in the selection's first launch, msa_index_select_pack_rows; every other key
is packed first and the row keys are left NaN until the step writes them),
the selection (msa_index_scores + msa_select_blocks for the prompt chunk) and
msa_prefill_tiled / msa_decode_tiled.

Each is checked two ways: bit for bit against the strided cache's path on
every row (block scores, selection, outputs, lse), and element by element
against the oracle on the sampled rows of the full-size parity test."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
import oracle
from gpu_helpers import check_lse, check_out, check_scores, check_selection, device_tensors, say, shape_of
from bench import SMALL_PROMPT_UNITS
from test_gpu_parity import FULL_ROWS
from workloads import config

pytestmark = pytest.mark.gpu

MODE = {"tiny": "prefill", "chunk": "prefill", "decode": "decode", "long": "decode", "windows": "decode"}


def bench_calls(case, t, batch, o, kvt):
    """The benchmark's timed calls for one workload on tensors t, writing the
    new keys into kvt and the results into o."""
    shape = shape_of(case)
    mode = MODE[case.name]
    if mode == "prefill" and case.total_rows * case.n_kv_heads > SMALL_PROMPT_UNITS:
        for k0, L, n in zip(case.kv_start, case.seq_lens, case.rows):   # one token range per sequence
            msa.msa_pack_kv_tiled(shape, t["k"], t["v"], kvt, k0 + L - n, k0 + L)
        msa.msa_index_scores(shape, batch, t["iq"], t["ik"], o["block_scores"])
        msa.msa_select_blocks(shape, batch, o["block_scores"], o["block_idx"])
        msa.msa_prefill_tiled(shape, batch, t["q"], kvt, o["block_idx"], o["out"], o["lse"])
    elif mode == "prefill":
        # a small prompt step: the new keys' write rides in the indexer's launch
        ws = msa.index_select_workspace(shape, batch)
        msa.msa_index_select_pack_rows(shape, batch, t["iq"], t["ik"], o["block_scores"], o["block_idx"],
                                       t["k"], t["v"], kvt, ws)
        msa.msa_prefill_tiled(shape, batch, t["q"], kvt, o["block_idx"], o["out"], o["lse"])
    else:
        # the new keys' write rides in the selection's launch
        ws = msa.index_select_workspace(shape, batch)
        msa.msa_index_select_pack_rows(shape, batch, t["iq"], t["ik"], o["block_scores"], o["block_idx"],
                                       t["k"], t["v"], kvt, ws)
        msa.msa_decode_tiled(shape, batch, t["q"], kvt, o["block_idx"], o["out"], o["lse"],
                             msa.decode_workspace(shape, batch.total_rows))


@pytest.mark.parametrize("name", list(MODE))
def test_benchmarked_path_full_size(name):
    case = config(name)
    assert all(k0 % 64 == 0 for k0 in case.kv_start)
    say(f"[gpu] full-size tiled path {name}: seqs={case.seq_lens} rows={case.rows}")
    t = device_tensors(case)
    shape = shape_of(case)
    batch = msa.Batch(case.seq_lens, case.rows)
    # the strided cache's path, separate launches (the reference for the bits)
    dense = msa.run_path(shape, batch, t, MODE[name])
    # the tiled cache: every key but the step's new ones packed first, the
    # rest left NaN for the step's own write
    kvt = msa.KVTiled.empty(t["k"].shape[0], case.n_kv_heads, "cuda", fill=float("nan"))
    for k0, L, n in zip(case.kv_start, case.seq_lens, case.rows):
        if L > n:
            msa.msa_pack_kv_tiled(shape, t["k"], t["v"], kvt, k0, k0 + L - n)
    got = {n: torch.full_like(x, float("nan")) if x.is_floating_point() else torch.full_like(x, -7)
           for n, x in dense.items() if n in ("block_scores", "block_idx", "out", "lse")}
    bench_calls(case, t, batch, got, kvt)
    torch.cuda.synchronize()
    dense = {n: dense[n].cpu() for n in got}
    got = {n: x.cpu() for n, x in got.items()}
    for n in ("block_scores", "block_idx", "out", "lse"):
        assert torch.equal(dense[n].view(torch.int32) if n != "out" else dense[n].view(torch.int16),
                           got[n].view(torch.int32) if n != "out" else got[n].view(torch.int16)), n
    # against the oracle on the sampled rows
    rows = FULL_ROWS[name](case)
    ref = oracle.run(case, rows)
    g = {n: x for n, x in got.items()}
    serr = check_scores(case, g, rows, ref)
    clear = check_selection(case, g, rows, ref, case.top_k)
    ok_rows = clear.all(axis=1)
    if ok_rows.any():
        check_out(got["out"][rows][ok_rows], ref["out"][ok_rows], f"{name}/tiled/e2e")
    o_own, l_own = oracle.attention(case, got["block_idx"].numpy()[rows], rows)
    mx, mean = check_out(got["out"][rows], o_own, f"{name}/tiled/own-selection")
    check_lse(got["lse"][rows], l_own, f"{name}/tiled/own-selection")
    say(f"[gpu] {name} tiled: score err {serr:.2e}, excluded {int((~clear).sum())} of {clear.size}, "
        f"max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert int((~clear).sum()) <= max(3, 0.05 * clear.size)
