"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on seeded inputs; plus the invariants the method implies (batch,
window/one-row and rerun bit-identity) and edge cases."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
import oracle
from gpu_helpers import check_lse, check_out, device_tensors, full_check, gpu_run, sample_rows, say, shape_of
from workloads import Case, config, make_case

pytestmark = pytest.mark.gpu

SMALL = {
    # > 16 rows: the LDS-tiled indexer; 300 rows span two 256-row tiles
    "ragged_tiled": dict(seq_lens=[700, 1500, 300, 64], rows=[300, 5, 300, 64], n_kv_heads=2, seed=101),
    # <= 16 rows per sequence: the streaming indexer; includes a 1-key sequence
    "ragged_window": dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[16, 1, 16, 7, 3], n_kv_heads=3, seed=102),
    # the same with key heads in fours: a workgroup scores 4 heads of one key range
    "ragged_window_h4": dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[16, 1, 16, 7, 3], n_kv_heads=4, seed=108),
    "ragged_window_h8": dict(seq_lens=[2000, 257, 1100], rows=[9, 16, 2], n_kv_heads=8, seed=109),
    # one index key shared by the key heads (head stride 0)
    "shared_ik": dict(seq_lens=[2000, 900], rows=[40, 8], n_kv_heads=4, seed=103, ik_shared=True),
    # indexer inputs scaled by 1/8 (exact), as in the tiny configuration
    "scaled_index": dict(seq_lens=[3000], rows=[100], n_kv_heads=1, seed=104, index_scale=0.125),
    "top1": dict(seq_lens=[1200, 800], rows=[20, 3], n_kv_heads=2, seed=105, top_k=1),
    "top5": dict(seq_lens=[1200, 800], rows=[20, 3], n_kv_heads=2, seed=106, top_k=5),
    "top32": dict(seq_lens=[4000, 2100], rows=[30, 2], n_kv_heads=2, seed=107, top_k=32),
}


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(name, mode):
    kw = dict(SMALL[name])
    case = make_case(name, **kw)
    full_check(case, mode)


FULL_ROWS = {
    "tiny": lambda c: np.unique(np.r_[0, 1, 63, 64, 1023, 1024, 1025, 2047,
                                      np.random.default_rng(1).choice(2048, 120, replace=False)]),
    "decode": lambda c: np.arange(c.total_rows),
    "chunk": lambda c: np.unique(np.r_[0, 1, 63, 64, 255, 256, 257, 1000, 2047, 2048, 4032, 4095,
                                       np.random.default_rng(2).choice(4096, 20, replace=False)]),
    "long": lambda c: np.arange(c.total_rows),
    "windows": lambda c: np.arange(c.total_rows),
}
FULL_MODE = {"tiny": "prefill", "decode": "decode", "chunk": "prefill", "long": "decode",
             "windows": "decode"}


@pytest.mark.parametrize("name", list(FULL_ROWS))
def test_full_configs(name):
    """The five named workloads at full size, through the entry point the
    benchmark uses for them; outputs compared on sampled rows."""
    case = config(name)
    m = full_check(case, FULL_MODE[name], rows=FULL_ROWS[name](case))
    if name == "windows":
        # the planted needle blocks are kept by every row and key head
        g = gpu_run(case, "decode")
        idx = g["block_idx"].numpy()
        for s in range(case.n_seqs):
            for r in range(case.cu_rows[s], case.cu_rows[s + 1]):
                for h in range(case.n_kv_heads):
                    assert set(case.needles[s]) <= set(idx[r, h].tolist())
    assert m["excluded"] <= max(3, 0.05 * m["units"])


def test_prefill_and_decode_agree():
    case = make_case("cross", [3000, 700], [16, 9], 2, seed=111)
    a = gpu_run(case, "prefill")
    b = gpu_run(case, "decode")
    assert np.array_equal(a["block_idx"].numpy(), b["block_idx"].numpy())
    d = (a["out"].float() - b["out"].float()).abs()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_reruns_are_bit_identical(mode):
    case = make_case("rerun", [5000, 2000], [64, 16], 2, seed=112)
    t = device_tensors(case)
    runs = [gpu_run(case, mode, t=t) for _ in range(3)]
    for r in runs[1:]:
        for k in ("block_scores", "block_idx", "out", "lse"):
            assert torch.equal(r[k], runs[0][k]), k


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_batch_invariance(mode):
    """A sequence alone gives the same bits as inside a ragged batch."""
    big = make_case("batch", [3000, 1700, 900], [20, 16, 5], 2, seed=113)
    g = gpu_run(big, mode)
    k0, L, r0, n = big.kv_start[1], big.seq_lens[1], big.cu_rows[1], big.rows[1]
    solo = Case(name="solo", seq_lens=[L], rows=[n], n_kv_heads=2, q=big.q[r0:r0 + n],
                k=big.k[k0:k0 + L], v=big.v[k0:k0 + L], iq=big.iq[r0:r0 + n], ik=big.ik[k0:k0 + L])
    s = gpu_run(solo, mode)
    nbk = s["block_scores"].shape[2]
    assert torch.equal(g["block_scores"][r0:r0 + n, :, :nbk], s["block_scores"])
    assert torch.equal(g["block_idx"][r0:r0 + n], s["block_idx"])
    assert torch.equal(g["out"][r0:r0 + n], s["out"])


def test_window_equals_one_row_steps():
    """A 16-row verify window through msa_decode gives, row by row, the same
    bits as 16 one-row decode steps on the growing cache."""
    L, n = 9000, 16
    win = make_case("win", [L], [n], 2, seed=114)
    gw = gpu_run(win, "decode")
    for i in range(n):
        p = L - n + i
        step = Case(name="step", seq_lens=[p + 1], rows=[1], n_kv_heads=2, q=win.q[i:i + 1],
                    k=win.k[:p + 1], v=win.v[:p + 1], iq=win.iq[i:i + 1], ik=win.ik[:p + 1])
        gs = gpu_run(step, "decode")
        assert torch.equal(gw["block_idx"][i], gs["block_idx"][0])
        assert torch.equal(gw["out"][i], gs["out"][0])
        nbk = gs["block_scores"].shape[2]
        assert torch.equal(gw["block_scores"][i, :, :nbk], gs["block_scores"][0])


def test_equal_scores_take_lowest_blocks():
    """All-zero indexer queries: every block scores 0, so the selection is the
    15 lowest blocks plus the local one (ties go to the lower index); this also
    drives the selection's many-ties path."""
    case = make_case("zeros", [8000, 3000], [17, 2], 2, seed=115)
    case.iq = torch.zeros_like(case.iq)
    g = gpu_run(case, "prefill")
    nb = oracle.causal_blocks(case)
    idx = g["block_idx"].numpy()
    for r in range(case.total_rows):
        want = list(range(15)) + [int(nb[r]) - 1]
        for h in range(2):
            assert list(idx[r, h]) == want
    full_check(case, "decode")


def test_integer_ties_exact():
    """Small-integer indexer inputs give exact scores on both sides, with many
    exact ties at the cut: the selection must match bit for bit everywhere."""
    case = make_case("ties", [6000, 2500], [24, 4], 2, seed=116)
    gen = torch.Generator().manual_seed(5)
    case.iq = torch.randint(-2, 3, case.iq.shape, generator=gen).to(torch.bfloat16)
    case.ik = torch.randint(-2, 3, case.ik.shape, generator=gen).to(torch.bfloat16)
    g = gpu_run(case, "decode")
    ref = oracle.run(case)
    assert np.array_equal(g["block_scores"].numpy().astype(np.float64), ref["scores64"])
    assert np.array_equal(g["block_idx"].numpy(), ref["block_idx"])


def test_constant_values_and_zero_keys():
    case = make_case("const", [2500], [33], 2, seed=117)
    case.v = torch.full_like(case.v, 0.75)
    for mode in ("prefill", "decode"):
        g = gpu_run(case, mode)
        assert torch.all(g["out"].float() == 0.75)
    case = make_case("zk", [2500], [33], 2, seed=118)
    case.k = torch.zeros_like(case.k)
    full_check(case, "prefill")


def test_empty_batch_is_noop():
    case = make_case("e", [100], [1], 1, seed=119)
    shape = shape_of(case)
    b = msa.Batch([], [])
    t = device_tensors(case)
    s = torch.full((1, 1, 2), 7.0, device="cuda")
    msa.msa_index_scores(shape, b, t["iq"], t["ik"], s)
    torch.cuda.synchronize()
    assert torch.all(s == 7.0)


def test_strided_kv_views():
    """k/v as views into a wider [tokens, heads, 2*128] buffer (token stride
    != heads*128) give the same result as contiguous copies."""
    case = make_case("strided", [2000], [20], 2, seed=120)
    t = device_tensors(case)
    wide_k = torch.zeros(case.total_keys, 2, 256, dtype=torch.bfloat16, device="cuda")
    wide_v = torch.zeros_like(wide_k)
    wide_k[:, :, 64:192] = t["k"]
    wide_v[:, :, 64:192] = t["v"]
    t2 = dict(t, k=wide_k[:, :, 64:192], v=wide_v[:, :, 64:192])
    for mode in ("prefill", "decode"):
        a = gpu_run(case, mode, t=t)
        b = gpu_run(case, mode, t=t2)
        assert torch.equal(a["out"], b["out"])


@pytest.mark.parametrize("top_k", [1, 2, 16, 32])
def test_selection_workgroup_mode(top_k):
    """Few (row, key head) units with more than 256 blocks: a workgroup takes
    one unit, selects per quarter and merges; the result must be the oracle's."""
    case = make_case("wgsel", [20000, 17000], [3, 2], 2, seed=130 + top_k, top_k=top_k)
    full_check(case, "decode", top_k=top_k)
    # all scores equal: the lowest top_k-1 blocks plus the local one
    case.iq = torch.zeros_like(case.iq)
    g = gpu_run(case, "decode", top_k=top_k)
    nb = oracle.causal_blocks(case)
    for r in range(case.total_rows):
        want = list(range(top_k - 1)) + [int(nb[r]) - 1]
        for h in range(2):
            assert list(g["block_idx"].numpy()[r, h]) == want


def test_decode_workspace_reuse():
    """One workspace across several msa_decode calls: the arrival counters
    return to zero after every call, so repeated calls give the same bits."""
    case = make_case("wsreuse", [9000, 3000], [5, 3], 2, seed=140)
    shape = shape_of(case)
    batch = msa.Batch(case.seq_lens, case.rows)
    t = device_tensors(case)
    first = msa.run_path(shape, batch, t, "prefill")          # block_idx from the path
    ws = msa.decode_workspace(shape, batch.total_rows)
    outs = []
    for _ in range(3):
        o = torch.empty_like(t["q"])
        msa.msa_decode(shape, batch, t["q"], t["k"], t["v"], first["block_idx"], o, workspace=ws)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    units = batch.total_rows * case.n_kv_heads
    assert int(ws[:units * 4].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.gpu
def test_correlated_rows_share_blocks():
    """Rows whose indexer queries are AR(1)-correlated keep mostly the same
    blocks, so the four rows of a walk share many entries (the secondary
    workload): the merged walk must still give every row exactly its own
    blocks' result.  2,100 rows x 4 key heads: enough waves for four rows per
    wave."""
    case = make_case("locality", [9000, 5000], [2000, 100], 4, seed=131, locality=0.95)
    ref_idx = oracle.run(case, np.arange(300))["block_idx"]
    shared = np.mean([len(set(ref_idx[r, 0]) & set(ref_idx[r + 1, 0])) for r in range(299)])
    say(f"[gpu] locality: neighbouring rows share {shared:.1f} of 16 blocks")
    assert shared >= 8
    full_check(case, "prefill", rows=sample_rows(case))
    full_check(case, "decode", rows=np.arange(0, case.total_rows, 37))


# Prefill cases large enough for the launch to put 4 (or 2) rows in each wave;
# smaller batches take one row per wave.
WALK = {
    "walk4": dict(seq_lens=[2600, 700], rows=[2000, 100], n_kv_heads=4, seed=150),
    "walk2": dict(seq_lens=[2600, 700], rows=[2000, 100], n_kv_heads=2, seed=151),
    "walk2_top32": dict(seq_lens=[2600, 2400], rows=[2000, 100], n_kv_heads=2, seed=152, top_k=32),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(WALK))
def test_prefill_rows_per_wave(name):
    """The merged multi-row walk (4 rows per wave, or 2 for top_k = 32 or on
    fewer waves) against the oracle on rows at sequence starts and ends, block
    edges and at random; and bit-identical to the one-row walk of the same rows
    run as a batch too small to group rows."""
    case = make_case(name, **WALK[name])
    full_check(case, "prefill", rows=sample_rows(case))
    # the same rows of sequence 1 on their own (100 rows: one row per wave)
    t = device_tensors(case)
    shape = shape_of(case)
    big = msa.Batch(case.seq_lens, case.rows)
    o_big = msa.run_path(shape, big, t, "prefill")
    r1 = case.cu_rows[1]
    n1 = case.rows[1]
    L1 = case.seq_lens[1]
    k0 = case.kv_start[1]
    small = msa.Batch([L1], [n1])
    sub = {"q": t["q"][r1:r1 + n1].contiguous(), "k": t["k"][k0:k0 + L1].contiguous(),
           "v": t["v"][k0:k0 + L1].contiguous(), "iq": t["iq"][r1:r1 + n1].contiguous(),
           "ik": t["ik"][k0:k0 + L1].contiguous()}
    o_small = msa.run_path(shape, small, sub, "prefill")
    torch.cuda.synchronize()
    assert torch.equal(o_big["block_idx"][r1:r1 + n1], o_small["block_idx"])
    assert torch.equal(o_big["out"][r1:r1 + n1], o_small["out"])
    assert torch.equal(o_big["lse"][r1:r1 + n1], o_small["lse"])


@pytest.mark.gpu
@pytest.mark.parametrize("top_k", [1, 5, 16, 32])
def test_decode_kernels_agree(top_k):
    """128 (row, key head) units take the one-workgroup-per-unit decode; each
    sequence alone (32 units) the split over workgroups.  Both must give the
    same bits, and the large batch must pass the oracle checks."""
    case = make_case(f"dk{top_k}", [9000, 5000, 3000, 700], [8, 8, 8, 8], 4, seed=160 + top_k, top_k=top_k)
    full_check(case, "decode")
    t = device_tensors(case)
    shape = shape_of(case)
    big = msa.run_path(shape, msa.Batch(case.seq_lens, case.rows), t, "decode")
    for s in range(case.n_seqs):
        r0, r1 = case.cu_rows[s], case.cu_rows[s + 1]
        k0, L = case.kv_start[s], case.seq_lens[s]
        sub = {"q": t["q"][r0:r1].contiguous(), "iq": t["iq"][r0:r1].contiguous(),
               "k": t["k"][k0:k0 + L].contiguous(), "v": t["v"][k0:k0 + L].contiguous(),
               "ik": t["ik"][k0:k0 + L].contiguous()}
        one = msa.run_path(shape, msa.Batch([L], [r1 - r0]), sub, "decode")
        torch.cuda.synchronize()
        assert torch.equal(big["block_idx"][r0:r1], one["block_idx"]), s
        assert torch.equal(big["out"][r0:r1], one["out"]), s
        assert torch.equal(big["lse"][r0:r1], one["lse"]), s


# Batches whose rows the prefill groups into waves per 64-row window of each
# key head: i.i.d. rows (ranked by their mean kept block and paired from both
# ends), correlated rows (kept consecutive), ragged batches whose last window
# holds an odd number of rows, and 4 or 2 rows per wave.
GROUPING = {
    "iid_w4_ragged": dict(seq_lens=[3000, 700, 65, 1900], rows=[1601, 37, 1, 464], n_kv_heads=4, seed=171),
    "iid_w2_ragged": dict(seq_lens=[3000, 900], rows=[1999, 102], n_kv_heads=2, seed=172),
    "correlated_w4": dict(seq_lens=[5000], rows=[2100], n_kv_heads=4, seed=173, locality=0.95),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(GROUPING))
def test_prefill_row_grouping(name):
    """Every row of the batch is computed exactly once, by whichever wave its
    window's grouping gives it: outputs start as NaN and must all be written,
    equal the oracle on the GPU's own selection on every row, and be
    bit-identical between the strided and the tiled cache."""
    from test_gpu_tiled import aligned_copy
    case = make_case(name, **GROUPING[name])
    R, H = case.total_rows, case.n_kv_heads
    say(f"[gpu] row grouping {name}: seqs={case.seq_lens} rows={case.rows} heads={H}")
    t = device_tensors(case)
    shape = shape_of(case)
    batch = msa.Batch(case.seq_lens, case.rows)
    sel = msa.run_path(shape, batch, t, "prefill")["block_idx"]
    nan_out = lambda: (torch.full_like(t["q"], float("nan")),
                       torch.full((R, H * 16), float("nan"), device="cuda"))
    o_s, l_s = nan_out()
    msa.msa_prefill(shape, batch, t["q"], t["k"], t["v"], sel, o_s, l_s)
    t2, starts = aligned_copy(case, t)
    kvt = msa.KVTiled.empty(t2["k"].shape[0], H, "cuda", fill=float("nan"))
    msa.msa_pack_kv_tiled(shape, t2["k"], t2["v"], kvt)
    o_t, l_t = nan_out()
    msa.msa_prefill_tiled(shape, msa.Batch(case.seq_lens, case.rows, kv_start=starts), t["q"], kvt, sel, o_t, l_t)
    torch.cuda.synchronize()
    assert not torch.isnan(o_s.float()).any() and not torch.isnan(l_s).any(), "a row was never written"
    assert torch.equal(o_t.view(torch.int16), o_s.view(torch.int16))
    assert torch.equal(l_t.view(torch.int32), l_s.view(torch.int32))
    o_ref, l_ref = oracle.attention(case, sel.cpu().numpy())
    check_out(o_s.cpu(), o_ref, f"{name}/all rows")
    check_lse(l_s.cpu(), l_ref, f"{name}/all rows")


@pytest.mark.gpu
def test_decode_unit_order_ragged():
    """100 (row, key head) units (not a multiple of the 8 XCDs) take the
    one-workgroup-per-unit decode, whose workgroups pick units in an
    XCD-aware order: every unit must be computed once and equal the same
    rows run a sequence at a time (the split kernel), bit for bit, and pass
    the oracle checks."""
    case = make_case("dk_ragged", [9000, 5000, 700], [9, 9, 7], 4, seed=190)
    assert case.total_rows * case.n_kv_heads == 100
    full_check(case, "decode")
    t = device_tensors(case)
    shape = shape_of(case)
    big = msa.run_path(shape, msa.Batch(case.seq_lens, case.rows), t, "decode")
    for s in range(case.n_seqs):
        r0, r1 = case.cu_rows[s], case.cu_rows[s + 1]
        k0, L = case.kv_start[s], case.seq_lens[s]
        sub = {"q": t["q"][r0:r1].contiguous(), "iq": t["iq"][r0:r1].contiguous(),
               "k": t["k"][k0:k0 + L].contiguous(), "v": t["v"][k0:k0 + L].contiguous(),
               "ik": t["ik"][k0:k0 + L].contiguous()}
        one = msa.run_path(shape, msa.Batch([L], [r1 - r0]), sub, "decode")
        torch.cuda.synchronize()
        assert torch.equal(big["block_idx"][r0:r1], one["block_idx"]), s
        assert torch.equal(big["out"][r0:r1], one["out"]), s
        assert torch.equal(big["lse"][r0:r1], one["lse"]), s
