"""Selection on hand-built scores with ties at the cut, shaped to steer every
path of the last step: candidate lists of up to 16 keys (kept by rank), of
17-64 keys (a bitwise search for the cut), whole short rows (one key per
lane), more than 64 keys at the cut (the exact fallback), the
workgroup-per-unit mode, and the one-launch selection of one-row batches.
The kept blocks must equal the oracle's selection bit for bit: ties at the cut
go to the lower blocks, which the hand-built scores make decisive."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
import oracle
from gpu_helpers import device_tensors, gpu_run, say
from workloads import make_case

pytestmark = pytest.mark.gpu

BLOCK = 64


def _causal_blocks(seq_lens, rows):
    nb = []
    for L, R in zip(seq_lens, rows):
        nb += [(L - R + i) // BLOCK + 1 for i in range(R)]
    return np.array(nb, dtype=np.int64)


def _cut_scores(rng, n, n_high, n_tie, spread=1):
    """n candidate scores: n_high distinct high ones, n_tie equal ones at the
    cut and the rest low.  The special blocks lie at distinct residues mod
    64*spread of the block index over spread, i.e. at distinct lanes of a
    per-lane maximum over keys (spread 1) or over 4-block ranges (spread 4)."""
    s = rng.integers(-250, -10, size=n).astype(np.float64)
    k = n_high + n_tie
    slots = n // spread
    residues = rng.choice(min(64, slots), size=k, replace=False)
    picks = []
    for r in residues:
        m = int(rng.integers(0, (slots - 1 - r) // 64 + 1))
        picks.append(int((r + 64 * m) * spread + rng.integers(0, spread)))
    picks = np.array(picks)
    s[picks[:n_high]] = 100 + np.arange(n_high)
    s[picks[n_high:]] = 50.0
    return s


def _unit_scores(rng, n, need, which):
    if n <= 64:
        return rng.integers(0, 4, size=n).astype(np.float64)     # many ties, one key per lane
    hi = need - 2
    return _cut_scores(rng, n, hi, (3, 10, 64 - hi)[which % 3])


@pytest.mark.parametrize("top_k", [16, 8])
@pytest.mark.parametrize("layout", ["wave", "workgroup"])
def test_select_cut_lists(top_k, layout):
    """msa_select_blocks on hand-built scores: each (row, key head) unit gets
    ties at the cut inside a candidate list of a chosen size."""
    if layout == "wave":     # one wave per unit: every sequence within 256 blocks
        seq_lens, rows = [16000, 9000, 1088, 1100, 600], [6, 5, 4, 3, 3]
    else:                    # few units over more than 256 blocks: a workgroup per unit
        seq_lens, rows = [20000, 17000], [3, 2]
    H = 3
    need = top_k - 1
    rng = np.random.default_rng(1000 + top_k + (layout == "wave"))
    nb = _causal_blocks(seq_lens, rows)
    batch = msa.Batch(seq_lens, rows)
    stride = batch.n_blocks
    scores = np.full((len(nb), H, stride), -np.inf, dtype=np.float32)
    which = 0
    for r in range(len(nb)):
        for g in range(H):
            n = int(nb[r]) - 1
            if n > 0:
                scores[r, g, :n] = _unit_scores(rng, n, need, which)
                which += 1
            scores[r, g, n] = 0.0     # the local block (always kept)
    idx = torch.empty(len(nb), H, top_k, dtype=torch.int32, device="cuda")
    msa.msa_select_blocks(msa.make_shape(H, top_k), batch, torch.from_numpy(scores).cuda(), idx)
    torch.cuda.synchronize()
    want = oracle.select_blocks(scores, nb, top_k)
    got = idx.cpu().numpy()
    bad = np.argwhere((got != want).any(axis=2))
    say(f"{layout} top_k {top_k}: {len(nb) * H} units, {len(bad)} differ")
    assert len(bad) == 0, (bad[:4], got[tuple(bad[0])], want[tuple(bad[0])])


def _fused_case(heads):
    """One-row sequences whose block scores are exact integers chosen per
    (sequence, key head): index queries one-hot on dimension 0, index keys
    equal to their block's score on dimension 0 (integers, exact in bf16)."""
    seq_lens = [40000, 9000, 2000]
    case = make_case("cut_lists", seq_lens, [1, 1, 1], heads, seed=219)
    rng = np.random.default_rng(23 + heads)
    iq = torch.zeros_like(case.iq)
    iq[:, :, 0] = 1.0
    ik = torch.zeros(case.ik.shape, dtype=torch.float32)
    need = case.top_k - 1
    hi = need - 2
    for s, L in enumerate(seq_lens):
        n = (L - 1) // BLOCK          # candidate blocks of the row (its local block is block n)
        k0 = case.kv_start[s]
        for g in range(heads):
            if s == 0:
                # ranges of 4 blocks: 16 listed keys (ranks), 23 (bitwise), 64
                # candidate ranges, then 60 ties two to a range (more than 64
                # keys at the cut: the exact fallback)
                if g < 3:
                    blk = _cut_scores(rng, n, hi, (3, 10, 64 - hi)[g], spread=4)
                else:
                    blk = _cut_scores(rng, n, hi, 30, spread=4)
                    ties = np.flatnonzero(blk == 50.0)
                    blk[np.minimum(ties ^ 1, n - 1)] = 50.0
            elif s == 1:
                blk = _cut_scores(rng, n, hi, 3, spread=4)
            else:
                blk = rng.integers(0, 4, size=n).astype(np.float64)
            vals = np.concatenate([np.repeat(blk, BLOCK), np.zeros(L - n * BLOCK)])[:L]
            ik[k0:k0 + L, g, 0] = torch.from_numpy(vals).float()
    case.iq = iq
    case.ik = ik.to(torch.bfloat16)
    return case


@pytest.mark.parametrize("heads", [4, 3])
def test_fused_one_row_cut_lists(heads):
    """msa_index_select's one-launch path on one-row sequences with exact
    integer block scores and ties at the cut in lists of 16, 23 and 64 keys and
    beyond 64: equal to the two launches and to the oracle, bit for bit."""
    case = _fused_case(heads)
    t = device_tensors(case)
    a = gpu_run(case, "decode", t=t)
    b = gpu_run(case, "decode", t=t, fused=True)
    assert torch.equal(a["block_scores"], b["block_scores"])
    assert torch.equal(a["block_idx"], b["block_idx"])
    ref = oracle.run(case)
    assert np.array_equal(b["block_scores"].numpy().astype(np.float64), ref["scores64"])
    assert np.array_equal(b["block_idx"].numpy(), ref["block_idx"])
