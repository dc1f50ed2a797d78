"""Shared machinery of the GPU parity tests: run the HIP path through the C ABI
on a seeded case and compare it with the oracle, element by element.

Tolerances (bf16 inputs, fp32 accumulation on the GPU, double in the oracle):
  block scores  |S_gpu - S| <= 64 * 2^-24 * max|iq| * max|ik|  (norms over the
                case): the worst-case fp32 error of a 64-term dot product whose
                products are exact (bf16 x bf16 fits fp32) -- Cauchy-Schwarz
                bounds sum|iq_d ik_d| by the norms.  -inf entries must match.
  selection     bit-exact on every (row, key head) whose oracle gap between
                the last kept and first dropped non-local score is >= 1e-4;
                rows below are counted and must still hold a valid selection;
                and on every row the GPU's selection must equal the oracle's
                selection *of the GPU's own scores* (selection is integer work).
  outputs       max-abs <= 2e-2 and mean-abs <= 2e-3 against the oracle's
                double result (P is rounded to bf16 for the PV product and the
                output to bf16: relative 2^-9 each).
  lse           |lse_gpu - lse| <= 1e-3 (fp32 sums of unrounded weights).
"""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_04_amd as msa
import oracle

GAP = 1e-4
MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3


def say(*a):
    print(*a, flush=True)


def device_tensors(case, dev="cuda"):
    return {n: getattr(case, n).to(dev) for n in ("q", "k", "v", "iq", "ik")}


def shape_of(case, top_k=None):
    return msa.make_shape(case.n_kv_heads, case.top_k if top_k is None else top_k, case.scale)


def gpu_run(case, mode, t=None, batch=None, top_k=None, block_idx=None, fused=False):
    """Run the path on the GPU; block_idx (host int32) replaces the GPU's own
    selection for the attention step when given.  fused: steps 1-3 through
    msa_index_select."""
    shape = shape_of(case, top_k)
    batch = batch or msa.Batch(case.seq_lens, case.rows)
    t = t or device_tensors(case)
    out = msa.run_path(shape, batch, t, mode, fused=fused)
    if block_idx is not None:
        bi = torch.as_tensor(block_idx, dtype=torch.int32).cuda().contiguous()
        o2 = torch.empty_like(t["q"])
        l2 = torch.empty_like(out["lse"])
        if mode == "prefill":
            msa.msa_prefill(shape, batch, t["q"], t["k"], t["v"], bi, o2, l2)
        else:
            msa.msa_decode(shape, batch, t["q"], t["k"], t["v"], bi, o2, l2)
        out["out_fed"], out["lse_fed"] = o2, l2
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items() if k not in ("workspace", "select_workspace")}


def score_tol(case) -> float:
    iq = case.iq.float().norm(dim=-1).max().item()
    ik = case.ik.float().norm(dim=-1).max().item()
    return 64 * 2.0 ** -24 * iq * ik + 1e-30


def check_scores(case, g, rows, ref) -> float:
    gs = g["block_scores"].numpy()[rows].astype(np.float64)
    rs = ref["scores64"]
    assert gs.shape == rs.shape, (gs.shape, rs.shape)
    ninf_r, ninf_g = np.isneginf(rs), np.isneginf(gs)
    assert np.array_equal(ninf_r, ninf_g), "causal extent (-inf pattern) differs"
    fin = ~ninf_r
    err = float(np.max(np.abs(gs[fin] - rs[fin]))) if fin.any() else 0.0
    assert err <= score_tol(case), f"block score error {err} > bound {score_tol(case)}"
    return err


def check_selection(case, g, rows, ref, top_k) -> np.ndarray:
    """Returns a boolean [n_rows, H] mask of decisions outside the gap band."""
    gi = g["block_idx"].numpy()[rows]
    nb = ref["nb"]
    # 1. given the GPU's own scores, the selection is exact integer work
    own = oracle.select_blocks(g["block_scores"].numpy()[rows], nb, top_k)
    assert np.array_equal(gi, own), "GPU selection differs from the oracle's selection of the GPU scores"
    # 2. against the oracle's own scores, outside the gap band
    gap = oracle.selection_gap(ref["scores32"], nb, top_k)
    clear = gap >= GAP
    bad = (gi != ref["block_idx"]).any(axis=2) & clear
    assert not bad.any(), f"{int(bad.sum())} clear (row, head) selections differ"
    return clear


def check_out(got_bf16, want, label):
    got = got_bf16.float().numpy().astype(np.float64)
    d = np.abs(got - want)
    mx, mean = float(d.max()), float(d.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{label}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


def check_lse(got, want, label):
    got = got.numpy().astype(np.float64)
    both_inf = np.isneginf(got) & np.isneginf(want)
    d = np.where(both_inf, 0.0, np.abs(got - want))
    assert float(d.max()) <= LSE_ABS, f"{label}: lse error {float(d.max()):.3e}"


def full_check(case, mode, rows=None, top_k=None, t=None, fused=False):
    """Everything for one case and one attention entry point; returns metrics."""
    top_k = case.top_k if top_k is None else top_k
    rows = np.arange(case.total_rows) if rows is None else np.asarray(rows)
    say(f"[gpu] {case.name} mode={mode} fused={fused} rows={len(rows)} top_k={top_k}")
    ref = oracle.run(case, rows, top_k=top_k)
    g = gpu_run(case, mode, t=t, top_k=top_k, block_idx=_expand(case, rows, ref["block_idx"], top_k),
                fused=fused)
    serr = check_scores(case, g, rows, ref)
    clear = check_selection(case, g, rows, ref, top_k)
    # attention on the oracle's selection (independent of near-ties), all rows
    mx1, mean1 = check_out(g["out_fed"][rows], ref["out"], f"{case.name}/{mode}/fed")
    check_lse(g["lse_fed"][rows], ref["lse"], f"{case.name}/{mode}/fed")
    # end to end on rows whose every key head decided clearly
    ok_rows = clear.all(axis=1)
    mx2 = mean2 = 0.0
    if ok_rows.any():
        mx2, mean2 = check_out(g["out"][rows][ok_rows], ref["out"][ok_rows], f"{case.name}/{mode}/e2e")
    # and with the GPU's own selection, against the oracle on that selection
    gsel = g["block_idx"].numpy()[rows]
    o_own, l_own = oracle.attention(case, gsel, rows)
    check_out(g["out"][rows], o_own, f"{case.name}/{mode}/own-selection")
    check_lse(g["lse"][rows], l_own, f"{case.name}/{mode}/own-selection")
    m = dict(score_err=serr, excluded=int((~clear).sum()), units=int(clear.size),
             fed_max=mx1, fed_mean=mean1, e2e_max=mx2, e2e_mean=mean2)
    say(f"[gpu] {case.name} {mode}: {m}")
    return m


def _expand(case, rows, idx_rows, top_k):
    """Oracle selection for the chosen rows placed into a full-size array
    (other rows get their causal blocks' first top_k, a valid selection)."""
    full = np.full((case.total_rows, case.n_kv_heads, top_k), -1, dtype=np.int32)
    nb = oracle.causal_blocks(case)
    for r in range(case.total_rows):
        k = min(top_k, int(nb[r]))
        full[r, :, :k] = np.arange(int(nb[r]) - k, int(nb[r]), dtype=np.int32)
    full[np.asarray(rows)] = idx_rows
    return full


def sample_rows(case, n_random=40, seed=5):
    """Rows to compare for a large prefill case: the first and last rows of
    each sequence, both sides of every 64-row block edge in the first 300 rows,
    and a random sample."""
    rows = set()
    for s in range(case.n_seqs):
        a, b = case.cu_rows[s], case.cu_rows[s + 1]
        rows.update(range(a, min(a + 9, b)))
        rows.update(range(max(a, b - 9), b))
    rows.update(r for e in range(64, 300, 64) for r in (e - 1, e) if r < case.total_rows)
    rows.update(np.random.default_rng(seed).choice(case.total_rows, n_random, replace=False).tolist())
    return np.array(sorted(rows))
