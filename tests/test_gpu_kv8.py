"""GPU parity of the int8 key/value cache: msa_quantize_kv8 against the
oracle's quantisation (bit-exact codes and scales: both decide the codes in
fp32 with IEEE division and round-half-even), and msa_prefill_kv8 /
msa_decode_kv8 against the oracle's attention over code * scale."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
import oracle
from gpu_helpers import check_lse, check_out, device_tensors, sample_rows, say, shape_of, _expand
from workloads import make_case, to_pages

pytestmark = pytest.mark.gpu


def quantize_gpu(case, x):
    codes, scales = msa.msa_quantize_kv8(shape_of(case), x.cuda())
    torch.cuda.synchronize()
    return codes, scales


def test_quantize_matches_oracle():
    g = torch.Generator().manual_seed(401)
    x = torch.randn(3000, 4, 128, generator=g) * torch.exp(torch.randn(3000, 4, 1, generator=g) * 4)
    x[17, 2] = 0.0
    x[18, 0, 5] = 1e30          # one huge element
    x = x.to(torch.bfloat16)
    case = make_case("q", [3000], [1], 4, seed=401)
    codes, scales = quantize_gpu(case, x)
    rc, rs = oracle.quantize_kv8(x)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def kv8_of(case):
    kc, ks = quantize_gpu(case, case.k)
    vc, vs = quantize_gpu(case, case.v)
    return msa.KV8(kc, vc, ks, vs), (kc.cpu().numpy(), vc.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy())


def run(case, mode, kv8, t=None, batch=None, fused=False):
    t = t or device_tensors(case)
    out = msa.run_path(shape_of(case), batch or msa.Batch(case.seq_lens, case.rows), t, mode, kv8=kv8,
                       fused=fused)
    torch.cuda.synchronize()
    return {n: x.cpu() for n, x in out.items() if n not in ("workspace", "select_workspace")}


CASES = {
    "tiled": (dict(seq_lens=[700, 1500, 300, 64], rows=[300, 5, 300, 64], n_kv_heads=2, seed=411), 16),
    "window": (dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[16, 1, 16, 7, 3], n_kv_heads=3, seed=412), 16),
    "top32": (dict(seq_lens=[4000, 2100], rows=[30, 2], n_kv_heads=2, seed=413, top_k=32), 32),
}


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("name", list(CASES))
def test_kv8_attention_against_oracle(name, mode):
    kw, top_k = CASES[name]
    case = make_case(name, **kw)
    kv8, (kc, vc, ks, vs) = kv8_of(case)
    g = run(case, mode, kv8)
    rows = np.arange(case.total_rows)
    # the GPU's own selection, attended by the oracle over the same int8 cache
    own_out, own_lse = oracle.attention_kv8(case, kc, vc, ks, vs, g["block_idx"].numpy(), rows)
    m1 = check_out(g["out"], own_out, f"kv8/{name}/{mode}/own-selection")
    check_lse(g["lse"], own_lse, f"kv8/{name}/{mode}/own-selection")
    # the oracle's selection fed to the int8 attention entry point
    ref = oracle.run(case, rows, top_k=top_k)
    bi = torch.as_tensor(_expand(case, rows, ref["block_idx"], top_k)).cuda()
    t = device_tensors(case)
    o2 = torch.empty_like(t["q"])
    l2 = torch.empty(case.total_rows, case.n_kv_heads * 16, dtype=torch.float32, device="cuda")
    batch = msa.Batch(case.seq_lens, case.rows)
    if mode == "prefill":
        msa.msa_prefill_kv8(shape_of(case), batch, t["q"], kv8, bi, o2, l2)
    else:
        msa.msa_decode_kv8(shape_of(case), batch, t["q"], kv8, bi, o2, l2)
    torch.cuda.synchronize()
    fed_out, fed_lse = oracle.attention_kv8(case, kc, vc, ks, vs, ref["block_idx"], rows)
    m2 = check_out(o2.cpu(), fed_out, f"kv8/{name}/{mode}/fed")
    check_lse(l2.cpu(), fed_lse, f"kv8/{name}/{mode}/fed")
    say(f"[gpu] kv8 {name} {mode}: own {m1} fed {m2}")


@pytest.mark.parametrize("name", ["walk4", "walk2_top32"])
def test_kv8_prefill_rows_per_wave(name):
    """The int8 prefill on batches large enough for 4 (or, at top_k = 32, 2)
    rows per wave, against the oracle over the same int8 cache on sampled
    rows (sequence starts and ends, block edges, random)."""
    kw = {"walk4": dict(seq_lens=[2600, 700], rows=[2000, 100], n_kv_heads=4, seed=416),
          "walk2_top32": dict(seq_lens=[2600, 2400], rows=[2000, 100], n_kv_heads=2, seed=417, top_k=32)}[name]
    case = make_case(name, **kw)
    kv8, (kc, vc, ks, vs) = kv8_of(case)
    g = run(case, "prefill", kv8)
    rows = sample_rows(case)
    own_out, own_lse = oracle.attention_kv8(case, kc, vc, ks, vs, g["block_idx"].numpy()[rows], rows)
    m = check_out(g["out"][rows], own_out, f"kv8/{name}/own-selection")
    check_lse(g["lse"][rows], own_lse, f"kv8/{name}/own-selection")
    say(f"[gpu] kv8 {name}: {m}")


def test_kv8_prefill_and_decode_agree():
    case = make_case("kv8x", [3000, 700], [16, 9], 2, seed=414)
    kv8, _ = kv8_of(case)
    a = run(case, "prefill", kv8)
    b = run(case, "decode", kv8)
    assert torch.equal(a["block_idx"], b["block_idx"])
    d = (a["out"].float() - b["out"].float()).abs()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


def test_kv8_paged_equals_contiguous():
    case = make_case("kv8p", [6000, 2500, 130], [24, 16, 3], 2, seed=415)
    kv8, (kc, vc, ks, vs) = kv8_of(case)
    dense = {m: run(case, m, kv8) for m in ("prefill", "decode")}
    # the same codes and scales scattered into 64-token pages
    pool, pt = to_pages(case, seed=415, extra_pages=3)
    n_tok = pool["k"].shape[0]
    pk = torch.zeros(n_tok, 2, 128, dtype=torch.int8)
    pv = torch.zeros_like(pk)
    pks = torch.zeros(n_tok, 2, dtype=torch.float32)
    pvs = torch.zeros_like(pks)
    for s, L in enumerate(case.seq_lens):
        for j0 in range(0, L, 64):
            n = min(64, L - j0)
            dst = slice(int(pt[s, j0 // 64]) * 64, int(pt[s, j0 // 64]) * 64 + n)
            src = slice(case.kv_start[s] + j0, case.kv_start[s] + j0 + n)
            pk[dst], pv[dst] = torch.from_numpy(kc[src]), torch.from_numpy(vc[src])
            pks[dst], pvs[dst] = torch.from_numpy(ks[src]), torch.from_numpy(vs[src])
    kv8p = msa.KV8(pk.cuda(), pv.cuda(), pks.cuda(), pvs.cuda())
    t = dict(device_tensors(case), **{n: x.cuda() for n, x in pool.items()})
    batch = msa.Batch(case.seq_lens, case.rows, page_table=pt)
    for m in ("prefill", "decode"):
        paged = run(case, m, kv8p, t=t, batch=batch)
        for n in ("block_idx", "out", "lse"):
            assert torch.equal(dense[m][n], paged[n]), (m, n)
