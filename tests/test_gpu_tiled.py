"""GPU parity of the tiled bf16 cache (include/msa.h, msa_kv_tiled): the pack
entry point writes exactly the layout the header defines (checked against a
numpy construction of that definition), and attention over the tiles gives
bit for bit what the strided cache gives -- the kernels read the same
operands, only their addresses differ -- and passes the oracle's check on
its own selection.  Keys no row can see are left NaN in the tiles."""
import numpy as np
import pytest
import torch

import block_sparse_attention_04_amd as msa
import oracle
from gpu_helpers import check_lse, check_out, device_tensors, say, shape_of
from workloads import make_case, to_pages

pytestmark = pytest.mark.gpu
NAN16 = 0x7FC0   # a bf16 quiet NaN


def tiles_reference(k, v, t0, t1, kt, vt):
    """Write tokens t0 .. t1-1 of k, v (uint16 [T, H, 128]) into kt, vt
    (uint16 [blocks, H, 8192]) by the layout's definition, one key at a time."""
    for t in range(t0, t1):
        b, j = divmod(t, 64)
        c, jj = divmod(j, 32)
        base = 4096 * c
        mt, lr = divmod(jj, 16)             # K: key 16*mt + l%16, dims 32*s + 8*(l/16) + 0..7
        for s in range(4):
            for lg in range(4):
                q = 256 * mt + 64 * s + 16 * lg + lr
                kt[b, :, base + 8 * q: base + 8 * q + 8] = k[t, :, 32 * s + 8 * lg: 32 * s + 8 * lg + 8]
        half, r = divmod(jj, 16)            # V: element 4*half + i of lane group lg holds key 16*half + 4*lg + i
        lg, i = divmod(r, 4)
        for dt in range(8):
            for lr2 in range(16):
                q = 64 * dt + 16 * lg + lr2
                vt[b, :, base + 8 * q + 4 * half + i] = v[t, :, 16 * dt + lr2]


def u16(x):
    return x.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("ranges", [[(0, 300)], [(0, 37), (37, 201), (201, 300)], [(70, 71), (130, 250)]])
def test_pack_writes_the_defined_layout(ranges):
    T, H = 300, 2
    g = torch.Generator().manual_seed(7)
    k = torch.randn(T, H, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(T, H, 128, generator=g).to(torch.bfloat16)
    kvt = msa.KVTiled.empty(T, H, "cuda", fill=float("nan"))
    shape = msa.make_shape(H)
    for t0, t1 in ranges:
        msa.msa_pack_kv_tiled(shape, k.cuda(), v.cuda(), kvt, t0, t1)
    torch.cuda.synchronize()
    nb = (T + 63) // 64
    kt = np.full((nb, H, 8192), NAN16, np.uint16)
    vt = np.full((nb, H, 8192), NAN16, np.uint16)
    for t0, t1 in ranges:
        tiles_reference(u16(k), u16(v), t0, t1, kt, vt)
    assert np.array_equal(u16(kvt.k), kt)
    assert np.array_equal(u16(kvt.v), vt)


def aligned_copy(case, t):
    """The case's k, v, ik with every sequence starting on a 64-token
    boundary (the tiled cache's contiguous-layout precondition); the gaps are
    NaN.  Returns (tensors, kv_start)."""
    starts, pos = [], 0
    for L in case.seq_lens:
        starts.append(pos)
        pos += (L + 63) // 64 * 64
    T2 = max(pos, 64)
    out = dict(t)
    for n in ("k", "v", "ik"):
        x = t[n]
        y = torch.full((T2,) + tuple(x.shape[1:]), float("nan"), dtype=x.dtype, device=x.device)
        src = 0
        for s0, L in zip(starts, case.seq_lens):
            y[s0:s0 + L] = x[src:src + L]
            src += L
        out[n] = y
    return out, starts


def run(case, t, batch, mode, kvt=None, fused=False):
    o = msa.run_path(shape_of(case), batch, t, mode, kvt=kvt, fused=fused)
    torch.cuda.synchronize()
    return {n: x.cpu() for n, x in o.items() if n not in ("workspace", "select_workspace")}


CASES = {
    # four-row walks (2,000-row sequence) and the two-row walk (top_k 32)
    "walk4": dict(seq_lens=[2600, 700], rows=[2000, 100], n_kv_heads=4, seed=501),
    "walk2_top32": dict(seq_lens=[2600, 2400], rows=[2000, 100], n_kv_heads=2, seed=502, top_k=32),
    # ragged sequences, a 1-key sequence, partial last blocks
    "ragged": dict(seq_lens=[700, 1500, 300, 64, 1], rows=[300, 5, 300, 64, 1], n_kv_heads=2, seed=503),
    # <= 16 rows: one-workgroup-per-unit decode (>= 80 units)
    "window": dict(seq_lens=[5000, 1, 64, 65, 3000], rows=[16, 1, 16, 7, 3], n_kv_heads=3, seed=504),
    # one-row steps: the split decode
    "one_row": dict(seq_lens=[40000, 7000, 300], rows=[1, 1, 1], n_kv_heads=2, seed=505),
    "top1": dict(seq_lens=[1200, 800], rows=[20, 3], n_kv_heads=2, seed=506, top_k=1),
    "top5": dict(seq_lens=[1200, 800], rows=[20, 3], n_kv_heads=2, seed=507, top_k=5),
}


@pytest.mark.parametrize("mode", ["prefill", "decode"])
@pytest.mark.parametrize("name", list(CASES))
def test_tiled_equals_strided(name, mode):
    case = make_case(name, **CASES[name])
    say(f"[gpu] tiled {name} {mode}")
    dense = run(case, device_tensors(case), msa.Batch(case.seq_lens, case.rows), mode)
    t2, starts = aligned_copy(case, device_tensors(case))
    shape = shape_of(case)
    kvt = msa.KVTiled.empty(t2["k"].shape[0], case.n_kv_heads, "cuda", fill=float("nan"))
    # the cache written a sequence at a time, as a server would write it
    for s0, L in zip(starts, case.seq_lens):
        msa.msa_pack_kv_tiled(shape, t2["k"], t2["v"], kvt, s0, s0 + L)
    batch = msa.Batch(case.seq_lens, case.rows, kv_start=starts)
    got = run(case, t2, batch, mode, kvt=kvt)
    for n in ("block_idx", "out", "lse"):
        assert torch.equal(dense[n], got[n]), n
    # and against the oracle on the GPU's own selection
    rows = np.arange(case.total_rows)
    o_ref, l_ref = oracle.attention(case, got["block_idx"].numpy(), rows)
    check_out(got["out"], o_ref, f"tiled/{name}/{mode}")
    check_lse(got["lse"], l_ref, f"tiled/{name}/{mode}")


@pytest.mark.parametrize("name", ["walk4", "window"])
def test_tiled_paged(name):
    """Pages of 64 tokens are tiles: a page table indexes the tiles directly."""
    case = make_case(name, **CASES[name])
    mode = "prefill" if name == "walk4" else "decode"
    dense = run(case, device_tensors(case), msa.Batch(case.seq_lens, case.rows), mode)
    pool, pt = to_pages(case, seed=11, extra_pages=3)
    t = dict(device_tensors(case), **{n: x.cuda() for n, x in pool.items()})
    shape = shape_of(case)
    kvt = msa.KVTiled.empty(t["k"].shape[0], case.n_kv_heads, "cuda", fill=float("nan"))
    msa.msa_pack_kv_tiled(shape, t["k"], t["v"], kvt)
    for fused in ([False, True] if mode == "decode" else [False]):
        got = run(case, t, msa.Batch(case.seq_lens, case.rows, page_table=pt), mode, kvt=kvt, fused=fused)
        say(f"[gpu] tiled paged {name} fused={fused}")
        for n in ("block_idx", "out", "lse"):
            assert torch.equal(dense[n], got[n]), n


def test_decode_step_appends_one_token():
    """A decode step writes its new key into the tiles (one token per call)
    and attends over it: the result equals the strided cache's."""
    case = make_case("append", [3001], [1], 2, seed=508)
    t = device_tensors(case)
    shape = shape_of(case)
    kvt = msa.KVTiled.empty(3001, 2, "cuda", fill=float("nan"))
    msa.msa_pack_kv_tiled(shape, t["k"], t["v"], kvt, 0, 3000)       # the prefix
    msa.msa_pack_kv_tiled(shape, t["k"], t["v"], kvt, 3000, 3001)    # the step's own key
    got = run(case, t, msa.Batch(case.seq_lens, case.rows), "decode", kvt=kvt)
    dense = run(case, t, msa.Batch(case.seq_lens, case.rows), "decode")
    for n in ("block_idx", "out", "lse"):
        assert torch.equal(dense[n], got[n]), n


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_pack_rows_writes_the_rows_keys(layout):
    """msa_pack_kv_tiled_rows writes exactly the batch's own keys: tiles packed
    from a cache whose row keys are zeroed, then given the rows' keys, equal
    tiles packed whole from the real cache."""
    kw = CASES["window"]
    case = make_case("rows", **kw)
    t = device_tensors(case)
    if layout == "paged":
        pool, pt = to_pages(case, seed=12, extra_pages=2)
        t.update({n: x.cuda() for n, x in pool.items()})
        batch = msa.Batch(case.seq_lens, case.rows, page_table=pt)
        tok = lambda s, j: int(pt[s, j // 64]) * 64 + j % 64
    else:
        t, starts = aligned_copy(case, t)
        batch = msa.Batch(case.seq_lens, case.rows, kv_start=starts)
        tok = lambda s, j: starts[s] + j
    kz, vz = t["k"].clone(), t["v"].clone()
    for s, (L, n) in enumerate(zip(case.seq_lens, case.rows)):
        for j in range(L - n, L):
            kz[tok(s, j)] = 0
            vz[tok(s, j)] = 0
    shape = shape_of(case)
    T = t["k"].shape[0]
    want = msa.KVTiled.empty(T, case.n_kv_heads, "cuda", fill=float("nan"))
    got = msa.KVTiled.empty(T, case.n_kv_heads, "cuda", fill=float("nan"))
    msa.msa_pack_kv_tiled(shape, t["k"], t["v"], want)
    msa.msa_pack_kv_tiled(shape, kz, vz, got)
    msa.msa_pack_kv_tiled_rows(shape, batch, t["k"], t["v"], got)
    torch.cuda.synchronize()
    assert np.array_equal(u16(got.k), u16(want.k))
    assert np.array_equal(u16(got.v), u16(want.v))
