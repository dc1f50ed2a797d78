"""Checks that pin an MSA reference implementation to facts other than itself.

Each check takes an implementation `impl` with the oracle's interface
(block_scores, select_blocks, attention, causal_blocks) and raises
AssertionError when the implementation disagrees with:
  - a closed form (one-hot index probes, integer inputs whose sums are exact,
    the single-key row, zero keys, constant values),
  - brute force on tiny inputs (per-key score enumeration, subset enumeration
    for the top-k),
  - a library routine in a special case (dense causal attention through
    torch's scaled_dot_product_attention when every block is kept; masked
    dense attention for any given block selection),
  - hand-derived fixtures in tests/golden/.
The real oracle must pass every check (test_oracle_pins.py); planted mutants of
it must fail at least one (test_planted_controls.py).

The method's steps, as the pages describe them: a lightning indexer scores
keys per row and key head; blocks are max-pooled; the top-16 blocks are kept
per GQA group with the local block forced ("minimax-m3-sm120", What this
fixes; TensorFold pull request 1388, the commit adding the minimax_m3 family);
the 16 query heads of a key head share its selection (same pull request, the
4,096-row prompt-chunk commit).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

from workloads import Case, make_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BF16 = torch.bfloat16


def custom_case(seq_lens, rows, n_kv_heads, *, top_k=16, group=16, head_dim=128,
                index_dim=64, block=64, scale=None, seed=7, ik_heads=None, **tensors):
    """A case with the given tensors (float values, rounded to bf16); any tensor
    not given is drawn N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    nr, nk = sum(rows), sum(seq_lens)
    h_i = n_kv_heads if ik_heads is None else ik_heads
    shapes = dict(q=(nr, n_kv_heads * group, head_dim), k=(nk, n_kv_heads, head_dim),
                  v=(nk, n_kv_heads, head_dim), iq=(nr, n_kv_heads, index_dim),
                  ik=(nk, h_i, index_dim))
    t = {}
    for name, shp in shapes.items():
        x = tensors.get(name)
        if x is None:
            x = torch.randn(*shp, generator=g)
        x = torch.as_tensor(x, dtype=torch.float32).reshape(shp)
        t[name] = x.to(BF16).contiguous()
    return Case(name="custom", seq_lens=list(seq_lens), rows=list(rows),
                n_kv_heads=n_kv_heads, group=group, head_dim=head_dim,
                index_dim=index_dim, block=block, top_k=top_k,
                scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                ik_shared=(h_i == 1 and n_kv_heads > 1), seed=seed, **t)


def _positions(case):
    out = []
    for s, (L, n) in enumerate(zip(case.seq_lens, case.rows)):
        out += [(s, L - n + i) for i in range(n)]
    return out


def _f(t):
    return t.to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# Step 1-2: index scores and block max-pool
# ----------------------------------------------------------------------------

def check_onehot_scores(impl):
    """iq is one-hot at dim d(r,g), so the score of key j is exactly
    ik[j, g, d(r,g)]; the block score is the max of those over the block's
    visible keys.  Catches a wrong key offset, head, dim or operand swap."""
    seq_lens, rows, H, dI = [200, 330, 64], [3, 70, 64], 2, 64
    nr, nk = sum(rows), sum(seq_lens)
    iq = np.zeros((nr, H, dI))
    dsel = np.zeros((nr, H), dtype=int)
    for r in range(nr):
        for g in range(H):
            dsel[r, g] = (r * 5 + g * 11) % dI
            iq[r, g, dsel[r, g]] = 1.0
    j, g, d = np.meshgrid(np.arange(nk), np.arange(H), np.arange(dI), indexing="ij")
    ik = ((j * 7 + g * 13 + d * 3) % 29 - 14).astype(np.float64)
    case = custom_case(seq_lens, rows, H, iq=iq, ik=ik)
    S = impl.block_scores(case)
    kv0 = case.kv_start
    for r, (s, p) in enumerate(_positions(case)):
        nb = p // 64 + 1
        for gg in range(H):
            vals = ik[kv0[s]:kv0[s] + p + 1, gg, dsel[r, gg]]
            for b in range(S.shape[2]):
                want = vals[b * 64:(b + 1) * 64].max() if b < nb else -np.inf
                assert S[r, gg, b] == want, (r, gg, b, S[r, gg, b], want)


def check_causal_scores(impl):
    """ik grows with the key's offset inside its block, so the local block's
    score is exactly the value at the row's own position: an off-by-one in the
    causal bound changes it."""
    seq_lens, rows, H, dI = [260, 130], [70, 130], 2, 64
    nk = sum(seq_lens)
    iq = np.ones((sum(rows), H, dI)) / dI          # score = mean over dims of ik
    ik = np.zeros((nk, H, dI))
    for s, L in enumerate(seq_lens):
        base = sum(seq_lens[:s])
        for j in range(L):
            ik[base + j, :, :] = (j % 64) + 64 * ((j // 64) % 2)
    case = custom_case(seq_lens, rows, H, iq=iq, ik=ik)
    S = impl.block_scores(case)
    for r, (s, p) in enumerate(_positions(case)):
        loc = p // 64
        want = (p % 64) + 64 * (loc % 2)
        assert np.all(S[r, :, loc] == want), (r, p, S[r, :, loc], want)
        for b in range(loc):
            assert np.all(S[r, :, b] == 63 + 64 * (b % 2))
        assert np.all(np.isneginf(S[r, :, loc + 1:]))


def check_integer_scores(impl):
    """Integer-valued bf16 inputs: every dot product is an exact integer, so the
    implementation must agree bit for bit with integer brute force."""
    rng = np.random.default_rng(3)
    seq_lens, rows, H, dI = [150, 257, 1], [20, 9, 1], 3, 64
    iq = rng.integers(-8, 9, size=(sum(rows), H, dI)).astype(np.float64)
    ik = rng.integers(-8, 9, size=(sum(seq_lens), H, dI)).astype(np.float64)
    case = custom_case(seq_lens, rows, H, iq=iq, ik=ik)
    S = impl.block_scores(case)
    iqi, iki = iq.astype(np.int64), ik.astype(np.int64)
    for r, (s, p) in enumerate(_positions(case)):
        k0 = case.kv_start[s]
        for g in range(H):
            per_key = [int(np.dot(iqi[r, g], iki[k0 + j, g])) for j in range(p + 1)]
            for b in range(p // 64 + 1):
                assert S[r, g, b] == max(per_key[b * 64:(b + 1) * 64])


def check_shared_index_key(impl):
    """A single index key shared by all key heads (head stride 0) gives every
    head the scores of the same keys with its own query."""
    rng = np.random.default_rng(4)
    seq_lens, rows, H, dI = [190], [5], 4, 64
    iq = rng.integers(-4, 5, size=(5, H, dI)).astype(np.float64)
    ik = rng.integers(-4, 5, size=(190, 1, dI)).astype(np.float64)
    case = custom_case(seq_lens, rows, H, iq=iq, ik=ik, ik_heads=1)
    S = impl.block_scores(case)
    for r, (s, p) in enumerate(_positions(case)):
        for g in range(H):
            per_key = [int(np.dot(iq[r, g].astype(np.int64), ik[j, 0].astype(np.int64)))
                       for j in range(p + 1)]
            for b in range(p // 64 + 1):
                assert S[r, g, b] == max(per_key[b * 64:(b + 1) * 64])


def check_float_scores_bound(impl):
    """Random bf16 inputs: the score must be within the double-precision
    summation bound of the exactly rounded sum (math.fsum of exact products)."""
    case = custom_case([300], [4], 2)
    S = impl.block_scores(case)
    iq, ik = _f(case.iq), _f(case.ik)
    for r, (s, p) in enumerate(_positions(case)):
        for g in range(2):
            per_key = []
            for j in range(p + 1):
                prods = [float(iq[r, g, d]) * float(ik[j, g, d]) for d in range(64)]
                exact = math.fsum(prods)
                per_key.append((exact, sum(abs(x) for x in prods)))
            for b in range(p // 64 + 1):
                blk = per_key[b * 64:(b + 1) * 64]
                want = max(e for e, _ in blk)
                tol = 64 * 2.0 ** -53 * max(a for _, a in blk) + 1e-300
                assert abs(S[r, g, b] - want) <= tol, (S[r, g, b], want)


# ----------------------------------------------------------------------------
# Step 3: top-k selection with a forced local block
# ----------------------------------------------------------------------------

def brute_select(scores, nb, top_k):
    """Enumerate every (top_k-1)-subset of the non-local blocks; keep the one
    with the largest score sum, the lexicographically smallest among equals
    (= ties prefer the lower block index)."""
    if nb <= top_k:
        sel = list(range(nb))
    else:
        best, best_sum = None, None
        for sub in itertools.combinations(range(nb - 1), top_k - 1):
            tot = sum(float(scores[b]) for b in sub)
            if best_sum is None or tot > best_sum:
                best, best_sum = sub, tot
        sel = sorted(best) + [nb - 1]
    return sel + [-1] * (top_k - len(sel))


def check_select_bruteforce(impl):
    rng = np.random.default_rng(11)
    for top_k, nbs in [(1, [1, 2, 9]), (2, [1, 2, 3, 12]), (4, [3, 4, 5, 11, 17]),
                       (16, [1, 15, 16, 17, 19])]:
        for nb in nbs:
            stride = 20
            sc = np.full((3, 2, stride), -np.inf, dtype=np.float32)
            sc[:, :, :nb] = rng.standard_normal((3, 2, nb)).astype(np.float32)
            got = impl.select_blocks(sc, np.array([nb] * 3), top_k)
            for i in range(3):
                for g in range(2):
                    assert list(got[i, g]) == brute_select(sc[i, g], nb, top_k), (top_k, nb)


def check_select_ties(impl):
    """Planted exact ties at the cut: the lower block index must win."""
    rng = np.random.default_rng(12)
    for top_k in (2, 3, 5, 16):
        nb = 19
        for trial in range(6):
            vals = rng.integers(0, 4, size=nb).astype(np.float32)   # many ties
            sc = np.full((1, 1, nb), -np.inf, dtype=np.float32)
            sc[0, 0] = vals
            got = impl.select_blocks(sc, np.array([nb]), top_k)
            assert list(got[0, 0]) == brute_select(vals, nb, top_k), (top_k, vals)


def check_select_invariants(impl):
    """On a random path: local block kept, size min(k, nb), ascending order,
    every kept non-local block scores >= every dropped one."""
    case = make_case("inv", [2000, 700], [40, 30], 2, seed=5)
    s64 = impl.block_scores(case)
    s32 = s64.astype(np.float32)
    nb = impl.causal_blocks(case)
    idx = impl.select_blocks(s32, nb, case.top_k)
    for r in range(idx.shape[0]):
        for g in range(idx.shape[1]):
            sel = [b for b in idx[r, g] if b >= 0]
            assert len(sel) == min(case.top_k, nb[r])
            assert sel == sorted(sel) and len(set(sel)) == len(sel)
            assert sel[-1] == nb[r] - 1
            if nb[r] > case.top_k:
                kept = set(sel[:-1])
                drop = [b for b in range(nb[r] - 1) if b not in kept]
                assert min(s32[r, g, b] for b in kept) >= max(s32[r, g, b] for b in drop)


# ----------------------------------------------------------------------------
# Step 4: attention over the kept keys
# ----------------------------------------------------------------------------

def sdpa_reference(case, allowed):
    """Dense attention in float64 through torch's scaled_dot_product_attention.
    allowed(s, p, g) -> boolean mask over the sequence's keys for the row at
    position p of sequence s and key head g."""
    q, k, v = case.q.double(), case.k.double(), case.v.double()
    outs = []
    r0 = 0
    for s, (L, n) in enumerate(zip(case.seq_lens, case.rows)):
        k0 = case.kv_start[s]
        qs = q[r0:r0 + n].transpose(0, 1)                        # [Hq, n, D]
        ks = k[k0:k0 + L].repeat_interleave(case.group, dim=1).transpose(0, 1).contiguous()
        vs = v[k0:k0 + L].repeat_interleave(case.group, dim=1).transpose(0, 1).contiguous()
        mask = torch.zeros(case.n_kv_heads * case.group, n, L, dtype=torch.bool)
        for i in range(n):
            p = L - n + i
            for g in range(case.n_kv_heads):
                m = torch.as_tensor(allowed(s, p, g, r0 + i))
                mask[g * case.group:(g + 1) * case.group, i] = m
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask,
                                                             scale=case.scale)
        outs.append(o.transpose(0, 1))
        r0 += n
    return torch.cat(outs).numpy()


def _causal(case):
    def allowed(s, p, g, r):
        m = np.zeros(case.seq_lens[s], dtype=bool)
        m[:p + 1] = True
        return m
    return allowed


def check_dense_equivalence(impl):
    """Every row has <= top_k causal blocks, so MSA is dense causal attention."""
    case = make_case("dense", [300, 130, 64, 1], [40, 130, 64, 1], 2, seed=21)
    s32 = impl.block_scores(case).astype(np.float32)
    idx = impl.select_blocks(s32, impl.causal_blocks(case), case.top_k)
    out, _ = impl.attention(case, idx)
    ref = sdpa_reference(case, _causal(case))
    assert np.max(np.abs(out - ref)) < 1e-10


def check_dense_topk_covers(impl):
    """top_k >= the number of causal blocks at any length: dense again."""
    case = make_case("dense32", [2048], [24], 2, seed=22, top_k=32)
    s32 = impl.block_scores(case).astype(np.float32)
    idx = impl.select_blocks(s32, impl.causal_blocks(case), 32)
    out, _ = impl.attention(case, idx)
    ref = sdpa_reference(case, _causal(case))
    assert np.max(np.abs(out - ref)) < 1e-10


def check_masked_dense(impl):
    """Any given block selection: attention equals dense attention masked to
    the kept blocks' causally visible keys (GQA: per key head)."""
    rng = np.random.default_rng(23)
    case = make_case("masked", [1500, 200], [30, 20], 3, seed=23, top_k=5)
    nb = impl.causal_blocks(case)
    idx = np.full((case.total_rows, 3, 5), -1, dtype=np.int32)
    for r in range(case.total_rows):
        for g in range(3):
            c = rng.choice(int(nb[r]), size=min(5, int(nb[r])), replace=False)
            if nb[r] - 1 not in c and rng.random() < 0.5:
                c[0] = nb[r] - 1
            c = np.sort(c)
            idx[r, g, :len(c)] = c
    out, _ = impl.attention(case, idx)

    def allowed(s, p, g, r):
        m = np.zeros(case.seq_lens[s], dtype=bool)
        for b in idx[r, g]:
            if b >= 0:
                m[b * 64:(b + 1) * 64] = True
        m[p + 1:] = False
        return m
    ref = sdpa_reference(case, allowed)
    assert np.max(np.abs(out - ref)) < 1e-10


def check_closed_forms(impl):
    # a row at position 0 sees one key: its output is v[0] and lse the score
    c0 = custom_case([1], [1], 2)
    idx = impl.select_blocks(impl.block_scores(c0).astype(np.float32), impl.causal_blocks(c0), 16)
    out, lse = impl.attention(c0, idx)
    v0 = _f(c0.v)[0]
    for h in range(32):
        assert np.array_equal(out[0, h], v0[h // 16])
        want = c0.scale * float(np.dot(_f(c0.q)[0, h], _f(c0.k)[0, h // 16]))
        assert abs(lse[0, h] - want) <= 1e-12 * (1 + abs(want))
    # zero keys: uniform weights, the output is the mean of v over kept keys
    cz = custom_case([700], [3], 2, k=np.zeros((700, 2, 128)), top_k=4)
    s32 = impl.block_scores(cz).astype(np.float32)
    idx = impl.select_blocks(s32, impl.causal_blocks(cz), 4)
    out, lse = impl.attention(cz, idx)
    v = _f(cz.v)
    for r, (s, p) in enumerate(_positions(cz)):
        for g in range(2):
            keys = [j for b in idx[r, g] if b >= 0 for j in range(b * 64, (b + 1) * 64) if j <= p]
            mean = v[keys, g].mean(axis=0)
            assert np.max(np.abs(out[r, g * 16:(g + 1) * 16] - mean)) < 1e-12
            assert np.allclose(lse[r, g * 16:(g + 1) * 16], math.log(len(keys)))
    # constant values: the output is that constant
    cc = custom_case([900], [5], 1, v=np.full((900, 1, 128), 0.75))
    s32 = impl.block_scores(cc).astype(np.float32)
    idx = impl.select_blocks(s32, impl.causal_blocks(cc), 16)
    out, _ = impl.attention(cc, idx)
    assert np.max(np.abs(out - 0.75)) < 1e-12


# ----------------------------------------------------------------------------
# Hand-derived fixtures
# ----------------------------------------------------------------------------

def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def check_golden_selection(impl):
    """tests/golden/selection_cases.json: block scores written out by hand with
    the kept set derived on paper (local block forced, best others, ties to the
    lower index)."""
    g = load_golden("selection_cases.json")
    for c in g["cases"]:
        sc = np.array([[c["scores"]]], dtype=np.float32)
        got = impl.select_blocks(sc, np.array([len(c["scores"])]), c["top_k"])
        assert list(got[0, 0]) == c["expected"], c["name"]


def check_golden_path(impl):
    """tests/golden/path_cases.json: tiny one-row cases whose index scores,
    selection and softmax weights are worked out by hand."""
    g = load_golden("path_cases.json")
    for c in g["cases"]:
        L, H = c["seq_len"], 1
        iq = np.zeros((1, H, 64))
        iq[0, 0, 0] = 1.0
        ik = np.zeros((L, H, 64))
        for j, val in c["ik_dim0"].items():
            ik[int(j), 0, 0] = val
        q = np.zeros((1, 16, 128))
        q[0, :, 0] = c["q_dim0"]
        k = np.zeros((L, H, 128))
        for j, val in c["k_dim0"].items():
            k[int(j), 0, 0] = val
        v = np.zeros((L, H, 128))
        for j, val in c["v_dim0"].items():
            v[int(j), 0, 0] = val
        case = custom_case([L], [1], H, iq=iq, ik=ik, q=q, k=k, v=v,
                           top_k=c["top_k"], scale=c["scale"])
        s = impl.block_scores(case)
        assert [float(x) for x in s[0, 0, :len(c["block_scores"])]] == c["block_scores"], c["name"]
        idx = impl.select_blocks(s.astype(np.float32), impl.causal_blocks(case), c["top_k"])
        assert list(idx[0, 0]) == c["expected_blocks"], c["name"]
        out, _ = impl.attention(case, idx)
        assert abs(out[0, 0, 0] - c["expected_out_dim0"]) < 1e-12, (c["name"], out[0, 0, 0])


def check_kv8_golden_codes(impl):
    """int8 cache quantisation on hand-derived rows: max |x| = 127 gives scale 1
    and max |x| = 63.5 gives scale 0.5 (both exact), so each code is x / scale
    rounded half to even: -3.5 -> -4, 2.5 -> 2, 0.5 -> 0, 1.5 -> 2, 2.5 -> 2,
    -1.5 -> -2, 0.5 -> 0, 20.5 -> 20."""
    x = torch.tensor([[[127., -3.5, 2.5, 0.5, -1.25, 100., 0., 1.5],
                       [63.5, 1.25, -0.75, 3., -63.5, 0.25, 10.25, -2.]]], dtype=torch.bfloat16)
    codes, sc = impl.quantize_kv8(x)
    assert [float(v) for v in sc[0]] == [1.0, 0.5]
    assert list(codes[0, 0]) == [127, -4, 2, 0, -1, 100, 0, 2]
    assert list(codes[0, 1]) == [127, 2, -2, 6, -127, 0, 20, -4]


def check_kv8_quant_bounds(impl):
    """Any row: |code| <= 127, the largest |x| gets |code| = 127, code * scale is
    within half a step of x (plus the fp32 quotient's own rounding, at most
    127 * 2^-24 of a step), and an all-zero row has scale 0 and codes 0."""
    g = torch.Generator().manual_seed(41)
    x = torch.randn(64, 3, 128, generator=g) * torch.exp(torch.randn(64, 3, 1, generator=g) * 3)
    x[5, 1] = 0.0
    x = x.to(torch.bfloat16)
    codes, sc = impl.quantize_kv8(x)
    xf = x.double().numpy()
    assert np.abs(codes.astype(np.int32)).max() <= 127
    assert sc[5, 1] == 0 and not codes[5, 1].any()
    nz = sc > 0
    am = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(np.abs(codes.astype(np.int32)), am[..., None], axis=2)[..., 0]
    assert (top[nz] == 127).all()
    err = np.abs(xf - codes.astype(np.float64) * sc.astype(np.float64)[..., None])
    assert (err <= sc.astype(np.float64)[..., None] * (0.5 + 2 ** -16) + 1e-300).all()


def _kv8_exact_case(seed):
    """A case whose K and V are codes times power-of-two scales, so the bf16
    tensors hold the dequantised values exactly."""
    case = make_case("kv8x", [700, 130, 64], [20, 5, 64], 2, seed=seed)
    g = torch.Generator().manual_seed(seed)
    T, H, D = case.k.shape
    out = []
    for _ in range(2):
        codes = torch.randint(-127, 128, (T, H, D), generator=g).to(torch.int8)
        e = torch.randint(3, 9, (T, H), generator=g)
        sc = torch.pow(2.0, -e.double()).float()
        out += [codes.numpy(), sc.numpy()]
    k8, ks, v8, vs = out
    case.k = torch.from_numpy(k8.astype(np.float64) * ks.astype(np.float64)[..., None]).to(torch.bfloat16)
    case.v = torch.from_numpy(v8.astype(np.float64) * vs.astype(np.float64)[..., None]).to(torch.bfloat16)
    return case, k8, ks, v8, vs


def check_kv8_attention_exact(impl):
    """Attention over the int8 cache equals attention over bf16 tensors holding
    the same values (codes times power-of-two scales are exact in bf16)."""
    case, k8, ks, v8, vs = _kv8_exact_case(42)
    s32 = impl.block_scores(case).astype(np.float32)
    idx = impl.select_blocks(s32, impl.causal_blocks(case), case.top_k)
    a, la = impl.attention(case, idx)
    b, lb = impl.attention_kv8(case, k8, v8, ks, vs, idx)
    assert np.max(np.abs(a - b)) < 1e-12 and np.max(np.abs(la - lb)) < 1e-12


def check_kv8_dense(impl):
    """Rows with <= top_k causal blocks over the int8 cache are dense causal
    attention over the dequantised keys and values (torch SDPA in float64)."""
    import copy
    case = make_case("kv8d", [300, 64, 1], [40, 64, 1], 2, seed=43)
    k8, ks = impl.quantize_kv8(case.k)
    v8, vs = impl.quantize_kv8(case.v)
    idx = impl.select_blocks(impl.block_scores(case).astype(np.float32), impl.causal_blocks(case), case.top_k)
    out, _ = impl.attention_kv8(case, k8, v8, ks, vs, idx)
    deq = copy.copy(case)
    deq.k = torch.from_numpy(k8.astype(np.float64) * ks.astype(np.float64)[..., None])
    deq.v = torch.from_numpy(v8.astype(np.float64) * vs.astype(np.float64)[..., None])
    ref = sdpa_reference(deq, _causal(deq))
    assert np.max(np.abs(out - ref)) < 1e-10


ALL_CHECKS = [
    check_onehot_scores, check_causal_scores, check_integer_scores, check_shared_index_key,
    check_float_scores_bound, check_select_bruteforce, check_select_ties,
    check_select_invariants, check_dense_equivalence, check_dense_topk_covers,
    check_masked_dense, check_closed_forms, check_golden_selection, check_golden_path,
    check_kv8_golden_codes, check_kv8_quant_bounds, check_kv8_attention_exact, check_kv8_dense,
]
