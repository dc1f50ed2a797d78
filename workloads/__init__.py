"""Seeded synthetic inputs for the MSA hot path.

This module is the only code shared by the oracle side and the GPU side.  It
draws random tensors and lays them out; it holds none of the method's
arithmetic (no scores, no pooling, no selection, no softmax).

Layouts (all bf16, token- or row-major, contiguous):
  q   [total_rows, n_kv_heads * group, head_dim]   query rows of every sequence
  k,v [total_keys, n_kv_heads, head_dim]           keys/values of every sequence
  iq  [total_rows, n_kv_heads, index_dim]          indexer queries
  ik  [total_keys, n_kv_heads or 1, index_dim]     indexer keys (1 = shared)
Sequence s owns rows cu_rows[s]:cu_rows[s+1] and keys kv_start[s]:+seq_lens[s];
its rows are its last rows[s] positions (causal within the chunk or window).

Draw order per sequence (fixed, so a seed names the data): q, k, v, then the
indexer tensors (iq, ik; for planted needles: w, z, ik, then the needle
blocks).  Values are fp32 N(0,1) rounded to bf16 (round-to-nearest-even).

The five named workloads follow the configurations the MSA hot path is
measured on: a tiny 2,048-token prefill, a 4 x 32,768-key batched decode, a
4,096-row chunk on a 65,536-key prefix, a 262,144-key decode and four 16-row
verify windows with planted needle blocks (whose index keys are 4x the
window's shared indexer direction, so those blocks must be kept).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import torch

BF16 = torch.bfloat16


@dataclass
class Case:
    name: str
    seq_lens: list
    rows: list
    n_kv_heads: int
    group: int = 16
    head_dim: int = 128
    index_dim: int = 64
    block: int = 64
    top_k: int = 16
    scale: float = 1.0 / math.sqrt(128.0)
    ik_shared: bool = False
    seed: int = 0
    q: torch.Tensor = None
    k: torch.Tensor = None
    v: torch.Tensor = None
    iq: torch.Tensor = None
    ik: torch.Tensor = None
    needles: list = field(default_factory=list)   # per sequence: planted block ids

    @property
    def n_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def cu_rows(self) -> list:
        out = [0]
        for n in self.rows:
            out.append(out[-1] + n)
        return out

    @property
    def kv_start(self) -> list:
        out, acc = [], 0
        for n in self.seq_lens:
            out.append(acc)
            acc += n
        return out

    @property
    def total_rows(self) -> int:
        return sum(self.rows)

    @property
    def total_keys(self) -> int:
        return sum(self.seq_lens)

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens) if self.seq_lens else 0

    @property
    def max_rows(self) -> int:
        return max(self.rows) if self.rows else 0

    def digests(self) -> dict:
        """SHA-256 of every generated tensor (bit patterns), for provenance."""
        out = {}
        for n in ("q", "k", "v", "iq", "ik"):
            t = getattr(self, n)
            out[n] = hashlib.sha256(t.contiguous().view(torch.int16).numpy().tobytes()).hexdigest()
        return out


def _randn(gen: torch.Generator, shape, scale: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x


def make_case(name: str, seq_lens, rows, n_kv_heads: int, seed: int, *,
              index_scale: float = 1.0, ik_shared: bool = False,
              needles_per_seq: int = 0, top_k: int = 16, group: int = 16,
              head_dim: int = 128, index_dim: int = 64, block: int = 64,
              scale: float | None = None, locality: float | None = None) -> Case:
    """Draw one ragged batch.

    index_scale multiplies both indexer tensors (a power of two keeps bf16 exact).
    needles_per_seq > 0 plants that many blocks per sequence whose index keys are
    4 * w_{s,g}, where the window's indexer queries are (w_{s,g} + z_r)/sqrt(2).
    locality (e.g. 0.95) makes consecutive rows' indexer queries correlated:
    iq_r = a*iq_{r-1} + sqrt(1-a^2)*z_r (a secondary, labelled workload).
    """
    seq_lens = [int(x) for x in seq_lens]
    rows = [int(x) for x in rows]
    assert len(seq_lens) == len(rows)
    for L, n in zip(seq_lens, rows):
        assert 1 <= n <= L, "each sequence needs 1 <= rows <= seq_len"
    gen = torch.Generator().manual_seed(seed)
    hq = n_kv_heads * group
    h_i = 1 if ik_shared else n_kv_heads
    qs, ks, vs, iqs, iks, planted = [], [], [], [], [], []
    for L, n in zip(seq_lens, rows):
        qs.append(_randn(gen, (n, hq, head_dim)))
        ks.append(_randn(gen, (L, n_kv_heads, head_dim)))
        vs.append(_randn(gen, (L, n_kv_heads, head_dim)))
        if needles_per_seq:
            w = _randn(gen, (n_kv_heads, index_dim))
            z = _randn(gen, (n, n_kv_heads, index_dim))
            iq = (w.unsqueeze(0) + z) / math.sqrt(2.0)
            ik = _randn(gen, (L, h_i, index_dim))
            first_local = (L - n) // block
            assert first_local >= needles_per_seq, "not enough earlier blocks for needles"
            blocks = torch.randperm(first_local, generator=gen)[:needles_per_seq]
            blocks = sorted(int(b) for b in blocks)
            for b in blocks:
                ik[b * block:(b + 1) * block, :, :] = 4.0 * w[:h_i].unsqueeze(0)
            planted.append(blocks)
        else:
            if locality is None:
                iq = _randn(gen, (n, n_kv_heads, index_dim), index_scale)
            else:
                z = _randn(gen, (n, n_kv_heads, index_dim), index_scale)
                iq = torch.empty_like(z)
                iq[0] = z[0]
                c = math.sqrt(1.0 - locality * locality)
                for r in range(1, n):
                    iq[r] = locality * iq[r - 1] + c * z[r]
            ik = _randn(gen, (L, h_i, index_dim), index_scale)
            planted.append([])
        iqs.append(iq)
        iks.append(ik)
    return Case(
        name=name, seq_lens=seq_lens, rows=rows, n_kv_heads=n_kv_heads,
        group=group, head_dim=head_dim, index_dim=index_dim, block=block,
        top_k=top_k, scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
        ik_shared=ik_shared, seed=seed,
        q=torch.cat(qs).to(BF16).contiguous(),
        k=torch.cat(ks).to(BF16).contiguous(),
        v=torch.cat(vs).to(BF16).contiguous(),
        iq=torch.cat(iqs).to(BF16).contiguous(),
        ik=torch.cat(iks).to(BF16).contiguous(),
        needles=planted,
    )


# The five named workloads: (seq_lens, rows per sequence, kv heads, seed, extras)
CONFIGS = {
    # 1 sequence, 2,048 tokens, 1 key head; indexer vectors scaled by 1/sqrt(64)
    "tiny": dict(seq_lens=[2048], rows=[2048], n_kv_heads=1, seed=1001, index_scale=0.125),
    # 4 sequences x 32,768 keys, one new row each
    "decode": dict(seq_lens=[32768] * 4, rows=[1] * 4, n_kv_heads=4, seed=1002),
    # one 4,096-row chunk on a 65,536-token cached prefix (69,632 keys)
    "chunk": dict(seq_lens=[69632], rows=[4096], n_kv_heads=4, seed=1003),
    # batch 1 at 262,144 keys
    "long": dict(seq_lens=[262144], rows=[1], n_kv_heads=4, seed=1004),
    # four 16-row verify windows with 8 planted needle blocks each
    "windows": dict(seq_lens=[131072, 98304, 65536, 16384], rows=[16] * 4,
                    n_kv_heads=4, seed=1005, needles_per_seq=8),
}


def config(name: str, **overrides) -> Case:
    kw = dict(CONFIGS[name])
    kw.update(overrides)
    return make_case(name, **kw)


def to_pages(case: Case, seed: int, extra_pages: int = 0, shared=None):
    """The case's k, v and ik laid out in pools of 64-token pages, in a random
    page order (a layout only: the values are the case's own).

    shared = (s_src, s_dst, n_pages): sequence s_dst's first n_pages blocks
    reuse s_src's pages (their keys must already be equal).  Returns
    ({"k", "v", "ik"} CPU pools, page_table int32 numpy [n_seqs, pages_per_seq]);
    key j of sequence s is pool token page_table[s, j // 64] * 64 + j % 64.
    """
    import numpy as np
    B = case.block
    n_blocks = [math.ceil(L / B) for L in case.seq_lens]
    total = sum(n_blocks) + extra_pages
    order = np.random.default_rng(seed).permutation(total)
    pt = np.zeros((case.n_seqs, max(n_blocks)), dtype=np.int32)
    k = torch.zeros(total * B, *case.k.shape[1:], dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    ik = torch.zeros(total * B, *case.ik.shape[1:], dtype=torch.bfloat16)
    used = 0
    for s, L in enumerate(case.seq_lens):
        k0 = case.kv_start[s]
        for blk in range(n_blocks[s]):
            if shared and s == shared[1] and blk < shared[2]:
                pt[s, blk] = pt[shared[0], blk]
                continue
            page = int(order[used])
            used += 1
            pt[s, blk] = page
            n = min(B, L - blk * B)
            src = slice(k0 + blk * B, k0 + blk * B + n)
            dst = slice(page * B, page * B + n)
            k[dst], v[dst], ik[dst] = case.k[src], case.v[src], case.ik[src]
    return {"k": k, "v": v, "ik": ik}, pt
