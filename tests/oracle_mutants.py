"""A second, NumPy implementation of the MSA reference with switchable planted
mistakes.  Used only by test_planted_controls.py to show that the pins in
pins.py are sensitive: with no mistake it must pass every pin, and with each
mistake at least one pin must fail.  Not an oracle for the GPU path."""
from __future__ import annotations

import numpy as np
import torch

MUTATIONS = ("causal_off_by_one", "drop_local", "head_map_mod", "no_scale",
             "mean_pool", "ties_high", "ik_head0", "local_plus_k",
             "quant_half_up", "quant_scale_128", "kv8_vscale_off")


def _f(t):
    return t.to(torch.float64).numpy()


class Impl:
    def __init__(self, mutation=None):
        assert mutation is None or mutation in MUTATIONS
        self.m = mutation

    @staticmethod
    def _pos(case):
        out = []
        for s, (L, n) in enumerate(zip(case.seq_lens, case.rows)):
            out += [(s, L - n + i) for i in range(n)]
        return out

    def causal_blocks(self, case, rows=None):
        p = np.array([p for _, p in self._pos(case)], dtype=np.int64)
        if rows is not None:
            p = p[np.asarray(rows)]
        return p // case.block + 1

    def block_scores(self, case, rows=None, bs_stride=None):
        B = case.block
        stride = bs_stride or -(-case.max_seq_len // B)
        iq, ik = _f(case.iq), _f(case.ik)
        pos = self._pos(case)
        rows = range(len(pos)) if rows is None else rows
        out = np.full((len(rows), case.n_kv_heads, stride), -np.inf)
        for o, r in enumerate(rows):
            s, p = pos[r]
            k0, L = case.kv_start[s], case.seq_lens[s]
            last = min(p + 1, L - 1) if self.m == "causal_off_by_one" else p
            for g in range(case.n_kv_heads):
                gi = 0 if (ik.shape[1] == 1 or self.m == "ik_head0") else g
                sc = ik[k0:k0 + last + 1, gi] @ iq[r, g]
                for b in range(p // B + 1):
                    blk = sc[b * B:(b + 1) * B]
                    out[o, g, b] = blk.mean() if self.m == "mean_pool" else blk.max()
        return out

    def select_blocks(self, scores32, nb, top_k):
        n, h, _ = scores32.shape
        out = np.full((n, h, top_k), -1, dtype=np.int32)
        for i in range(n):
            for g in range(h):
                nbi = int(nb[i])
                if nbi <= top_k:
                    sel = list(range(nbi))
                else:
                    cand = list(range(nbi)) if self.m == "drop_local" else list(range(nbi - 1))
                    keyf = (lambda b: (-scores32[i, g, b], -b)) if self.m == "ties_high" \
                        else (lambda b: (-scores32[i, g, b], b))
                    cand.sort(key=keyf)
                    if self.m == "drop_local":
                        sel = sorted(cand[:top_k])
                    elif self.m == "local_plus_k":
                        sel = sorted(cand[:top_k]) + [nbi - 1]
                    else:
                        sel = sorted(cand[:top_k - 1]) + [nbi - 1]
                sel = sel[:top_k]
                out[i, g, :len(sel)] = sel
        return out

    def attention(self, case, block_idx, rows=None):
        B = case.block
        q, k, v = _f(case.q), _f(case.k), _f(case.v)
        pos = self._pos(case)
        rows = range(len(pos)) if rows is None else rows
        hq = case.n_kv_heads * case.group
        out = np.zeros((len(rows), hq, case.head_dim))
        lse = np.full((len(rows), hq), -np.inf)
        scale = 1.0 if self.m == "no_scale" else case.scale
        for o, r in enumerate(rows):
            s, p = pos[r]
            k0, L = case.kv_start[s], case.seq_lens[s]
            last = min(p + 1, L - 1) if self.m == "causal_off_by_one" else p
            for h in range(hq):
                g = h % case.n_kv_heads if self.m == "head_map_mod" else h // case.group
                keys = [j for b in block_idx[o, h // case.group] if b >= 0
                        for j in range(b * B, (b + 1) * B) if j <= last]
                if not keys:
                    continue
                z = scale * (k[k0 + np.array(keys), g] @ q[r, h])
                m = z.max()
                w = np.exp(z - m)
                out[o, h] = w @ v[k0 + np.array(keys), g] / w.sum()
                lse[o, h] = m + np.log(w.sum())
        return out, lse

    def quantize_kv8(self, x):
        xf = x.float().numpy()
        amax = np.abs(xf).max(axis=2).astype(np.float32)
        div = np.float32(128.0 if self.m == "quant_scale_128" else 127.0)
        sc = (amax / div).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = (xf / sc[..., None]).astype(np.float32)
        c = np.floor(ratio + np.float32(0.5)) if self.m == "quant_half_up" else np.rint(ratio)
        c = np.clip(np.nan_to_num(c), -127, 127)
        c[sc == 0] = 0
        return c.astype(np.int8), sc

    def attention_kv8(self, case, k8, v8, k_scale, v_scale, block_idx, rows=None):
        import copy
        vs = np.ones_like(v_scale) if self.m == "kv8_vscale_off" else v_scale
        c = copy.copy(case)
        c.k = torch.from_numpy(k8.astype(np.float64) * k_scale.astype(np.float64)[..., None])
        c.v = torch.from_numpy(v8.astype(np.float64) * vs.astype(np.float64)[..., None])
        return self.attention(c, block_idx, rows)
