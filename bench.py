"""Benchmark of the MSA hot path on one MI355X.

Headline step = the whole path on the two workloads the metric is quoted on:
  chunk: one 4,096-row prompt chunk on a 65,536-token cached prefix (69,632
         keys), 4 key heads x 16 query heads: the chunk's 4,096 new keys
         written into the tiled cache (msa_pack_kv_tiled) -> index scores ->
         block selection -> msa_prefill_tiled;
  long:  one decode row at 262,144 keys, 4 key heads x 16 query heads: the
         row's new key written into the tiled cache -> msa_index_select
         (index scores and block selection in one launch) ->
         msa_decode_tiled (split-K, last-arriver combine); --unfused runs the
         two separate selection steps instead.
The key/value cache is the library's tiled bf16 layout (the cached prefix
is packed before timing, as earlier steps would have written it; each step
writes its own new keys); --kv-layout strided attends over the plain
[tokens, heads, 128] cache instead (msa_prefill / msa_decode, no cache write).
value = rows per second of the headline step (4,097 rows).  Inputs are
resident in HBM before timing; the timed region enqueues K steps back to
back, bracketed by a device synchronisation on both sides.  Inputs rotate
over replicas so the 256 MB Infinity Cache cannot hold a step's working set.
A second stream runs each step's chunk cache write and then the long row's
calls, beside the chunk's indexer and selection; the chunk attention waits
for the write and runs alone.

Per configuration (`configs`): each of the five named workloads (2,048-row
prefill, batched decode, the chunk, the long row, the verify windows) alone,
as a loop of back-to-back steps on one stream with one HIP-event pair per
block of steps: mean, p10 / median / p90 per step, rows/s, and the fraction
of the roofline over the whole path (MFMA for prompt chunks, HBM for decode
shapes, algorithmic bytes counted from the distinct (sequence, key head,
block) triples of the run's own selection).  prefill_rows_per_s and
decode_rows_per_s come from the chunk's and the long row's loops.  A separate
untimed pass with an event pair around every library call gives the
per-kernel breakdown.

The dominant kernel (the chunk attention) is also bracketed by HIP events in
the headline's timed steps; its mean there gives the roofline entry.  The
oracle (CPU) is timed on a bounded sample of the same workloads as a
reported baseline, and its results check the run's own outputs.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA prefill rows/s + decode rows/s at 64K–256K ctx; % of MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3   # FLOP per byte


def kept_kv_bytes(case, block_idx=None, kv_bytes_per_key=None):
    """K and V bytes of the distinct kept blocks: each (sequence, key head,
    block) that any row keeps counts once, with the keys of it that the
    sequence's last row can see.  block_idx: the run's own selection (int32
    [rows, H, top_k]); without it, an upper bound (every causal block kept
    by some row when a sequence has >= 64 rows, else top_k per row)."""
    import numpy as np
    B, H = case.block, case.n_kv_heads
    per_key = kv_bytes_per_key or case.head_dim * 2 * 2       # K and V, bf16
    total = 0
    for s, (L, n) in enumerate(zip(case.seq_lens, case.rows)):
        nb_last = (L - 1) // B + 1
        if block_idx is None:
            blocks = nb_last if n >= 64 else min(nb_last, case.top_k * n)
            full = blocks * B - (nb_last * B - L if blocks == nb_last else 0)
            total += full * per_key * H
            continue
        r0 = case.cu_rows[s]
        sel = np.asarray(block_idx[r0:r0 + n])
        for g in range(H):
            kept = np.unique(sel[:, g, :])
            kept = kept[kept >= 0]
            keys = np.minimum(B, L - kept * B)
            total += int(keys.sum()) * per_key
    return total


def algorithmic_work(case, kv8=False, block_idx=None):
    """Per-launch algorithmic FLOPs and bytes of each step for one workload
    (kv8: the int8 cache, 128 + 4 bytes per key and key head for K and for
    V; write_cache: the step's new keys' K and V read once and written
    once; block_idx: the run's selection, for the distinct kept blocks)."""
    import numpy as np
    H, G, D, dI, B, k = case.n_kv_heads, case.group, case.head_dim, case.index_dim, case.block, case.top_k
    pairs = 0           # causal (row, key) pairs per key head
    kept = 0            # kept visible keys per key head
    for L, n in zip(case.seq_lens, case.rows):
        p = np.arange(L - n, L, dtype=np.int64)
        pairs += int((p + 1).sum())
        nb = p // B + 1
        full = np.minimum(nb, k) - 1                         # kept blocks other than the local one
        kept += int((full * B + (p % B) + 1).sum())
    rows = case.total_rows
    nbk = -(-case.max_seq_len // B)
    keys = case.total_keys
    ik_heads = case.ik.shape[1]
    w = {}
    w["index_scores"] = dict(
        flops=2 * dI * pairs * H,
        bytes=keys * ik_heads * dI * 2 + rows * H * dI * 2 + rows * H * nbk * 4)
    w["select_blocks"] = dict(flops=0, bytes=rows * H * nbk * 4 + rows * H * k * 4)
    # fused: the scores are written once (the exchange buffer) and read back from cache
    w["index_select"] = dict(flops=w["index_scores"]["flops"],
                             bytes=w["index_scores"]["bytes"] + rows * H * k * 4)
    attn_bytes = rows * H * G * D * 2 * 2 + rows * H * k * 4     # q in, out
    attn_bytes += kept_kv_bytes(case, block_idx, (D + 4) * 2 if kv8 else None)
    w["attention"] = dict(flops=4 * D * kept * H * G, bytes=attn_bytes)
    w["write_cache"] = dict(flops=0, bytes=rows * H * D * 2 * 2 * 2)
    # the write carried by the selection's launch (msa_index_select_pack_rows)
    w["write_index_select"] = {q: w["write_cache"][q] + w["index_select"][q] for q in ("flops", "bytes")}
    # the same call on a prompt chunk: the indexer (with the writer) and the selection, scores through memory
    w["write_index_scores_select"] = {q: w["write_cache"][q] + w["index_scores"][q] + w["select_blocks"][q]
                                      for q in ("flops", "bytes")}
    return w


def path_work(work, steps):
    """FLOPs and bytes of a whole step: the sum over the path's calls."""
    return {"flops": sum(work[s]["flops"] for s in steps), "bytes": sum(work[s]["bytes"] for s in steps)}


def bound_of(wk):
    return "mfma" if wk["flops"] and wk["flops"] / max(wk["bytes"], 1) > RIDGE else "hbm"


def fraction(wk, ms, measured=None):
    """Achieved rate of work wk in ms against its bound's published peak (and
    the measured one, if given)."""
    if bound_of(wk) == "mfma":
        ach = wk["flops"] / (ms * 1e-3) / 1e12
        out = dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=ach / PEAK_BF16_TFLOPS)
        if measured:
            out["frac_of_measured"] = ach / measured["bf16_mfma_TFLOPs"]
    else:
        ach = wk["bytes"] / (ms * 1e-3) / 1e9
        out = dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s", frac=ach / PEAK_HBM_GBS)
        if measured:
            out["frac_of_measured"] = ach / measured["hbm_read_GBs"]
    return out


PROFILE_KERNELS = {"chunk/attention": "prefill_kernel", "chunk/index_scores": "index_scores_tiled",
                   "long/index_scores": "index_scores_window", "long/index_select": "index_scores_window",
                   "long/write_index_select": "index_scores_window"}


def source_digest() -> str:
    """SHA-256 over the library's kernel sources and build flags: counters
    taken on other sources no longer describe the kernels that run."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "block_sparse_attention_04_amd")
    files = [os.path.join("csrc", n) for n in sorted(os.listdir(os.path.join(pkg, "csrc")))] + ["build.py"]
    for name in files:
        with open(os.path.join(pkg, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def profiled_traffic(kernel: str):
    """Bytes past L2 per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by its copy-kernel calibration), or
    None when no summary exists or the kernel sources changed since."""
    short = PROFILE_KERNELS.get(kernel)
    if short is None:
        return None
    path = os.path.join(ROOT, "profiles", f"{short}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timed:
    """Collects HIP-event pairs around library calls on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}

    def run(self, name, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.ev.setdefault(name, []).append((a, b))

    def mean_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.ev.items()}

    def quantiles_ms(self):
        """(p10, median, p90) of each call's event times."""
        return {k: quantiles([a.elapsed_time(b) for a, b in v]) for k, v in self.ev.items()}


def quantiles(xs):
    ts = sorted(xs)
    at = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
    return at(0.1), at(0.5), at(0.9)


SMALL_PROMPT_UNITS = 4096   # prompt steps up to this many (row, key head) units carry their cache write


class Workload:
    """One named workload on the device: input replicas (rotated so the
    Infinity Cache cannot hold a step's working set), the tiled cache of each
    replica with its prefix packed, output buffers, and the library calls of
    one step."""

    def __init__(self, torch, msa, dev, name, case, mode, n_rep, *, fused, tiled=True, paged=False,
                 head_major=False, kv8=False, ik_head_major=False, fold_write=True):
        self.name, self.case, self.mode, self.fused = name, case, mode, fused
        self.kv8, self.msa = kv8, msa
        base = {n: getattr(case, n).to(dev) for n in ("q", "k", "v", "iq", "ik")}
        if head_major:
            for n in ("k", "v", "ik"):
                base[n] = base[n].permute(1, 0, 2).contiguous().permute(1, 0, 2)
        elif ik_head_major and not paged:
            base["ik"] = base["ik"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
        self.ik_layout = "head-major" if (head_major or (ik_head_major and not paged)) else "token-major"
        page_table = None
        if paged:
            from workloads import to_pages
            pool, page_table = to_pages(case, seed=7)
            base.update({n: x.to(dev) for n, x in pool.items()})
        self.inputs = [base] + [{n: x.clone() for n, x in base.items()} for _ in range(n_rep - 1)]
        self.shape = msa.make_shape(case.n_kv_heads, case.top_k, case.scale)
        if kv8:
            for t in self.inputs:
                kc, ks = msa.msa_quantize_kv8(self.shape, t["k"])
                vc, vs = msa.msa_quantize_kv8(self.shape, t["v"])
                t["kv8"] = msa.KV8(kc, vc, ks, vs)
                del t["k"], t["v"]
        self.tiled = tiled and not kv8 and (paged or all(k0 % 64 == 0 for k0 in case.kv_start))
        if self.tiled:
            for t in self.inputs:   # the cached prefix, written before timing (set-up)
                t["kvt"] = msa.KVTiled.empty(t["k"].shape[0], case.n_kv_heads, dev)
                msa.msa_pack_kv_tiled(self.shape, t["k"], t["v"], t["kvt"])
        self.batch = msa.Batch(case.seq_lens, case.rows, device=dev, page_table=page_table)
        # the paged pools' new keys are not one token range per sequence:
        # there the whole pool is packed before timing and the steps write nothing
        self.write = self.tiled and not paged
        self.new_keys = [(k0 + L - n, k0 + L) for k0, L, n in zip(case.kv_start, case.seq_lens, case.rows)]
        self.o = msa.run_path(self.shape, self.batch, self.inputs[0], mode, fused=fused,
                              kv8=self.inputs[0].get("kv8"), kvt=self.inputs[0].get("kvt"))
        # The new keys' write rides in the selection's first launch
        # (msa_index_select_pack_rows) unless fold_write is off: for decode
        # steps, and for prompt steps of at most SMALL_PROMPT_UNITS (row, key
        # head) units, whose indexer leaves the chip partly idle (the 2,048-row
        # prefill's is 256 workgroups: 46.4 -> 42.9 us a step).  Larger prompt
        # chunks write their token range with msa_pack_kv_tiled: beside a
        # chip-filling indexer the carried writer measured slower (headline
        # step 679-680 against 675-676 us)
        small_prompt = mode == "prefill" and case.total_rows * case.n_kv_heads <= SMALL_PROMPT_UNITS
        self.fold = self.write and fold_write and (mode == "decode" or small_prompt)
        if self.fold:
            self.steps = ("write_index_select" if fused else "write_index_scores_select", "attention")
            if "select_workspace" not in self.o:
                self.o["select_workspace"] = msa.index_select_workspace(self.shape, self.batch, dev)
        else:
            self.steps = ((("write_cache",) if self.write else ()) +
                          (("index_select",) if fused else ("index_scores", "select_blocks")) + ("attention",))

    @property
    def kv_cache(self):
        if self.kv8:
            return "int8 codes + fp32 scale per (token, key head)"
        if self.tiled:
            return ("bf16, tiled (64-key tiles in matrix-core operand order; each step writes its new keys "
                    "into it)" if self.write else "bf16, tiled (pool packed before timing)")
        return "bf16, strided"

    def calls(self, i):
        """[(step name, callable)] of step i (replica i mod the replicas)."""
        msa, sh, b, o = self.msa, self.shape, self.batch, self.o
        t = self.inputs[i % len(self.inputs)]
        c = []
        if self.fold:
            c.append((self.steps[0], lambda: msa.msa_index_select_pack_rows(
                sh, b, t["iq"], t["ik"], o["block_scores"], o["block_idx"], t["k"], t["v"], t["kvt"],
                o["select_workspace"])))
        elif self.write:
            if len(self.new_keys) == 1:
                t0, t1 = self.new_keys[0]
                c.append(("write_cache", lambda: msa.msa_pack_kv_tiled(sh, t["k"], t["v"], t["kvt"], t0, t1)))
            else:
                c.append(("write_cache", lambda: msa.msa_pack_kv_tiled_rows(sh, b, t["k"], t["v"], t["kvt"])))
        if self.fold:
            pass
        elif self.fused:
            c.append(("index_select", lambda: msa.msa_index_select(sh, b, t["iq"], t["ik"], o["block_scores"],
                                                                   o["block_idx"], o["select_workspace"])))
        else:
            c.append(("index_scores", lambda: msa.msa_index_scores(sh, b, t["iq"], t["ik"], o["block_scores"])))
            c.append(("select_blocks", lambda: msa.msa_select_blocks(sh, b, o["block_scores"], o["block_idx"])))
        prefill = self.mode == "prefill"
        if self.kv8:
            c.append(("attention", (lambda: msa.msa_prefill_kv8(sh, b, t["q"], t["kv8"], o["block_idx"], o["out"],
                                                                o["lse"])) if prefill else
                      (lambda: msa.msa_decode_kv8(sh, b, t["q"], t["kv8"], o["block_idx"], o["out"], o["lse"],
                                                  o["workspace"]))))
        elif self.tiled:
            c.append(("attention", (lambda: msa.msa_prefill_tiled(sh, b, t["q"], t["kvt"], o["block_idx"], o["out"],
                                                                  o["lse"])) if prefill else
                      (lambda: msa.msa_decode_tiled(sh, b, t["q"], t["kvt"], o["block_idx"], o["out"], o["lse"],
                                                    o["workspace"]))))
        else:
            c.append(("attention", (lambda: msa.msa_prefill(sh, b, t["q"], t["k"], t["v"], o["block_idx"], o["out"],
                                                            o["lse"])) if prefill else
                      (lambda: msa.msa_decode(sh, b, t["q"], t["k"], t["v"], o["block_idx"], o["out"], o["lse"],
                                              o["workspace"]))))
        return c

    def run_step(self, i):
        for _, fn in self.calls(i):
            fn()

    def host_outputs(self):
        o = self.o
        return {"block_idx": o["block_idx"].cpu().numpy(), "out": o["out"].float().cpu().numpy(),
                "lse": o["lse"].cpu().numpy()}


def loop_timing(torch, w, steps, block):
    """w's steps back to back on the current stream after a warm-up of two
    passes over the replicas: one event pair around the whole loop (the mean
    per step) and one around each block of `block` steps (p10 / median / p90
    of the per-step time over the blocks)."""
    for i in range(2 * len(w.inputs)):
        w.run_step(i)
    torch.cuda.synchronize()
    n_blk = max(1, steps // block)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_blk)]
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc.disable()
    first.record()
    i = 0
    for a, b in ev:
        a.record()
        for _ in range(block):
            w.run_step(i)
            i += 1
        b.record()
    last.record()
    torch.cuda.synchronize()
    gc.enable()
    per = [a.elapsed_time(b) / block for a, b in ev]
    p10, p50, p90 = quantiles(per)
    return {"steps": i, "steps_per_event_block": block, "ms_mean": first.elapsed_time(last) / i,
            "ms_p10": p10, "ms_median": p50, "ms_p90": p90}


def per_call_timing(torch, w, n_steps):
    """An untimed pass with an event pair around every call of w's steps:
    each call's mean and (p10, median, p90); an event pair costs the stream
    a few microseconds, so short calls read high."""
    timer = Timed(torch)
    gc.disable()
    for i in range(n_steps):
        for k, fn in w.calls(i):
            timer.run(k, fn)
    torch.cuda.synchronize()
    gc.enable()
    return timer.mean_ms(), timer.quantiles_ms()


# Per configuration: (mode, fused selection, input replicas, back-to-back
# steps, steps per event block).  Replicas: >= 512 MB rotated where a step's
# working set would otherwise fit the 256 MB Infinity Cache.
CONFIG_PLAN = {
    "tiny": ("prefill", False, 1, 200, 10),
    "decode": ("decode", True, 8, 400, 10),
    "chunk": ("prefill", False, 2, 40, 2),
    "long": ("decode", True, 4, 400, 10),
    "windows": ("decode", True, 3, 300, 10),
}
CONFIG_LETTER = {"tiny": "T", "decode": "D", "chunk": "C", "long": "L", "windows": "W"}
TARGETS = {"chunk": ("mfma", 0.60), "long": ("hbm", 0.70)}


def config_entry(torch, w, steps, block, measured=None, kv8=False):
    """One configuration alone: back-to-back loop, per-call breakdown, the
    path's algorithmic work (distinct kept blocks from the run's selection)
    and its fraction of the roofline."""
    lt = loop_timing(torch, w, steps, block)
    kms, kq = per_call_timing(torch, w, min(50, steps))
    case = w.case
    work = algorithmic_work(case, kv8=kv8, block_idx=w.o["block_idx"].cpu().numpy())
    pw = path_work(work, w.steps)
    rows = case.total_rows
    ent = {"letter": CONFIG_LETTER.get(w.name), "mode": w.mode, "rows": rows, "seq_lens": case.seq_lens,
           "kv_heads": case.n_kv_heads, "kv_cache": w.kv_cache, "replicas": len(w.inputs),
           "path": list(w.steps), **lt,
           "rows_per_s": rows / (lt["ms_mean"] * 1e-3), "rows_per_s_median": rows / (lt["ms_median"] * 1e-3),
           "algorithmic_flops": pw["flops"], "algorithmic_bytes": pw["bytes"],
           "kv_distinct_bytes": kept_kv_bytes(case, w.o["block_idx"].cpu().numpy()),
           "path_fraction": fraction(pw, lt["ms_mean"], measured),
           "path_fraction_median": fraction(pw, lt["ms_median"], measured)["frac"],
           "kernels": {}}
    for k in w.steps:
        e = {"ms": kms[k], "ms_p10": kq[k][0], "ms_median": kq[k][1], "ms_p90": kq[k][2],
             "algorithmic_flops": work[k]["flops"], "algorithmic_bytes": work[k]["bytes"]}
        e.update({n: v for n, v in fraction(work[k], kms[k], measured).items() if n in ("bound", "achieved",
                                                                                     "unit", "frac")})
        ent["kernels"][k] = e
    ent["kernel_timing"] = (f"event pair around every call in an untimed pass of {min(50, steps)} steps "
                            f"(each pair costs the stream a few microseconds)")
    if w.name in TARGETS:
        b, tgt = TARGETS[w.name]
        ent["target"] = {"bound": b, "frac": tgt, "met": ent["path_fraction"]["frac"] >= tgt}
    return ent


# Oracle sample per configuration: rows timed and checked (all rows of the
# small decode batches, a spread of rows elsewhere).
ORACLE_SAMPLES = {"tiny": 64, "decode": None, "windows": 16, "chunk": 96, "long": None}


def oracle_sample(case, name):
    import numpy as np
    n = ORACLE_SAMPLES.get(name)
    if n is None or n >= case.total_rows:
        return np.arange(case.total_rows)
    if name == "chunk":
        return np.sort(np.random.default_rng(0).choice(case.total_rows, n, replace=False))
    return np.unique(np.linspace(0, case.total_rows - 1, n).round().astype(np.int64))


def oracle_leg(case, name, threads, gpu=None):
    """The oracle on the sample of one workload: its rows/s on the host cores
    (scaled to the whole workload) and, given the GPU's outputs, the check of
    them."""
    import oracle
    rows = oracle_sample(case, name)
    t0 = time.perf_counter()
    ref = oracle.run(case, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    out = {"cpu_baseline": {"value": len(rows) / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
                            "sample": f"{len(rows)} of {case.total_rows} rows ({dt:.2f} s)"}}
    if gpu is not None:
        out["validation"] = validate({name: case}, {name: (rows, ref)}, {name: gpu})[name]
    return out, (rows, ref, dt)


def measured_peaks(torch, msa, dev):
    """What this device sustains, beside the published peaks.  HBM: the
    library's streaming-read kernel swept over loads in flight per thread (1
    to 16), load width (4, 8, 16 bytes), plain or nontemporal loads and
    workgroups per CU (2 to 32), over 2 GiB, best of 3 launches each (the
    best variant is the measured floor); the same sweep's best over four
    rotating 134 MB buffers (the long row's index-key read).  MFMA: a loop of
    independent bf16 MFMA chains."""
    def best_ms(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        return best
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    sweep = []
    for unroll in (1, 2, 4, 8, 16):
        for width in (4, 8, 16):
            for nt in (0, 1):
                for wg in (2, 4, 8, 16, 32):
                    ms = best_ms(lambda: msa.msa_peaks_stream_read_variant(buf, sink, unroll, width, nt, wg))
                    sweep.append({"unroll": unroll, "width": width, "nontemporal": nt, "wg_per_cu": wg,
                                  "GBs": nbytes / (ms * 1e-3) / 1e9})
    sweep.sort(key=lambda e: -e["GBs"])
    best = sweep[0]
    t_default = best_ms(lambda: msa.msa_peaks_stream_read(buf, sink))
    del buf
    # the long row's read size: 134,217,728 bytes, four rotating buffers
    small = [torch.ones((128 << 20) // 4, dtype=torch.int32, device=dev) for _ in range(4)]
    it = {"i": 0}

    def small_read(u, wd, nt, wg):
        msa.msa_peaks_stream_read_variant(small[it["i"] % 4], sink, u, wd, nt, wg)
        it["i"] += 1
    small_sweep = []
    for e in sweep[:12]:
        ms = best_ms(lambda: small_read(e["unroll"], e["width"], e["nontemporal"], e["wg_per_cu"]), reps=8)
        small_sweep.append(dict(e, GBs=(128 << 20) / (ms * 1e-3) / 1e9))
    small_sweep.sort(key=lambda e: -e["GBs"])
    del small
    wg, iters = 256 * 8, 4000
    t_mfma = best_ms(lambda: msa.msa_peaks_mfma(sink, wg, iters))
    flops = wg * 4 * iters * 4 * 16384
    return {"hbm_read_GBs": best["GBs"],
            "hbm_read_frac_of_published": best["GBs"] / PEAK_HBM_GBS,
            "hbm_read_best_variant": {k: best[k] for k in ("unroll", "width", "nontemporal", "wg_per_cu")},
            "hbm_read_default_GBs": nbytes / (t_default * 1e-3) / 1e9,
            "hbm_read_sweep_top": sweep[:8], "hbm_read_sweep_worst": sweep[-3:],
            "hbm_read_134MB_GBs": small_sweep[0]["GBs"], "hbm_read_134MB_variant": small_sweep[0],
            "bf16_mfma_TFLOPs": flops / (t_mfma * 1e-3) / 1e12,
            "bf16_mfma_frac_of_published": flops / (t_mfma * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "sclk": _sclk(),
            "method": "msa_peaks_stream_read_variant over 2 GiB, 150 variants (loads in flight 1-16, width 4/8/16 "
                      "B, plain/nontemporal, 2-32 workgroups per CU), best of 3 launches each; the top 12 again on "
                      "four rotating 128 MiB buffers, best of 8; msa_peaks_mfma with 2,048 workgroups x 4 waves x "
                      "4,000 rounds of 4 independent v_mfma_f32_16x16x32_bf16, best of 3"}


def _sclk():
    """The shader clock rocm-smi reports right after the MFMA loop, or None."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for line in out.splitlines():
        if "sclk" in line:
            return line.split(":", 2)[-1].strip()
    return None


# Tolerances of the parity tests: selection exact outside the near-tie band,
# outputs within max-abs 2e-2 / mean-abs 2e-3, lse within 1e-3.
GAP, MAX_ABS, MEAN_ABS, LSE_ABS = 1e-4, 2e-2, 2e-3, 1e-3


def validate(cases, refs, gpu):
    """The timed run's selection and outputs on the oracle's sample rows."""
    import numpy as np
    import oracle
    out = {}
    for name, (rows, ref) in refs.items():
        g = gpu[name]
        top_k = cases[name].top_k
        gi = g["block_idx"][rows]
        clear = oracle.selection_gap(ref["scores32"], ref["nb"], top_k) >= GAP
        sel_ok = bool(((gi == ref["block_idx"]).all(axis=2) | ~clear).all())
        rows_ok = clear.all(axis=1)
        go = g["out"][rows][rows_ok].astype(np.float64)
        d = np.abs(go - ref["out"][rows_ok]) if rows_ok.any() else np.zeros(1)
        gl, rl = g["lse"][rows][rows_ok].astype(np.float64), ref["lse"][rows_ok]
        dl = np.where(np.isneginf(gl) & np.isneginf(rl), 0.0, np.abs(gl - rl)) if rows_ok.any() else np.zeros(1)
        ent = {"rows": int(len(rows)), "selection_exact": sel_ok, "near_tie_units": int((~clear).sum()),
               "out_max_abs": float(d.max()), "out_mean_abs": float(d.mean()), "lse_max_abs": float(dl.max())}
        ent["pass"] = bool(sel_ok and ent["out_max_abs"] <= MAX_ABS and ent["out_mean_abs"] <= MEAN_ABS
                           and ent["lse_max_abs"] <= LSE_ABS)
        out[name] = ent
    return out


def host_cpu():
    """The host's CPU as the OS reports it: model, logical CPUs, and the
    CPUs this process may run on."""
    info = {"logical_cpus": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0))}
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping", "cpu MHz", "vendor_id") and k not in fields:
                    fields[k] = v
    except OSError:
        pass
    info.update({k.replace(" ", "_"): v for k, v in fields.items()})
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "Socket(s)", "Core(s) per socket", "Thread(s) per core", "CPU max MHz"):
                info["lscpu_" + k.strip().lower().replace(" ", "_").replace("(s)", "s")] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps for at least this much wall time before the warm-up steps, so the "
                         "timed steps run at the device's steady clocks (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=len(os.sched_getaffinity(0)),
                    help="oracle threads (default: every CPU this process may run on)")
    ap.add_argument("--paged", action="store_true",
                    help="keys in pools of 64-token pages in a random page order, addressed through a page "
                         "table (the contiguous layout is the default)")
    ap.add_argument("--head-major", action="store_true",
                    help="contiguous key, value and index-key caches stored head-major ([heads, tokens, dim], "
                         "passed as [tokens, heads, dim] views with their strides) instead of token-major")
    ap.add_argument("--locality", type=float, default=None, metavar="A",
                    help="secondary workload, not the headline one: the chunk's indexer queries follow "
                         "iq_r = A*iq_(r-1) + sqrt(1-A^2)*z_r (e.g. 0.95), so neighbouring rows share blocks")
    ap.add_argument("--kv8", action="store_true",
                    help="attention over the int8 key/value cache (codes + one fp32 scale per token and key "
                         "head, written by msa_quantize_kv8 before timing); the selection is unchanged")
    ap.add_argument("--kv-layout", choices=("tiled", "strided"), default="tiled",
                    help="tiled: the library's tiled bf16 cache (msa_kv_tiled; each step packs its own new "
                         "keys into it); strided: the plain [tokens, heads, 128] cache")
    ap.add_argument("--ik-layout", choices=("token-major", "head-major"), default="token-major",
                    help="the index-key cache: [tokens, heads, 64] (token-major) or [heads, tokens, 64] "
                         "(head-major, passed as a strided [tokens, heads, 64] view)")
    ap.add_argument("--overlap", choices=("write", "indexer", "attention", "free", "none"), default="write",
                    help="the long row's calls: on a second stream after the chunk's cache write (write, "
                         "the default: the write and the long row beside the chunk's indexer and selection; "
                         "the chunk attention waits for the write), on a second stream starting when the "
                         "chunk's cache write on the first stream is done (indexer), when the chunk's "
                         "selection is done (attention: beside the chunk attention), on a free-running second "
                         "stream (free), or after the chunk's on one stream (none)")
    ap.add_argument("--separate-write", action="store_true",
                    help="decode workloads: write the new keys with their own launch "
                         "(msa_pack_kv_tiled_rows / msa_pack_kv_tiled) instead of inside the selection's "
                         "launch (msa_index_select_pack_rows)")
    ap.add_argument("--unfused", action="store_true",
                    help="long row: msa_index_scores + msa_select_blocks instead of msa_index_select")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration back-to-back loops after the headline step")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the device's sustained HBM read and bf16 MFMA rates after timing")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one device copy of this size (a known-size reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters in a profiler run)")
    args = ap.parse_args()
    if args.paged and args.head_major:
        ap.error("--head-major applies to the contiguous layout only")
    if args.kv8 or args.head_major:
        args.kv_layout = "strided"   # their own layouts of the strided cache
    tiled = args.kv_layout == "tiled"
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sharding by key head is described in the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_04_amd as msa
    from workloads import config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    cases = {"chunk": config("chunk") if args.locality is None else config("chunk", locality=args.locality),
             "long": config("long")}
    ik_hm = args.ik_layout == "head-major"
    opts = dict(tiled=tiled, paged=args.paged, head_major=args.head_major, kv8=args.kv8, ik_head_major=ik_hm,
                fold_write=not args.separate_write)
    wl = {"chunk": Workload(torch, msa, dev, "chunk", cases["chunk"], "prefill", CONFIG_PLAN["chunk"][2],
                            fused=False, **opts),
          "long": Workload(torch, msa, dev, "long", cases["long"], "decode", CONFIG_PLAN["long"][2],
                           fused=not args.unfused, **opts)}
    torch.cuda.synchronize()

    side = None if args.overlap == "none" else torch.cuda.Stream()
    # --overlap write moves the chunk's cache write to the second stream; a
    # chunk that writes nothing (strided cache, packed paged pool) starts its
    # long row with the step instead (the indexer placement)
    overlap = ("indexer" if args.overlap == "write" and "write_cache" not in wl["chunk"].steps
               else args.overlap)
    timer = Timed(torch)
    bracket = set()
    marks = [torch.cuda.Event() for _ in range(8)]
    write_marks = [torch.cuda.Event() for _ in range(8)]

    def run_calls(name, calls, timed):
        for kname, fn in calls:
            key = f"{name}/{kname}"
            if timed and key in bracket:
                timer.run(key, fn)
            else:
                fn()

    def step(i, timed):
        """One headline step: the long row (second stream unless --overlap
        none) and the chunk; `timed`: bracket the calls named in `bracket`.
        --overlap write (the default): the chunk's cache write and then the
        long row on the second stream, beside the chunk's indexer and
        selection; indexer: the long row's calls start once the chunk's cache
        write on the first stream is done."""
        chunk_calls = wl["chunk"].calls(i)
        if side is not None and overlap == "write":
            # second stream: the chunk's cache write, then the long row, once
            # everything enqueued before this step on the first stream is
            # done (a replica's tiles are rewritten only after the attention
            # that read them); the chunk attention waits for the write
            mk, wk = marks[i % len(marks)], write_marks[i % len(write_marks)]
            mk.record()
            side.wait_event(mk)
            with torch.cuda.stream(side):
                run_calls("chunk", chunk_calls[:1], timed)
                wk.record()
                run_calls("long", wl["long"].calls(i), timed)
            run_calls("chunk", chunk_calls[1:-1], timed)
            torch.cuda.current_stream().wait_event(wk)
            run_calls("chunk", chunk_calls[-1:], timed)
            return
        if side is not None and overlap in ("indexer", "attention"):
            # the chunk's calls before the long row's start: its cache write
            # (indexer), or everything before its attention (attention)
            n_head = (int(chunk_calls[0][0] == "write_cache") if overlap == "indexer"
                      else len(chunk_calls) - 1)
            run_calls("chunk", chunk_calls[:n_head], timed)
            chunk_calls = chunk_calls[n_head:]
            mk = marks[i % len(marks)]
            mk.record()
            side.wait_event(mk)
        with torch.cuda.stream(side) if side is not None else contextlib.nullcontext():
            run_calls("long", wl["long"].calls(i), timed)
        run_calls("chunk", chunk_calls, timed)

    # Settle: the device raises its clocks over the first tens of milliseconds
    # of sustained work (measured: ~7% slower steps after 3 warm-up steps than
    # after 50), so untimed steps run for at least --settle-ms of wall time
    # before the warm-up steps; the timed steps then see the steady state.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        step(settle_steps, False)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # which call dominates: an untimed one-stream pass with events around each
    n_call_steps = max(1, min(args.steps, 20))
    kms = {}
    for name in ("chunk", "long"):
        m, _ = per_call_timing(torch, wl[name], n_call_steps)
        kms.update({f"{name}/{k}": v for k, v in m.items()})
    dominant = max(kms, key=kms.get)
    bracket.add(dominant)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    gc.disable()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    ms_step = elapsed / args.steps * 1e3
    rows = sum(c.total_rows for c in cases.values())
    dom_ms = timer.mean_ms()[dominant]
    dom_q = timer.quantiles_ms()[dominant]
    dname, dk = dominant.split("/")
    dom_work = algorithmic_work(cases[dname], kv8=args.kv8,
                                block_idx=wl[dname].o["block_idx"].cpu().numpy())[dk]
    roofline = {k: v for k, v in fraction(dom_work, dom_ms).items()}
    # the committed counter summaries describe the default workload and layout only
    variant = args.kv8 or args.paged or args.head_major or args.locality is not None or not tiled
    roofline.update(kernel=dominant, ms=dom_ms, ms_p10=dom_q[0], ms_median=dom_q[1], ms_p90=dom_q[2],
                    algorithmic_flops=dom_work["flops"], algorithmic_bytes=dom_work["bytes"],
                    traffic=None if variant else profiled_traffic(dominant))

    res = {
        "metric": METRIC,
        "value": rows / (ms_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (int8 key/value cache)" if args.kv8 else "bf16",
        "data": "synthetic",
        "config": {"workload": "chunked prefill (1 seq, 4,096 rows on a 65,536-key prefix, 69,632 keys) "
                               "+ long decode (1 row at 262,144 keys); 4 key heads x 16 query heads, "
                               "head_dim 128, index_dim 64, block 64, top-16 incl. local block",
                   "rows_per_step": rows, "kv_heads": 4, "q_heads": 64,
                   "kv_layout": ("paged (64-token pages, random order)" if args.paged else
                                 "contiguous, head-major" if args.head_major else "contiguous, token-major"),
                   "kv_cache": wl["chunk"].kv_cache,
                   "index_key_cache": wl["chunk"].ik_layout,
                   "index_queries": ("i.i.d. N(0,1) per row" if args.locality is None else
                                     f"secondary workload: AR(1) across the chunk's rows, a = {args.locality}")},
        "inputs": {"generator": "torch.Generator (CPU) seeded per workload, randn in fp32 rounded to bf16",
                   "torch": torch.__version__,
                   "seeds": {n: c.seed for n, c in cases.items()},
                   "sha256": {n: c.digests() for n, c in cases.items()}},
        "roofline": roofline,
        "roofline_timing": (f"{dominant}: HIP event pair around each of its launches in the {args.steps} timed "
                            f"steps, on its launch stream; algorithmic work of one launch over that mean"),
        "streams": {"none": "one: the long row's calls after the chunk's",
                    "write": "two (default priority): each step's chunk cache write and then its long row on a "
                             "second stream, beside the chunk's indexer and selection; the chunk attention "
                             "waits for the write",
                    "free": "two (default priority): the long row's calls on a free-running second stream",
                    "attention": "two (default priority): each step's long row on a second stream, starting "
                                 "when the chunk's selection of the same step is done (beside its attention)",
                    "indexer": "two (default priority): each step's long row on a second stream, starting when "
                               "the chunk's cache write of the same step is done (beside its indexer and "
                               "selection)"}[overlap],
    }
    print(f"[bench] headline {ms_step:.4f} ms/step ({res['value'] / 1e6:.3f} M rows/s)", file=sys.stderr,
          flush=True)

    measured = None
    if not args.no_peaks:
        measured = measured_peaks(torch, msa, dev)
        res["measured_peaks"] = measured
        meas = measured["hbm_read_GBs"] if roofline["unit"] == "GB/s" else measured["bf16_mfma_TFLOPs"]
        roofline["measured_peak"] = meas
        roofline["frac_of_measured"] = roofline["achieved"] / meas

    configs = {}
    if not args.no_configs:
        for name in ("tiny", "decode", "chunk", "long", "windows"):
            mode, fused, n_rep, steps, block = CONFIG_PLAN[name]
            if name in wl:
                w = wl[name]
            else:
                w = Workload(torch, msa, dev, name, config(name), mode, n_rep, fused=fused, tiled=tiled,
                             ik_head_major=ik_hm, fold_write=not args.separate_write)
            print(f"[bench] config {name}: {steps} steps back to back", file=sys.stderr, flush=True)
            configs[name] = config_entry(torch, w, steps, block, measured, kv8=args.kv8 and name in wl)
            if name not in wl:
                configs[name]["_workload"] = w
        res["prefill_rows_per_s"] = configs["chunk"]["rows_per_s"]
        res["decode_rows_per_s"] = configs["long"]["rows_per_s"]
        res["config_fractions"] = {CONFIG_LETTER[n]: {"bound": e["path_fraction"]["bound"],
                                                      "frac": e["path_fraction"]["frac"],
                                                      "frac_median": e["path_fraction_median"],
                                                      **({"frac_of_measured": e["path_fraction"]["frac_of_measured"]}
                                                         if measured else {}),
                                                      "ms_mean": e["ms_mean"], "rows_per_s": e["rows_per_s"],
                                                      **({"target": e["target"]["frac"]} if "target" in e else {})}
                                   for n, e in configs.items()}
        res["rows_per_s_basis"] = ("prefill_rows_per_s: the chunk alone, back to back; decode_rows_per_s: the "
                                   "262,144-key row alone, back to back (each step's cache write included)")
    if args.copy_calibration_mib:
        # an elementwise kernel that reads n bytes and writes n bytes once
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n

    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        res["host_cpu"] = host_cpu()
        threads = args.cpu_threads
        legs = {}
        for name in ("chunk", "long"):
            gpu = None if args.kv8 else wl[name].host_outputs()
            legs[name] = oracle_leg(cases[name], name, threads, gpu)
        # the headline step's oracle time: per-row time of the chunk's sample
        # scaled to its 4,096 rows, plus the decode row
        (_, (rc, _, dt_c)), (_, (rl, _, dt_l)) = legs["chunk"], legs["long"]
        t_step = dt_c / len(rc) * cases["chunk"].total_rows + dt_l / len(rl) * cases["long"].total_rows
        res["cpu_baseline"] = {
            "value": rows / t_step, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"96 random rows of the 4,096-row chunk ({dt_c / len(rc) * 1e3:.1f} ms/row) and the "
                      f"262,144-key decode row ({dt_l * 1e3:.0f} ms); step time extrapolated to 4,096 + 1 rows "
                      f"= {t_step:.1f} s",
            "cpu": res["host_cpu"].get("model_name", "unknown")}
        if not args.kv8:
            res["validation"] = {n: legs[n][0]["validation"] for n in legs}
        for name, e in configs.items():
            if name in legs:
                e.update(legs[name][0])
            else:
                w = e["_workload"]
                e.update(oracle_leg(w.case, name, threads, w.host_outputs())[0])
    for e in configs.values():
        e.pop("_workload", None)
    if configs:
        res["configs"] = configs
    print(json.dumps(res))


if __name__ == "__main__":
    main()
