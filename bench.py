"""Benchmark of the MSA hot path on one MI355X.

One step = the whole path on the two workloads the metric is quoted on:
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
value = rows per second of the step (4,097 rows).  Inputs are resident in HBM
before timing; the timed region enqueues K steps back to back, bracketed by a
device synchronisation on both sides.  Inputs rotate over replicas so the
256 MB Infinity Cache cannot hold a whole step's working set.

Every library call is bracketed by HIP events recorded on the stream the
library launches on (torch's current stream), so per-kernel average durations
come from the same timed region; the dominant kernel's duration gives the
roofline entry.  The oracle (CPU) is timed on a bounded sample of the same
workloads as a reported baseline.
"""
from __future__ import annotations

import argparse
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


def algorithmic_work(case, kv8=False):
    """Per-launch algorithmic FLOPs and bytes of each step for one workload
    (kv8: the int8 cache, 128 + 4 bytes per key and key head for K and for V;
    write_cache: the step's new keys' K and V read once and written once)."""
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
    # kept K/V blocks, counted once per distinct (sequence, key head, block)
    attn_bytes += kept_kv_bytes(case) * (132 if kv8 else 256) // 256
    w["attention"] = dict(flops=4 * D * kept * H * G, bytes=attn_bytes)
    w["write_cache"] = dict(flops=0, bytes=rows * H * D * 2 * 2 * 2)
    return w


def kept_kv_bytes(case):
    """Distinct K/V bytes a perfect cache would read: for the chunk every
    block below its last row is kept by some row, so K and V are read whole;
    for a single row, its 16 blocks."""
    total = 0
    B, k = case.block, case.top_k
    for L, n in zip(case.seq_lens, case.rows):
        nb_last = (L - 1) // B + 1
        blocks = nb_last if n >= 64 else min(nb_last, k * n)
        total += blocks * B * case.head_dim * 2 * 2 * case.n_kv_heads
    return total


PROFILE_KERNELS = {"chunk/attention": "prefill_kernel", "chunk/index_scores": "index_scores_tiled",
                   "long/index_scores": "index_scores_window", "long/index_select": "index_scores_window"}


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
        out = {}
        for k, v in self.ev.items():
            ts = sorted(a.elapsed_time(b) for a, b in v)
            at = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
            out[k] = (at(0.1), at(0.5), at(0.9))
        return out


# The other named workloads: (name, mode, input replicas rotated so the 256 MB
# Infinity Cache cannot hold a call's working set across calls, timed passes).
OTHER_CONFIGS = (("tiny", "prefill", 1, 50), ("decode", "decode", 8, 200), ("windows", "decode", 3, 200))


def other_configs(torch, msa, dev, keep=None, tiled=True):
    """The other named workloads, for reference beside the headline line (not
    part of `value`): the 2,048-token prefill, the batched decode of 4 x 32,768
    keys and the four 16-row verify windows, each timed per library call with
    HIP events (mean and p10 / median / p90 over the timed passes, after two
    warm-up passes per replica).  keep: a dict that receives each workload's
    case and host copies of its outputs, for the oracle leg.  tiled: attend
    over the tiled cache (every sequence of these workloads starts on a
    64-token boundary), each pass writing its new keys into it first."""
    from workloads import config
    out = {}
    for name, mode, n_rep, steps in OTHER_CONFIGS:
        case = config(name)
        base = {n: getattr(case, n).to(dev) for n in ("q", "k", "v", "iq", "ik")}
        reps = [base] + [{n: x.clone() for n, x in base.items()} for _ in range(n_rep - 1)]
        shape = msa.make_shape(case.n_kv_heads, case.top_k, case.scale)
        batch = msa.Batch(case.seq_lens, case.rows, device=dev)
        fused = mode == "decode"
        use_tiles = tiled and all(k0 % 64 == 0 for k0 in case.kv_start)
        new_keys = [(k0 + L - n, k0 + L) for k0, L, n in zip(case.kv_start, case.seq_lens, case.rows)]
        if use_tiles:
            for t in reps:
                t["kvt"] = msa.KVTiled.empty(t["k"].shape[0], case.n_kv_heads, dev)
                msa.msa_pack_kv_tiled(shape, t["k"], t["v"], t["kvt"])
        o = msa.run_path(shape, batch, base, mode, fused=fused, kvt=base.get("kvt"))

        def write(t):   # one token range, or every sequence's new keys in one launch
            if len(new_keys) == 1:
                msa.msa_pack_kv_tiled(shape, t["k"], t["v"], t["kvt"], *new_keys[0])
            else:
                msa.msa_pack_kv_tiled_rows(shape, batch, t["k"], t["v"], t["kvt"])

        def calls(t):
            c = [("write_cache", lambda: write(t))] if use_tiles else []
            if fused:
                c += [("index_select", lambda: msa.msa_index_select(shape, batch, t["iq"], t["ik"], o["block_scores"],
                                                                   o["block_idx"], o["select_workspace"]))]
            else:
                c += [("index_scores", lambda: msa.msa_index_scores(shape, batch, t["iq"], t["ik"],
                                                                    o["block_scores"])),
                     ("select_blocks", lambda: msa.msa_select_blocks(shape, batch, o["block_scores"],
                                                                     o["block_idx"]))]
            if mode == "prefill" and use_tiles:
                c.append(("attention", lambda: msa.msa_prefill_tiled(shape, batch, t["q"], t["kvt"], o["block_idx"],
                                                                     o["out"], o["lse"])))
            elif mode == "prefill":
                c.append(("attention", lambda: msa.msa_prefill(shape, batch, t["q"], t["k"], t["v"], o["block_idx"],
                                                               o["out"], o["lse"])))
            elif use_tiles:
                c.append(("attention", lambda: msa.msa_decode_tiled(shape, batch, t["q"], t["kvt"], o["block_idx"],
                                                                    o["out"], o["lse"], o["workspace"])))
            else:
                c.append(("attention", lambda: msa.msa_decode(shape, batch, t["q"], t["k"], t["v"], o["block_idx"],
                                                              o["out"], o["lse"], o["workspace"])))
            return c

        timer = Timed(torch)
        warm = 2 * n_rep
        gc.disable()   # a collection between an event and its call would show up as kernel time
        for i in range(steps + warm):
            for kname, fn in calls(reps[i % n_rep]):
                if i < warm:
                    fn()
                else:
                    timer.run(kname, fn)
        torch.cuda.synchronize()
        gc.enable()
        kms, kq = timer.mean_ms(), timer.quantiles_ms()
        work = algorithmic_work(case)
        total = sum(kms.values())
        total_median = sum(q[1] for q in kq.values())
        ent = {"mode": mode, "rows": case.total_rows, "seq_lens": case.seq_lens, "kv_heads": case.n_kv_heads,
               "kv_cache": "bf16, tiled (new keys written in each pass)" if use_tiles else "bf16, strided",
               "replicas": n_rep, "steps": steps, "ms": total, "rows_per_s": case.total_rows / (total * 1e-3),
               "ms_median": total_median, "rows_per_s_median": case.total_rows / (total_median * 1e-3),
               "kernels": {k: {"ms": v, "ms_p10": kq[k][0], "ms_median": kq[k][1], "ms_p90": kq[k][2]}
                           for k, v in kms.items()}}
        for k, v in kms.items():
            wk = work[k]
            if wk["flops"] and wk["flops"] / max(wk["bytes"], 1) > PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
                ent["kernels"][k].update(tflops=wk["flops"] / (v * 1e-3) / 1e12,
                                         frac=wk["flops"] / (v * 1e-3) / 1e12 / PEAK_BF16_TFLOPS)
            else:
                ent["kernels"][k].update(gbs=wk["bytes"] / (v * 1e-3) / 1e9,
                                         frac=wk["bytes"] / (v * 1e-3) / 1e9 / PEAK_HBM_GBS)
        out[name] = ent
        if keep is not None:
            keep[name] = (case, {"block_idx": o["block_idx"].cpu().numpy(), "out": o["out"].float().cpu().numpy(),
                                 "lse": o["lse"].cpu().numpy()})
        del base, reps, o
    return out


# Oracle sample per other workload: rows timed and checked (all rows of the
# small decode batches, a spread of rows elsewhere).
OTHER_SAMPLES = {"tiny": 64, "decode": None, "windows": 16}


def other_cpu_baselines(kept, threads):
    """The oracle on a sample of each other workload: its rows/s on the host
    cores (scaled to the whole workload) and the same check of the GPU outputs
    as the headline validation."""
    import numpy as np
    import oracle
    out = {}
    for name, (case, gpu) in kept.items():
        n = OTHER_SAMPLES.get(name)
        rows = (np.arange(case.total_rows) if n is None or n >= case.total_rows
                else np.unique(np.linspace(0, case.total_rows - 1, n).round().astype(np.int64)))
        t0 = time.perf_counter()
        ref = oracle.run(case, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        per_row = dt / len(rows)
        out[name] = {"cpu_baseline": {"value": 1.0 / per_row, "unit": "rows/s", "cores": threads, "kind": "oracle",
                                      "sample": f"{len(rows)} of {case.total_rows} rows ({dt:.2f} s)"},
                     "validation": validate({name: case}, {name: (rows, ref)}, {name: gpu})[name]}
    return out


def measured_peaks(torch, msa, dev):
    """What this device sustains, beside the published peaks: the library's
    streaming-read kernel over 2 GiB and its loop of independent bf16 MFMA
    chains (include/msa_peaks.h), each the best of 5 timed launches."""
    def best_ms(fn, reps=5):
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
    t_read = best_ms(lambda: msa.msa_peaks_stream_read(buf, sink))
    del buf
    wg, iters = 256 * 8, 4000
    t_mfma = best_ms(lambda: msa.msa_peaks_mfma(sink, wg, iters))
    flops = wg * 4 * iters * 4 * 16384
    return {"hbm_read_GBs": nbytes / (t_read * 1e-3) / 1e9,
            "bf16_mfma_TFLOPs": flops / (t_mfma * 1e-3) / 1e12,
            "hbm_read_frac_of_published": nbytes / (t_read * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "bf16_mfma_frac_of_published": flops / (t_mfma * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "sclk": _sclk(),
            "method": "msa_peaks_stream_read over 2 GiB; msa_peaks_mfma with 2,048 workgroups x 4 waves x "
                      "4,000 rounds of 4 independent v_mfma_f32_16x16x32_bf16; best of 5 launches each"}


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


def cpu_baseline(cases, threads, gpu=None):
    """Time the oracle as it stands on a bounded sample: 96 rows of the chunk
    and the decode row; scale to rows/s of the full step.  With `gpu` (the
    timed run's outputs on the host), the same oracle results also check them:
    returns (baseline, validation)."""
    import numpy as np
    import oracle
    chunk, long_ = cases["chunk"], cases["long"]
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(chunk.total_rows, 96, replace=False))
    t0 = time.perf_counter()
    ref_chunk = oracle.run(chunk, rows=sample, threads=threads)
    t_chunk_row = (time.perf_counter() - t0) / len(sample)
    t0 = time.perf_counter()
    ref_long = oracle.run(long_, threads=threads)
    t_long = time.perf_counter() - t0
    step = t_chunk_row * chunk.total_rows + t_long
    base = {"value": (chunk.total_rows + long_.total_rows) / step, "unit": "rows/s", "cores": threads,
            "kind": "oracle",
            "sample": f"96 random rows of the 4,096-row chunk ({t_chunk_row * 1e3:.1f} ms/row) and the "
                      f"262,144-key decode row ({t_long * 1e3:.0f} ms); step time extrapolated to "
                      f"4,096 + 1 rows = {step:.1f} s",
            "cpu": _cpu_model()}
    if gpu is None:
        return base, None
    return base, validate(cases, {"chunk": (sample, ref_chunk), "long": (np.arange(long_.total_rows), ref_long)},
                          gpu)


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


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps for at least this much wall time before the warm-up steps, so the "
                         "timed steps run at the device's steady clocks (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=min(16, os.cpu_count() or 1))
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
    ap.add_argument("--no-overlap", action="store_true",
                    help="enqueue the long row's calls after the chunk's on one stream (default: on a second "
                         "stream, concurrent with the chunk's; the two workloads share no data)")
    ap.add_argument("--unfused", action="store_true",
                    help="long row: msa_index_scores + msa_select_blocks instead of msa_index_select")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the reference timings of the other named workloads after the headline step")
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
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
    reps = {"chunk": 2, "long": 4}       # replicas: >= 512 MB rotated per workload
    modes = {"chunk": "prefill", "long": "decode"}
    fused = {"chunk": False, "long": not args.unfused}
    # the paged pools' new keys are not one token range: there the whole pool
    # is packed before timing and the steps write nothing
    write = tiled and not args.paged
    steps_of = {n: (("write_cache",) if write else ()) +
                   (("index_select", "attention") if fused[n] else ("index_scores", "select_blocks", "attention"))
                for n in modes}
    state = {}
    for name, case in cases.items():
        base = {n: getattr(case, n).to(dev) for n in ("q", "k", "v", "iq", "ik")}
        if args.head_major:
            for n in ("k", "v", "ik"):
                base[n] = base[n].permute(1, 0, 2).contiguous().permute(1, 0, 2)
        page_table = None
        if args.paged:
            from workloads import to_pages
            pool, page_table = to_pages(case, seed=7)
            base.update({n: x.to(dev) for n, x in pool.items()})
        inputs = [base] + [{n: x.clone() for n, x in base.items()} for _ in range(reps[name] - 1)]
        shape = msa.make_shape(case.n_kv_heads, case.top_k, case.scale)
        if args.kv8:
            for t in inputs:
                kc, ks = msa.msa_quantize_kv8(shape, t["k"])
                vc, vs = msa.msa_quantize_kv8(shape, t["v"])
                t["kv8"] = msa.KV8(kc, vc, ks, vs)
                del t["k"], t["v"]
        if tiled:
            for t in inputs:   # the cached prefix, written before timing (set-up)
                t["kvt"] = msa.KVTiled.empty(t["k"].shape[0], case.n_kv_heads, dev)
                msa.msa_pack_kv_tiled(shape, t["k"], t["v"], t["kvt"])
        batch = msa.Batch(case.seq_lens, case.rows, device=dev, page_table=page_table)
        outs = msa.run_path(shape, batch, inputs[0], modes[name], fused=fused[name], kv8=inputs[0].get("kv8"),
                            kvt=inputs[0].get("kvt"))
        state[name] = (shape, batch, inputs, outs)
    torch.cuda.synchronize()

    # Per-call HIP events cost the stream ~5 us each (measured: 0.82 against
    # 0.77 ms per step with an event pair around each of the 5 calls), so the
    # timed steps bracket only the dominant kernel's call; every call's
    # duration comes from a separate untimed pass with events around each.
    per_call = Timed(torch)
    timer = Timed(torch)
    bracket = set()

    # The long row's calls go to a second stream (default priority) in the
    # timed and warm-up steps: its kernels are latency-bound on few
    # workgroups and share nothing with the chunk's, so they run beside them
    # (a serving step that carries a prompt chunk and a decode row at once).
    # The per-call timing pass keeps everything on one stream.
    import contextlib
    side = None if args.no_overlap else torch.cuda.Stream()

    def step(i, timed):
        for name in ("long", "chunk"):
            shape, batch, inputs, o = state[name]
            t = inputs[i % len(inputs)]
            calls = []
            if write:   # the step's new keys (the last total_rows tokens) into the tiles
                n_tok = t["k"].shape[0]
                calls.append(("write_cache", lambda: msa.msa_pack_kv_tiled(shape, t["k"], t["v"], t["kvt"],
                                                                           n_tok - batch.total_rows, n_tok)))
            if fused[name]:
                calls += [("index_select", lambda: msa.msa_index_select(shape, batch, t["iq"], t["ik"],
                                                                       o["block_scores"], o["block_idx"],
                                                                       o["select_workspace"]))]
            else:
                calls += [
                    ("index_scores", lambda: msa.msa_index_scores(shape, batch, t["iq"], t["ik"],
                                                                  o["block_scores"])),
                    ("select_blocks", lambda: msa.msa_select_blocks(shape, batch, o["block_scores"],
                                                                    o["block_idx"])),
                ]
            if modes[name] == "prefill" and args.kv8:
                calls.append(("attention", lambda: msa.msa_prefill_kv8(shape, batch, t["q"], t["kv8"],
                                                                       o["block_idx"], o["out"], o["lse"])))
            elif modes[name] == "prefill" and tiled:
                calls.append(("attention", lambda: msa.msa_prefill_tiled(shape, batch, t["q"], t["kvt"],
                                                                         o["block_idx"], o["out"], o["lse"])))
            elif modes[name] == "prefill":
                calls.append(("attention", lambda: msa.msa_prefill(shape, batch, t["q"], t["k"], t["v"],
                                                                   o["block_idx"], o["out"], o["lse"])))
            elif args.kv8:
                calls.append(("attention", lambda: msa.msa_decode_kv8(shape, batch, t["q"], t["kv8"],
                                                                      o["block_idx"], o["out"], o["lse"],
                                                                      o["workspace"])))
            elif tiled:
                calls.append(("attention", lambda: msa.msa_decode_tiled(shape, batch, t["q"], t["kvt"],
                                                                        o["block_idx"], o["out"], o["lse"],
                                                                        o["workspace"])))
            else:
                calls.append(("attention", lambda: msa.msa_decode(shape, batch, t["q"], t["k"], t["v"],
                                                                  o["block_idx"], o["out"], o["lse"],
                                                                  o["workspace"])))
            on_side = side is not None and name == "long" and timed != "all"
            with torch.cuda.stream(side) if on_side else contextlib.nullcontext():
                for kname, fn in calls:
                    key = f"{name}/{kname}"
                    if timed == "all":
                        per_call.run(key, fn)
                    elif timed and key in bracket:
                        timer.run(key, fn)
                    else:
                        fn()

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
    # untimed pass with an event pair around every call: each kernel's duration
    n_call_steps = max(1, min(args.steps, 50))
    gc.disable()   # a collection between an event and its call would show up as kernel time
    for i in range(n_call_steps):
        step(i, "all")
    torch.cuda.synchronize()
    kms, kq = per_call.mean_ms(), per_call.quantiles_ms()
    dominant = max(kms, key=kms.get)
    bracket.add(dominant)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    ms_step = elapsed / args.steps * 1e3
    rows = sum(c.total_rows for c in cases.values())
    # the dominant kernel: its launches inside the timed steps
    kms[dominant] = timer.mean_ms()[dominant]
    kq[dominant] = timer.quantiles_ms()[dominant]

    kernels = []
    for name, case in cases.items():
        work = algorithmic_work(case, kv8=args.kv8)
        for kname in steps_of[name]:
            ms = kms[f"{name}/{kname}"]
            wk = work[kname]
            bound = "mfma" if wk["flops"] and wk["flops"] / max(wk["bytes"], 1) > PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3 else "hbm"
            if bound == "mfma":
                ach = wk["flops"] / (ms * 1e-3) / 1e12
                ent = dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s")
            else:
                ach = wk["bytes"] / (ms * 1e-3) / 1e9
                ent = dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s")
            ent["frac"] = ent["achieved"] / ent["peak"]
            p10, p50, p90 = kq[f"{name}/{kname}"]
            ent.update(kernel=f"{name}/{kname}", ms=ms, ms_p10=p10, ms_median=p50, ms_p90=p90,
                       algorithmic_flops=wk["flops"], algorithmic_bytes=wk["bytes"],
                       timed_in="timed steps" if f"{name}/{kname}" == dominant else
                       f"untimed pass of {n_call_steps} steps")
            kernels.append(ent)
    dom = next(e for e in kernels if e["kernel"] == dominant)
    roofline = {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    # the committed counter summaries describe the default workload and layout only
    variant = args.kv8 or args.paged or args.head_major or args.locality is not None
    roofline.update(kernel=dom["kernel"], traffic=None if variant else profiled_traffic(dom["kernel"]))

    t_chunk = sum(kms[f"chunk/{k}"] for k in steps_of["chunk"])
    t_long = sum(kms[f"long/{k}"] for k in steps_of["long"])
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
                   "kv_cache": ("int8 codes + fp32 scale per (token, key head)" if args.kv8 else
                                "bf16, tiled (64-key tiles in matrix-core operand order; each step writes its "
                                "new keys into it" + (")" if write else "; pool packed before timing)")
                                if tiled else "bf16"),
                   "index_queries": ("i.i.d. N(0,1) per row" if args.locality is None else
                                     f"secondary workload: AR(1) across the chunk's rows, a = {args.locality}")},
        "inputs": {"generator": "torch.Generator (CPU) seeded per workload, randn in fp32 rounded to bf16",
                   "torch": torch.__version__,
                   "seeds": {n: c.seed for n, c in cases.items()},
                   "sha256": {n: c.digests() for n, c in cases.items()}},
        "prefill_rows_per_s": cases["chunk"].total_rows / (t_chunk * 1e-3),
        "decode_rows_per_s": cases["long"].total_rows / (t_long * 1e-3),
        "roofline": roofline,
        "kernels": kernels,
        "kernel_timing": (f"HIP event pairs on the launch stream: around every launch of the dominant kernel "
                          f"({dominant}) in the timed steps; around every call in an untimed pass of "
                          f"{n_call_steps} steps, all on one stream, for the others (events in the timed steps "
                          f"cost ~5 us each)"),
        "streams": ("one: the long row's calls after the chunk's" if side is None else
                    "two (default priority): the long row's calls on a second stream, concurrent with the "
                    "chunk's; prefill_rows_per_s and decode_rows_per_s come from the one-stream per-call pass"),
    }
    if not args.no_others:
        kept = {} if not args.no_cpu_baseline else None
        res["other_configs"] = other_configs(torch, msa, dev, keep=kept, tiled=tiled)
    if not args.no_peaks:
        peaks = measured_peaks(torch, msa, dev)
        res["measured_peaks"] = peaks
        meas = peaks["hbm_read_GBs"] if roofline["unit"] == "GB/s" else peaks["bf16_mfma_TFLOPs"]
        roofline["measured_peak"] = meas
        roofline["frac_of_measured"] = roofline["achieved"] / meas
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
        # the timed run's outputs (every input replica holds the same values)
        gpu = {}
        for name in cases:
            o = state[name][3]
            gpu[name] = {"block_idx": o["block_idx"].cpu().numpy(), "out": o["out"].float().cpu().numpy(),
                         "lse": o["lse"].cpu().numpy()}
        print("[bench] timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        base, val = cpu_baseline(cases, args.cpu_threads, None if args.kv8 else gpu)
        res["cpu_baseline"] = base
        if val is not None:
            res["validation"] = val
        if not args.no_others:
            for name, ent in other_cpu_baselines(kept, args.cpu_threads).items():
                res["other_configs"][name].update(ent)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
