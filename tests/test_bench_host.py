"""Host checks of bench.py's arithmetic: the algorithmic work its roofline
divides by (against closed forms of the workload definitions), and the
validation it runs against the oracle."""
import numpy as np
import pytest

import bench
import oracle
from workloads import config, make_case


def test_algorithmic_work_of_the_chunk():
    """4,096 rows at positions 65,536..69,631, 4 key heads x 16 query heads,
    top-16 of 64-key blocks including the local one."""
    case = config("chunk")
    w = bench.algorithmic_work(case)
    rows = np.arange(65536, 69632, dtype=np.int64)
    pairs = int((rows + 1).sum()) * 4                       # every causal (row, key) pair, per key head
    assert pairs == 4096 * 65536 * 4 + 4096 * 4097 // 2 * 4
    assert w["index_scores"]["flops"] == 2 * 64 * pairs      # 141.7 GFLOP
    assert abs(w["index_scores"]["flops"] - 141.7e9) < 0.05e9
    # each row keeps 15 whole earlier blocks plus its local block up to itself
    kept = 15 * 64 * 4096 + 64 * (64 * 65 // 2)
    assert kept == 4_065_280
    assert w["attention"]["flops"] == 4 * 128 * kept * 4 * 16   # 133.2 GFLOP
    assert abs(w["attention"]["flops"] - 133.2e9) < 0.05e9


def test_algorithmic_work_of_the_long_row():
    case = config("long")
    w = bench.algorithmic_work(case)
    # the index keys read once: 262,144 keys x 4 key heads x 64 dims x 2 bytes
    assert w["index_select"]["bytes"] >= 262144 * 4 * 64 * 2
    assert abs(w["index_select"]["bytes"] - 134.3e6) < 0.1e6
    # one row: 16 kept blocks of 64 keys, K and V of 128 bf16 each, per key head
    assert w["attention"]["bytes"] >= 16 * 64 * 4 * 256 * 2


def test_cache_write_bytes():
    """A step's cache write reads and writes each new key's K and V once:
    rows x key heads x (128 bf16 of K + 128 of V) x (read + write)."""
    for name, rows in (("chunk", 4096), ("long", 1)):
        w = bench.algorithmic_work(config(name))
        assert w["write_cache"] == {"flops": 0, "bytes": rows * 4 * (256 + 256) * 2}


def test_folded_write_work_is_the_sum_of_its_calls():
    """msa_index_select_pack_rows does the cache write and the selection in one
    call: its algorithmic work is theirs added, so a decode step's whole-path
    fraction does not depend on whether the write is folded."""
    for name in ("long", "decode", "windows"):
        w = bench.algorithmic_work(config(name))
        for q in ("flops", "bytes"):
            assert w["write_index_select"][q] == w["write_cache"][q] + w["index_select"][q]
        assert (bench.path_work(w, ("write_index_select", "attention")) ==
                bench.path_work(w, ("write_cache", "index_select", "attention")))
    w = bench.algorithmic_work(config("chunk"))
    assert (bench.path_work(w, ("write_index_scores_select", "attention")) ==
            bench.path_work(w, ("write_cache", "index_scores", "select_blocks", "attention")))


@pytest.fixture(scope="module")
def small():
    c = make_case("v", [3000], [200], 2, seed=5)
    l = make_case("l", [5000], [1], 2, seed=6)
    return c, l, oracle.run(c), oracle.run(l)


def _gpu_like(ref):
    return {"block_idx": ref["block_idx"], "out": ref["out"].astype(np.float32),
            "lse": ref["lse"].astype(np.float32)}


def test_validation_passes_on_the_oracle_outputs(small):
    c, l, full_c, full_l = small
    rows = np.array([0, 5, 77, 199])
    refs = {"chunk": (rows, oracle.run(c, rows=rows)), "long": (np.arange(1), full_l)}
    v = bench.validate({"chunk": c, "long": l}, refs, {"chunk": _gpu_like(full_c), "long": _gpu_like(full_l)})
    assert v["chunk"]["pass"] and v["long"]["pass"]
    assert v["chunk"]["selection_exact"] and v["chunk"]["out_max_abs"] < 1e-6


def test_validation_fails_on_wrong_outputs(small):
    c, l, full_c, full_l = small
    rows = np.array([0, 5, 77, 199])
    refs = {"chunk": (rows, oracle.run(c, rows=rows)), "long": (np.arange(1), full_l)}
    bad = _gpu_like(full_c)
    bad["out"] = bad["out"] + 0.05                               # above the 2e-2 bound
    v = bench.validate({"chunk": c, "long": l}, refs, {"chunk": bad, "long": _gpu_like(full_l)})
    assert not v["chunk"]["pass"]
    wrong = _gpu_like(full_c)
    wrong["block_idx"] = wrong["block_idx"].copy()
    wrong["block_idx"][77, 0, 0] = wrong["block_idx"][77, 0, 1]   # a wrong selection
    v = bench.validate({"chunk": c, "long": l}, refs, {"chunk": wrong, "long": _gpu_like(full_l)})
    assert not v["chunk"]["selection_exact"] and not v["chunk"]["pass"]


def test_kept_bytes_count_distinct_blocks():
    """The attention's K/V bytes count each (sequence, key head, block) kept
    by any row once, with the keys of it that the sequence's last row sees."""
    case = make_case("d", [1000, 300], [3, 2], 2, seed=9, top_k=4)
    idx = np.full((5, 2, 4), -1, dtype=np.int32)
    idx[0, 0, :3] = [0, 1, 15]          # sequence 0 (1,000 keys: block 15 holds 40 of them)
    idx[1, 0, :3] = [1, 2, 15]
    idx[2, 0, :4] = [0, 7, 9, 15]
    idx[:3, 1, :2] = [3, 15]            # head 1: the same two blocks on every row
    idx[3, 0, :2] = [0, 4]              # sequence 1 (300 keys: block 4 holds 44 of them)
    idx[4, 0, :1] = [4]
    idx[3:, 1, :1] = [4]
    per_key = 128 * 2 * 2               # K and V, bf16
    want = (5 * 64 + 40) + (64 + 40) + (64 + 44) + 44
    assert bench.kept_kv_bytes(case, idx) == want * per_key
    w = bench.algorithmic_work(case, block_idx=idx)
    assert w["attention"]["bytes"] == 5 * 2 * 16 * 128 * 2 * 2 + 5 * 2 * 4 * 4 + want * per_key
