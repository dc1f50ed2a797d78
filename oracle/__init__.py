"""CPU oracle for the MSA hot path -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It never imports the GPU library, and the GPU library never
imports it.  The arithmetic lives in msa_oracle.c (plain C, double precision,
sequential sums); this file only builds it, marshals arrays and rounds block
scores to float before the top-k (the precision the kernels decide in).

Functions and what pins them (tests/test_oracle_pins.py):
  block_scores  -- index dot products + block max-pool.  Pinned by one-hot
                   probes (closed form), integer inputs (exact), brute force.
  select_blocks -- top-k with a forced local block.  Pinned by brute-force
                   subset enumeration on tiny inputs and by invariants.
  attention     -- softmax attention over the kept keys.  Pinned against dense
                   causal attention (a library routine) when every block is
                   kept, against masked dense attention for a given selection,
                   and by closed forms (row 0, zero keys, constant values).
Parity with the trained model's own indexer is unpinned (no weights exist
here); see the readings in msa_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# An AddressSanitizer + UndefinedBehaviorSanitizer build of the same source,
# loaded instead when MSA_ORACLE_SANITIZED=1 (the process must preload the
# sanitizer runtimes; tests/test_oracle_sanitized.py runs the pins that way).
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
_lock = threading.Lock()
_lib = None

I32P = ctypes.POINTER(ctypes.c_int32)
I64P = ctypes.POINTER(ctypes.c_int64)
U16P = ctypes.POINTER(ctypes.c_uint16)
F32P = ctypes.POINTER(ctypes.c_float)
F64P = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True, sanitized: bool = False) -> str:
    """Compile liboracle.so with the host compiler (no fast-math: sums keep
    their order); sanitized: liboracle_san.so, the same source built with
    AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts)."""
    lib = _LIB_SAN if sanitized else _LIB
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(_SRC):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    opt = SAN_FLAGS if sanitized else ["-O2"]
    cmd = ["gcc", *opt, "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def loaded_path() -> str:
    """Path of the oracle library this process uses."""
    return _LIB_SAN if os.environ.get("MSA_ORACLE_SANITIZED") == "1" else _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            sanitized = os.environ.get("MSA_ORACLE_SANITIZED") == "1"
            build(force=False, sanitized=sanitized)
            lib = ctypes.CDLL(_LIB_SAN if sanitized else _LIB)
            lib.oracle_block_scores.restype = ctypes.c_int
            lib.oracle_block_scores.argtypes = [
                ctypes.c_int, I32P, I32P, I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                U16P, U16P, ctypes.c_int64, ctypes.c_int64, I32P, ctypes.c_int,
                ctypes.c_int, F64P, ctypes.c_int]
            lib.oracle_select_blocks.restype = ctypes.c_int
            lib.oracle_select_blocks.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, I64P, F32P, ctypes.c_int,
                I32P, ctypes.c_int]
            I8P = ctypes.POINTER(ctypes.c_int8)
            lib.oracle_attention_kv8.restype = ctypes.c_int
            lib.oracle_attention_kv8.argtypes = [
                ctypes.c_int, I32P, I32P, I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_double, U16P, I8P, I8P, F32P, F32P,
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                I32P, I32P, ctypes.c_int, F64P, F64P, ctypes.c_int]
            lib.oracle_quantize_kv8.restype = None
            lib.oracle_quantize_kv8.argtypes = [
                ctypes.c_int64, ctypes.c_int, ctypes.c_int, U16P, ctypes.c_int64, ctypes.c_int64,
                I8P, ctypes.c_int64, ctypes.c_int64, F32P, ctypes.c_int64, ctypes.c_int64]
            lib.oracle_attention.restype = ctypes.c_int
            lib.oracle_attention.argtypes = [
                ctypes.c_int, I32P, I32P, I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_double, U16P, U16P, U16P,
                ctypes.c_int64, ctypes.c_int64, I32P, I32P, ctypes.c_int, F64P, F64P,
                ctypes.c_int]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def _bits(t) -> np.ndarray:
    """bf16 torch tensor (CPU) or uint16 array -> contiguous uint16 bit array."""
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t, dtype=np.uint16)
    import torch
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _meta(case):
    cu = np.asarray(case.cu_rows, dtype=np.int32)
    sl = np.asarray(case.seq_lens, dtype=np.int32)
    ks = np.asarray(case.kv_start, dtype=np.int64)
    return cu, sl, ks


def _rows(case, rows):
    if rows is None:
        return np.arange(case.total_rows, dtype=np.int32)
    return np.ascontiguousarray(rows, dtype=np.int32)


def threads_default() -> int:
    return os.cpu_count() or 1


def row_positions(case, rows=None) -> np.ndarray:
    """Position of each row: the rows of a sequence are its last n positions."""
    rows = _rows(case, rows)
    cu, sl, _ = _meta(case)
    seq = np.searchsorted(cu, rows, side="right") - 1
    return (sl[seq].astype(np.int64) - (cu[seq + 1] - cu[seq]) + (rows - cu[seq])).astype(np.int64)


def causal_blocks(case, rows=None) -> np.ndarray:
    """Number of causal blocks of each row: floor(p / B) + 1."""
    return row_positions(case, rows) // case.block + 1


def block_scores(case, rows=None, bs_stride=None, threads=None) -> np.ndarray:
    """Double-precision block scores [n_rows, n_kv_heads, bs_stride] (-inf past
    the row's causal blocks)."""
    lib = _load()
    rows = _rows(case, rows)
    if bs_stride is None:
        bs_stride = -(-case.max_seq_len // case.block)
    cu, sl, ks = _meta(case)
    iq, ik = _bits(case.iq), _bits(case.ik)
    h_i = ik.shape[1]
    tok_stride = h_i * case.index_dim
    head_stride = 0 if h_i == 1 else case.index_dim   # 0: one shared index key
    out = np.empty((len(rows), case.n_kv_heads, bs_stride), dtype=np.float64)
    rc = lib.oracle_block_scores(
        case.n_seqs, _ptr(cu, I32P), _ptr(sl, I32P), _ptr(ks, I64P),
        case.n_kv_heads, case.index_dim, case.block, _ptr(iq, U16P), _ptr(ik, U16P),
        tok_stride, head_stride, _ptr(rows, I32P), len(rows), bs_stride,
        _ptr(out, F64P), threads or threads_default())
    if rc != 0:
        raise ValueError("oracle_block_scores: malformed metadata")
    return out


def select_blocks(scores32: np.ndarray, nb: np.ndarray, top_k: int, threads=None) -> np.ndarray:
    """Top-k with the forced local block on float32 scores [n, H, stride];
    nb[n] causal block counts.  Returns int32 [n, H, top_k] ascending, -1 padded."""
    lib = _load()
    s = np.ascontiguousarray(scores32, dtype=np.float32)
    nb = np.ascontiguousarray(nb, dtype=np.int64)
    n, h, stride = s.shape
    out = np.empty((n, h, top_k), dtype=np.int32)
    lib.oracle_select_blocks(n, h, stride, _ptr(nb, I64P), _ptr(s, F32P), top_k,
                             _ptr(out, I32P), threads or threads_default())
    return out


def attention(case, block_idx: np.ndarray, rows=None, threads=None):
    """Softmax attention over the kept keys.  block_idx [n_rows, H_kv, top_k]
    follows `rows`.  Returns (out double [n, H_q, D], lse double [n, H_q])."""
    lib = _load()
    rows = _rows(case, rows)
    cu, sl, ks = _meta(case)
    q, k, v = _bits(case.q), _bits(case.k), _bits(case.v)
    bi = np.ascontiguousarray(block_idx, dtype=np.int32)
    top_k = bi.shape[2]
    hq = case.n_kv_heads * case.group
    out = np.empty((len(rows), hq, case.head_dim), dtype=np.float64)
    lse = np.empty((len(rows), hq), dtype=np.float64)
    rc = lib.oracle_attention(
        case.n_seqs, _ptr(cu, I32P), _ptr(sl, I32P), _ptr(ks, I64P),
        case.n_kv_heads, case.group, case.head_dim, case.block, top_k, float(case.scale),
        _ptr(q, U16P), _ptr(k, U16P), _ptr(v, U16P),
        case.n_kv_heads * case.head_dim, case.head_dim,
        _ptr(bi, I32P), _ptr(rows, I32P), len(rows), _ptr(out, F64P), _ptr(lse, F64P),
        threads or threads_default())
    if rc != 0:
        raise ValueError("oracle_attention: malformed metadata or block list")
    return out, lse


def quantize_kv8(x):
    """int8 codes and fp32 scales of a bf16 [tokens, heads, dim] tensor, one
    scale per (token, head): scale = max|x| / 127, code = round-half-even(x /
    scale) clamped to +-127, both in fp32.  Returns (codes int8 numpy
    [tokens, heads, dim], scales float32 numpy [tokens, heads])."""
    lib = _load()
    T, H, D = x.shape
    xb = _bits(x).reshape(T, H, D)
    codes = np.empty((T, H, D), dtype=np.int8)
    scales = np.empty((T, H), dtype=np.float32)
    lib.oracle_quantize_kv8(T, H, D, _ptr(xb, U16P), H * D, D, codes.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)),
                            H * D, D, _ptr(scales, F32P), H, 1)
    return codes, scales


def attention_kv8(case, k8, v8, k_scale, v_scale, block_idx: np.ndarray, rows=None, threads=None):
    """As attention(), over an int8 cache: every key / value element is
    code * scale (codes [tokens, H_kv, D] int8, scales [tokens, H_kv] fp32, in
    the case's token order).  Returns (out, lse) in double."""
    lib = _load()
    rows = _rows(case, rows)
    cu, sl, ks = _meta(case)
    q = _bits(case.q)
    k8 = np.ascontiguousarray(k8, dtype=np.int8)
    v8 = np.ascontiguousarray(v8, dtype=np.int8)
    ksc = np.ascontiguousarray(k_scale, dtype=np.float32)
    vsc = np.ascontiguousarray(v_scale, dtype=np.float32)
    bi = np.ascontiguousarray(block_idx, dtype=np.int32)
    top_k = bi.shape[2]
    H, D = case.n_kv_heads, case.head_dim
    hq = H * case.group
    out = np.empty((len(rows), hq, D), dtype=np.float64)
    lse = np.empty((len(rows), hq), dtype=np.float64)
    i8 = ctypes.POINTER(ctypes.c_int8)
    rc = lib.oracle_attention_kv8(
        case.n_seqs, _ptr(cu, I32P), _ptr(sl, I32P), _ptr(ks, I64P), H, case.group, D, case.block, top_k,
        float(case.scale), _ptr(q, U16P), k8.ctypes.data_as(i8), v8.ctypes.data_as(i8), _ptr(ksc, F32P),
        _ptr(vsc, F32P), H * D, D, H, 1, _ptr(bi, I32P), _ptr(rows, I32P), len(rows), _ptr(out, F64P),
        _ptr(lse, F64P), threads or threads_default())
    if rc != 0:
        raise ValueError("oracle_attention_kv8: malformed metadata or block list")
    return out, lse


def run(case, rows=None, threads=None, top_k=None) -> dict:
    """The whole path for the chosen rows: scores, selection, attention."""
    rows = _rows(case, rows)
    top_k = case.top_k if top_k is None else top_k
    s64 = block_scores(case, rows, threads=threads)
    s32 = s64.astype(np.float32)
    nb = causal_blocks(case, rows)
    idx = select_blocks(s32, nb, top_k, threads=threads)
    out, lse = attention(case, idx, rows, threads=threads)
    return dict(rows=rows, nb=nb, scores64=s64, scores32=s32, block_idx=idx, out=out, lse=lse)


def selection_gap(scores32: np.ndarray, nb: np.ndarray, top_k: int) -> np.ndarray:
    """For each (row, head): the gap between the last kept and the first dropped
    non-local block score (rank top_k-1 vs top_k among blocks below the local
    one).  Rows with nb <= top_k have no decision: +inf."""
    n, h, _ = scores32.shape
    gap = np.full((n, h), np.inf)
    for i in range(n):
        m = int(nb[i]) - 1                      # candidates: blocks 0..nb-2
        if nb[i] <= top_k:
            continue
        cand = np.sort(scores32[i, :, :m].astype(np.float64), axis=1)[:, ::-1]
        gap[i] = cand[:, top_k - 2] - cand[:, top_k - 1]
    return gap
