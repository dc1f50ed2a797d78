"""Python binding of libmsa.so, the MI355X block-sparse attention (MSA) library.

Argument marshalling only: every step runs in the library's HIP kernels.  The
functions carry the C ABI's names (include/msa.h) and take torch tensors for
device memory; PyTorch supplies memory and the current stream.  If the
library is not built, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # loads the HIP runtime the library binds to

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa.so")

GROUP, HEAD_DIM, INDEX_DIM, BLOCK = 16, 128, 64, 64

_lock = threading.Lock()
_lib = None


class MsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"msa status {status}: {detail}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block", ctypes.c_int32), ("top_k", ctypes.c_int32), ("scale", ctypes.c_float)]


class _BatchC(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("total_rows", ctypes.c_int32),
                ("max_rows", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("cu_rows", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("kv_start", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("pages_per_seq", ctypes.c_int32)]


EXPORTS = ("msa_index_scores", "msa_select_blocks", "msa_index_select", "msa_prefill", "msa_decode",
           "msa_quantize_kv8", "msa_prefill_kv8", "msa_decode_kv8",
           "msa_pack_kv_tiled", "msa_pack_kv_tiled_rows", "msa_prefill_tiled", "msa_decode_tiled",
           "msa_decode_tiled_noalloc", "msa_index_select_pack_rows",
           "msa_decode_workspace_bytes", "msa_index_select_workspace_bytes", "msa_status_string",
           "msa_last_error", "msa_version", "msa_peaks_stream_read", "msa_peaks_stream_read_variant",
           "msa_peaks_mfma")


class _KV8C(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("tok_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("scale_tok_stride", ctypes.c_int64), ("scale_head_stride", ctypes.c_int64)]


class _KVTiledC(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            SP, BP = ctypes.POINTER(Shape), ctypes.POINTER(_BatchC)
            L.msa_index_scores.argtypes = [SP, BP, vp, vp, i64, i64, vp, i32, vp]
            L.msa_select_blocks.argtypes = [SP, BP, vp, i32, vp, vp]
            L.msa_prefill.argtypes = [SP, BP, vp, vp, vp, i64, i64, vp, vp, vp, vp]
            L.msa_decode.argtypes = [SP, BP, vp, vp, vp, i64, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.msa_index_select.argtypes = [SP, BP, vp, vp, i64, i64, vp, i32, vp, vp, ctypes.c_size_t, vp]
            KP = ctypes.POINTER(_KV8C)
            L.msa_quantize_kv8.argtypes = [SP, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, vp]
            L.msa_prefill_kv8.argtypes = [SP, BP, vp, KP, vp, vp, vp, vp]
            L.msa_decode_kv8.argtypes = [SP, BP, vp, KP, vp, vp, vp, vp, ctypes.c_size_t, vp]
            TP = ctypes.POINTER(_KVTiledC)
            L.msa_pack_kv_tiled.argtypes = [SP, i64, i64, vp, vp, i64, i64, vp, vp, i64, i64, vp]
            L.msa_pack_kv_tiled_rows.argtypes = [SP, BP, vp, vp, i64, i64, vp, vp, i64, i64, vp]
            L.msa_index_select_pack_rows.argtypes = [SP, BP, vp, vp, i64, i64, vp, i32, vp, vp, ctypes.c_size_t,
                                                     vp, vp, i64, i64, vp, vp, i64, i64, vp]
            L.msa_prefill_tiled.argtypes = [SP, BP, vp, TP, vp, vp, vp, vp]
            L.msa_decode_tiled.argtypes = [SP, BP, vp, TP, vp, vp, vp, vp, ctypes.c_size_t, vp]
            L.msa_decode_tiled_noalloc.argtypes = [SP, BP, vp, TP, vp, vp, vp, vp]
            for n in ("msa_index_scores", "msa_select_blocks", "msa_index_select", "msa_prefill", "msa_decode",
                      "msa_quantize_kv8", "msa_prefill_kv8", "msa_decode_kv8", "msa_pack_kv_tiled",
                      "msa_pack_kv_tiled_rows",
                      "msa_prefill_tiled", "msa_decode_tiled", "msa_decode_tiled_noalloc"):
                getattr(L, n).restype = ctypes.c_int
            L.msa_decode_workspace_bytes.argtypes = [SP, i32]
            L.msa_index_select_workspace_bytes.argtypes = [SP, BP]
            for n in ("msa_decode_workspace_bytes", "msa_index_select_workspace_bytes"):
                getattr(L, n).restype = ctypes.c_size_t
            L.msa_status_string.argtypes = [ctypes.c_int]
            L.msa_status_string.restype = ctypes.c_char_p
            L.msa_last_error.argtypes = []
            L.msa_last_error.restype = ctypes.c_char_p
            L.msa_version.argtypes = []
            L.msa_version.restype = ctypes.c_char_p
            L.msa_peaks_stream_read.argtypes = [vp, i64, vp, vp]
            L.msa_peaks_mfma.argtypes = [vp, i32, i32, vp]
            L.msa_peaks_stream_read_variant.argtypes = [vp, i64, vp, i32, i32, i32, i32, vp]
            L.msa_peaks_stream_read_variant.restype = ctypes.c_int
            L.msa_peaks_stream_read.restype = ctypes.c_int
            L.msa_peaks_mfma.restype = ctypes.c_int
            _lib = L
    return _lib


def make_shape(n_kv_heads: int, top_k: int = 16, scale: float | None = None) -> Shape:
    return Shape(n_kv_heads, GROUP, HEAD_DIM, INDEX_DIM, BLOCK, top_k,
                 (1.0 / HEAD_DIM ** 0.5) if scale is None else scale)


class Batch:
    """A ragged batch: host sizes plus device arrays (kept alive here).
    Sequence s has seq_lens[s] keys and rows[s] query rows, its last positions;
    its keys start at token kv_start[s] (default: packed back to back), or,
    with page_table (int32 [n_seqs, pages_per_seq]), key j of sequence s is
    token page_table[s, j // 64] * 64 + j % 64 of the k / v / ik pools."""

    def __init__(self, seq_lens, rows, device="cuda", kv_start=None, page_table=None):
        seq_lens = [int(x) for x in seq_lens]
        rows = [int(x) for x in rows]
        cu = [0]
        for n in rows:
            cu.append(cu[-1] + n)
        if kv_start is None:
            kv_start, acc = [], 0
            for n in seq_lens:
                kv_start.append(acc)
                acc += n
        self.seq_lens, self.rows, self.kv_start_host = seq_lens, rows, list(kv_start)
        self.n_seqs, self.total_rows = len(seq_lens), cu[-1]
        self.max_rows = max(rows) if rows else 0
        self.max_seq_len = max(seq_lens) if seq_lens else 0
        self.cu_rows = torch.tensor(cu, dtype=torch.int32, device=device)
        self.seq_lens_d = torch.tensor(seq_lens or [0], dtype=torch.int32, device=device)
        self.kv_start = torch.tensor(list(kv_start) or [0], dtype=torch.int64, device=device)
        self.page_table = None
        pt_ptr, pps = None, 0
        if page_table is not None:
            pt = torch.as_tensor(page_table, dtype=torch.int32)
            if pt.dim() != 2 or pt.shape[0] != self.n_seqs:
                raise ValueError("page_table must be [n_seqs, pages_per_seq]")
            self.page_table = pt.to(device).contiguous()
            pt_ptr, pps = self.page_table.data_ptr(), int(pt.shape[1])
        self.c = _BatchC(self.n_seqs, self.total_rows, self.max_rows, self.max_seq_len,
                         self.cu_rows.data_ptr(), self.seq_lens_d.data_ptr(), self.kv_start.data_ptr(),
                         pt_ptr, pps)

    @property
    def n_blocks(self) -> int:
        return -(-self.max_seq_len // BLOCK)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc: int):
    if rc != 0:
        L = lib()
        raise MsaError(rc, f"{L.msa_status_string(rc).decode()}: {L.msa_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name, contiguous=True):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _strides_tok_head(t, name):
    """(token stride, head stride) of a [tokens, heads, dim] view; a single
    head (or a stride-0 broadcast) gives head stride 0 (shared)."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be [tokens, heads, dim] with a contiguous dim axis")
    head = 0 if t.shape[1] == 1 else t.stride(1)
    return t.stride(0), head


def msa_index_scores(shape: Shape, batch: Batch, iq, ik, block_scores, stream=None):
    _need(iq, torch.bfloat16, "iq")
    _need(ik, torch.bfloat16, "ik", contiguous=False)
    _need(block_scores, torch.float32, "block_scores")
    tok, head = _strides_tok_head(ik, "ik")
    _check(lib().msa_index_scores(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(iq), _ptr(ik),
                                  tok, head, _ptr(block_scores), block_scores.shape[-1],
                                  _stream(stream)))


def msa_select_blocks(shape: Shape, batch: Batch, block_scores, block_idx, stream=None):
    _need(block_scores, torch.float32, "block_scores")
    _need(block_idx, torch.int32, "block_idx")
    _check(lib().msa_select_blocks(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(block_scores),
                                   block_scores.shape[-1], _ptr(block_idx), _stream(stream)))


def msa_index_select_workspace_bytes(shape: Shape, batch: Batch) -> int:
    return int(lib().msa_index_select_workspace_bytes(ctypes.byref(shape), ctypes.byref(batch.c)))


def index_select_workspace(shape: Shape, batch: Batch, device="cuda"):
    """A zero-filled workspace for msa_index_select on this batch (its arrival
    counters must start at 0; the library leaves them at 0 after every
    completed call, so it serves any batch it is large enough for)."""
    n = max(msa_index_select_workspace_bytes(shape, batch), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def chunk_select_eligible(shape: Shape, batch: Batch) -> bool:
    """Whether msa_index_select can take this batch with block_scores=None
    (more than 16 rows in a sequence, top_k <= 16): the scores then never
    reach memory."""
    return batch.max_rows > 16 and shape.top_k <= 16


def msa_index_select(shape: Shape, batch: Batch, iq, ik, block_scores, block_idx, workspace=None,
                     stream=None):
    """block_scores=None: the fused prompt-chunk path (no scores written)."""
    _need(iq, torch.bfloat16, "iq")
    _need(ik, torch.bfloat16, "ik", contiguous=False)
    if block_scores is not None:
        _need(block_scores, torch.float32, "block_scores")
    _need(block_idx, torch.int32, "block_idx")
    tok, head = _strides_tok_head(ik, "ik")
    if workspace is None:
        workspace = index_select_workspace(shape, batch, iq.device)
    _check(lib().msa_index_select(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(iq), _ptr(ik), tok, head,
                                  _ptr(block_scores), 0 if block_scores is None else block_scores.shape[-1],
                                  _ptr(block_idx), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)))


def msa_prefill(shape: Shape, batch: Batch, q, k, v, block_idx, out, lse=None, stream=None):
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(block_idx, torch.int32, "block_idx")
    _need(k, torch.bfloat16, "k", contiguous=False)
    _need(v, torch.bfloat16, "v", contiguous=False)
    tok, head = _strides_tok_head(k, "k")
    if _strides_tok_head(v, "v") != (tok, head):
        raise ValueError("k and v must share strides")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(lib().msa_prefill(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(q), _ptr(k), _ptr(v),
                             tok, head, _ptr(block_idx), _ptr(out), _ptr(lse), _stream(stream)))


def msa_decode_workspace_bytes(shape: Shape, total_rows: int) -> int:
    return int(lib().msa_decode_workspace_bytes(ctypes.byref(shape), int(total_rows)))


def decode_workspace(shape: Shape, total_rows: int, device="cuda"):
    """A zero-filled workspace for msa_decode (its counters must start at 0;
    the library leaves them at 0 after every completed call)."""
    n = max(msa_decode_workspace_bytes(shape, total_rows), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def msa_decode(shape: Shape, batch: Batch, q, k, v, block_idx, out, lse=None, workspace=None,
               stream=None):
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(block_idx, torch.int32, "block_idx")
    _need(k, torch.bfloat16, "k", contiguous=False)
    _need(v, torch.bfloat16, "v", contiguous=False)
    tok, head = _strides_tok_head(k, "k")
    if _strides_tok_head(v, "v") != (tok, head):
        raise ValueError("k and v must share strides")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    if workspace is None:
        workspace = decode_workspace(shape, batch.total_rows, q.device)
    _check(lib().msa_decode(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(q), _ptr(k), _ptr(v),
                            tok, head, _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)))


class KV8:
    """An int8 key/value cache: codes int8 [tokens, H, 128] and scales fp32
    [tokens, H] for k and v (device tensors, kept alive here)."""

    def __init__(self, k_codes, v_codes, k_scale, v_scale):
        for t, name in ((k_codes, "k codes"), (v_codes, "v codes")):
            _need(t, torch.int8, name, contiguous=False)
        for t, name in ((k_scale, "k scale"), (v_scale, "v scale")):
            _need(t, torch.float32, name, contiguous=False)
        tok, head = _strides_tok_head(k_codes, "k codes")
        if _strides_tok_head(v_codes, "v codes") != (tok, head):
            raise ValueError("k and v codes must share strides")
        if k_scale.dim() != 2 or k_scale.stride() != v_scale.stride():
            raise ValueError("scales must be [tokens, heads] with equal strides")
        sh = 0 if k_scale.shape[1] == 1 else k_scale.stride(1)
        self.tensors = (k_codes, v_codes, k_scale, v_scale)
        self.c = _KV8C(k_codes.data_ptr(), v_codes.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
                       tok, head, k_scale.stride(0), sh)


def msa_quantize_kv8(shape: Shape, x, codes=None, scales=None, stream=None):
    """int8 codes and fp32 scales of a bf16 [tokens, H, 128] tensor (one
    (token, head) row at a time: scale = max|x| / 127, code = round half to
    even of x / scale).  Returns (codes, scales)."""
    _need(x, torch.bfloat16, "x", contiguous=False)
    tok, head = _strides_tok_head(x, "x")
    T, H, D = x.shape
    if codes is None:
        codes = torch.empty(T, H, D, dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(T, H, dtype=torch.float32, device=x.device)
    _need(codes, torch.int8, "codes", contiguous=False)
    _need(scales, torch.float32, "scales", contiguous=False)
    ctok, chead = _strides_tok_head(codes, "codes")
    sh = 0 if scales.shape[1] == 1 else scales.stride(1)
    _check(lib().msa_quantize_kv8(ctypes.byref(shape), T, _ptr(x), tok, head, _ptr(codes), ctok, chead,
                                  _ptr(scales), scales.stride(0), sh, _stream(stream)))
    return codes, scales


def msa_prefill_kv8(shape: Shape, batch: Batch, q, kv: KV8, block_idx, out, lse=None, stream=None):
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(block_idx, torch.int32, "block_idx")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(lib().msa_prefill_kv8(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(q), ctypes.byref(kv.c),
                                 _ptr(block_idx), _ptr(out), _ptr(lse), _stream(stream)))


def msa_decode_kv8(shape: Shape, batch: Batch, q, kv: KV8, block_idx, out, lse=None, workspace=None,
                   stream=None):
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(block_idx, torch.int32, "block_idx")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    if workspace is None:
        workspace = decode_workspace(shape, batch.total_rows, q.device)
    _check(lib().msa_decode_kv8(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(q), ctypes.byref(kv.c),
                                _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


TILE_ELEMS = 64 * 128   # one key head's K (or V) of one 64-key block


class KVTiled:
    """A tiled bf16 key/value cache (include/msa.h, msa_kv_tiled): K and V
    tiles as bf16 device tensors [blocks, H, 8192] with a contiguous last axis
    (tile (t, g) holds key head g of tokens 64t .. 64t+63), kept alive here."""

    def __init__(self, k_tiles, v_tiles):
        for x, name in ((k_tiles, "k tiles"), (v_tiles, "v tiles")):
            _need(x, torch.bfloat16, name, contiguous=False)
            if x.dim() != 3 or x.shape[2] != TILE_ELEMS or x.stride(2) != 1:
                raise ValueError(f"{name} must be [blocks, heads, {TILE_ELEMS}] with a contiguous last axis")
        if k_tiles.shape != v_tiles.shape or k_tiles.stride() != v_tiles.stride():
            raise ValueError("k and v tiles must share shape and strides")
        self.k, self.v = k_tiles, v_tiles
        self.c = _KVTiledC(k_tiles.data_ptr(), v_tiles.data_ptr(), k_tiles.stride(0), k_tiles.stride(1))

    @staticmethod
    def empty(n_tokens: int, n_kv_heads: int, device="cuda", fill: float | None = None) -> "KVTiled":
        """Tiles for tokens 0 .. n_tokens-1 (block-major); `fill` sets every
        element first (the attention never reads keys no row can see)."""
        nb = max(1, (int(n_tokens) + 63) // 64)
        mk = (lambda: torch.empty(nb, n_kv_heads, TILE_ELEMS, dtype=torch.bfloat16, device=device)) \
            if fill is None else \
            (lambda: torch.full((nb, n_kv_heads, TILE_ELEMS), fill, dtype=torch.bfloat16, device=device))
        return KVTiled(mk(), mk())


def msa_pack_kv_tiled(shape: Shape, k, v, tiles: KVTiled, tok_begin: int = 0, tok_end: int | None = None,
                      stream=None):
    """Write tokens tok_begin .. tok_end-1 of the strided cache (k, v:
    [tokens, H, 128]) into their tiles; other keys of those tiles are kept."""
    _need(k, torch.bfloat16, "k", contiguous=False)
    _need(v, torch.bfloat16, "v", contiguous=False)
    tok, head = _strides_tok_head(k, "k")
    if _strides_tok_head(v, "v") != (tok, head):
        raise ValueError("k and v must share strides")
    tok_end = k.shape[0] if tok_end is None else tok_end
    if not 0 <= tok_begin < tok_end <= min(k.shape[0], v.shape[0]):
        raise ValueError(f"token range [{tok_begin}, {tok_end}) outside k/v of {k.shape[0]} tokens")
    if (tok_end - 1) // 64 >= tiles.k.shape[0] or k.shape[1] != tiles.k.shape[1]:
        raise ValueError("the tiles do not cover the token range or the key heads")
    c = tiles.c
    _check(lib().msa_pack_kv_tiled(ctypes.byref(shape), int(tok_begin), int(tok_end), _ptr(k), _ptr(v), tok, head,
                                   ctypes.c_void_p(c.k), ctypes.c_void_p(c.v), c.block_stride, c.head_stride,
                                   _stream(stream)))


def msa_pack_kv_tiled_rows(shape: Shape, batch: Batch, k, v, tiles: KVTiled, stream=None):
    """Write the batch's own keys (each sequence's last rows_s tokens) from the
    strided cache (k, v: [tokens, H, 128]) into their tiles, in one launch."""
    _need(k, torch.bfloat16, "k", contiguous=False)
    _need(v, torch.bfloat16, "v", contiguous=False)
    tok, head = _strides_tok_head(k, "k")
    if _strides_tok_head(v, "v") != (tok, head):
        raise ValueError("k and v must share strides")
    if k.shape[1] != tiles.k.shape[1] or (k.shape[0] + 63) // 64 > tiles.k.shape[0]:
        raise ValueError("the tiles do not cover k's tokens or key heads")
    c = tiles.c
    _check(lib().msa_pack_kv_tiled_rows(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(k), _ptr(v), tok, head,
                                        ctypes.c_void_p(c.k), ctypes.c_void_p(c.v), c.block_stride, c.head_stride,
                                        _stream(stream)))


def msa_index_select_pack_rows(shape: Shape, batch: Batch, iq, ik, block_scores, block_idx, k, v, tiles: KVTiled,
                               workspace=None, stream=None):
    """msa_pack_kv_tiled_rows(k, v -> tiles) and msa_index_select in one call
    (the writes ride in the selection's launch for decode-shaped batches)."""
    _need(iq, torch.bfloat16, "iq")
    _need(ik, torch.bfloat16, "ik", contiguous=False)
    if block_scores is not None:
        _need(block_scores, torch.float32, "block_scores")
    _need(block_idx, torch.int32, "block_idx")
    _need(k, torch.bfloat16, "k", contiguous=False)
    _need(v, torch.bfloat16, "v", contiguous=False)
    itok, ihead = _strides_tok_head(ik, "ik")
    tok, head = _strides_tok_head(k, "k")
    if _strides_tok_head(v, "v") != (tok, head):
        raise ValueError("k and v must share strides")
    if k.shape[1] != tiles.k.shape[1] or (k.shape[0] + 63) // 64 > tiles.k.shape[0]:
        raise ValueError("the tiles do not cover k's tokens or key heads")
    if workspace is None:
        workspace = index_select_workspace(shape, batch, iq.device)
    c = tiles.c
    _check(lib().msa_index_select_pack_rows(
        ctypes.byref(shape), ctypes.byref(batch.c), _ptr(iq), _ptr(ik), itok, ihead, _ptr(block_scores),
        0 if block_scores is None else block_scores.shape[-1], _ptr(block_idx), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(k), _ptr(v), tok, head, ctypes.c_void_p(c.k),
        ctypes.c_void_p(c.v), c.block_stride, c.head_stride, _stream(stream)))


def msa_prefill_tiled(shape: Shape, batch: Batch, q, kv: KVTiled, block_idx, out, lse=None, stream=None):
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(block_idx, torch.int32, "block_idx")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(lib().msa_prefill_tiled(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(q), ctypes.byref(kv.c),
                                   _ptr(block_idx), _ptr(out), _ptr(lse), _stream(stream)))


def msa_decode_tiled(shape: Shape, batch: Batch, q, kv: KVTiled, block_idx, out, lse=None, workspace=None,
                     stream=None):
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(block_idx, torch.int32, "block_idx")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    if workspace is None:
        workspace = decode_workspace(shape, batch.total_rows, q.device)
    _check(lib().msa_decode_tiled(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(q), ctypes.byref(kv.c),
                                  _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20   # MSA_DECODE_NOALLOC_SCRATCH_BYTES


def msa_decode_tiled_noalloc(shape: Shape, batch: Batch, q, kv: KVTiled, block_idx, out, lse=None, stream=None):
    """msa_decode_tiled with the library's static per-device workspace: the
    call allocates nothing (calls overlapping in time on one device race)."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(block_idx, torch.int32, "block_idx")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(lib().msa_decode_tiled_noalloc(ctypes.byref(shape), ctypes.byref(batch.c), _ptr(q), ctypes.byref(kv.c),
                                          _ptr(block_idx), _ptr(out), _ptr(lse), _stream(stream)))


def run_path(shape: Shape, batch: Batch, t: dict, mode: str = "prefill", out: dict | None = None,
             stream=None, fused: bool = False, kv8: KV8 | None = None, kvt: KVTiled | None = None) -> dict:
    """Enqueue the whole path -- index scores, selection, attention -- on
    device tensors t = {q, k, v, iq, ik}.  mode: "prefill" or "decode".
    fused: steps 1-3 through msa_index_select (for batches of more than 16
    rows in a sequence with top_k <= 16, the fused prompt-chunk kernel: no
    block scores are written then).
    kv8: attend over this int8 cache instead of t["k"], t["v"].
    kvt: attend over this tiled cache instead of t["k"], t["v"].
    Output buffers are allocated unless given in `out`."""
    out = {} if out is None else out
    dev = t["q"].device
    H, rows, nb = shape.n_kv_heads, batch.total_rows, batch.n_blocks
    if "block_scores" not in out:
        out["block_scores"] = torch.empty(rows, H, nb, dtype=torch.float32, device=dev)
    if "block_idx" not in out:
        out["block_idx"] = torch.empty(rows, H, shape.top_k, dtype=torch.int32, device=dev)
    if "out" not in out:
        out["out"] = torch.empty_like(t["q"])
    if "lse" not in out:
        out["lse"] = torch.empty(rows, H * GROUP, dtype=torch.float32, device=dev)
    if fused:
        if "select_workspace" not in out:
            out["select_workspace"] = index_select_workspace(shape, batch, dev)
        # prompt chunks: no scores written (block_scores is left as allocated)
        scores = None if chunk_select_eligible(shape, batch) else out["block_scores"]
        msa_index_select(shape, batch, t["iq"], t["ik"], scores, out["block_idx"],
                         out["select_workspace"], stream)
    else:
        msa_index_scores(shape, batch, t["iq"], t["ik"], out["block_scores"], stream)
        msa_select_blocks(shape, batch, out["block_scores"], out["block_idx"], stream)
    if mode == "prefill":
        if kv8 is not None:
            msa_prefill_kv8(shape, batch, t["q"], kv8, out["block_idx"], out["out"], out["lse"], stream)
        elif kvt is not None:
            msa_prefill_tiled(shape, batch, t["q"], kvt, out["block_idx"], out["out"], out["lse"], stream)
        else:
            msa_prefill(shape, batch, t["q"], t["k"], t["v"], out["block_idx"], out["out"], out["lse"], stream)
    elif mode == "decode":
        if "workspace" not in out:
            out["workspace"] = decode_workspace(shape, rows, dev)
        if kv8 is not None:
            msa_decode_kv8(shape, batch, t["q"], kv8, out["block_idx"], out["out"], out["lse"],
                           out["workspace"], stream)
        elif kvt is not None:
            msa_decode_tiled(shape, batch, t["q"], kvt, out["block_idx"], out["out"], out["lse"],
                             out["workspace"], stream)
        else:
            msa_decode(shape, batch, t["q"], t["k"], t["v"], out["block_idx"], out["out"], out["lse"],
                       out["workspace"], stream)
    else:
        raise ValueError(mode)
    return out


# Measurement kernels (include/msa_peaks.h), not part of the method.
def msa_peaks_stream_read(buf, sink, stream=None):
    """Read every byte of the device tensor buf once (the device's sustained
    HBM read rate, timed by the caller).  sink: a device tensor of >= 1 uint32."""
    _check(lib().msa_peaks_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def msa_peaks_stream_read_variant(buf, sink, unroll: int, width: int, nontemporal: int, wg_per_cu: int,
                                  stream=None):
    """msa_peaks_stream_read with its knobs: loads in flight per thread,
    load width in bytes, nontemporal loads, workgroups per CU."""
    _check(lib().msa_peaks_stream_read_variant(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                               int(unroll), int(width), int(nontemporal), int(wg_per_cu),
                                               _stream(stream)))


def msa_peaks_mfma(sink, workgroups: int, iters: int, stream=None):
    """workgroups x 4 waves x iters x 4 bf16 16x16x32 MFMAs (16,384 FLOP each):
    the device's sustained dense bf16 rate, timed by the caller.  sink: a
    device float32 tensor of >= 256 elements."""
    _check(lib().msa_peaks_mfma(_ptr(sink), int(workgroups), int(iters), _stream(stream)))
