// api.hip -- the library's C ABI (include/msa.h): host-side validation, then
// one launch sequence per entry point on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "msa.h"
#include "msa_device.h"
#include "msa_launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return MSA_OK;
}

}  // namespace

// Library-internal: the message msa_last_error() returns (other sources of
// the library report through it too).
namespace msa {
int report(int status, const char *msg) {
    snprintf(g_last_error, sizeof g_last_error, "%s", msg);
    return status;
}
}  // namespace msa

namespace {

int check_shape(const msa_shape *sh) {
    if (!sh) return fail(MSA_ERR_INVALID, "shape is NULL");
    if (sh->n_kv_heads < 1) return fail(MSA_ERR_INVALID, "n_kv_heads=%d must be >= 1", sh->n_kv_heads);
    if (sh->n_kv_heads > 4096) return fail(MSA_ERR_UNSUPPORTED, "n_kv_heads=%d > 4096", sh->n_kv_heads);
    if (sh->group != msa::kGroup || sh->head_dim != msa::kHeadDim || sh->index_dim != msa::kIndexDim ||
        sh->block != msa::kBlock)
        return fail(MSA_ERR_UNSUPPORTED,
                    "group=%d head_dim=%d index_dim=%d block=%d: only 16/128/64/64 are built",
                    sh->group, sh->head_dim, sh->index_dim, sh->block);
    if (sh->top_k < 1 || sh->top_k > msa::kMaxTopK)
        return fail(MSA_ERR_UNSUPPORTED, "top_k=%d outside [1, %d]", sh->top_k, msa::kMaxTopK);
    if (!(sh->scale > 0.f) || !isfinite(sh->scale))
        return fail(MSA_ERR_INVALID, "scale must be finite and > 0");
    return MSA_OK;
}

// Returns MSA_OK with *empty set when there is nothing to do.
int check_batch(const msa_batch *b, const msa_shape *sh, bool *empty) {
    if (!b) return fail(MSA_ERR_INVALID, "batch is NULL");
    if (b->n_seqs < 0 || b->total_rows < 0 || b->max_rows < 0 || b->max_seq_len < 0)
        return fail(MSA_ERR_INVALID, "negative batch size field");
    *empty = b->n_seqs == 0;
    if (*empty) {
        if (b->total_rows != 0) return fail(MSA_ERR_INVALID, "n_seqs=0 but total_rows=%d", b->total_rows);
        return MSA_OK;
    }
    if (!b->cu_rows || !b->seq_lens || (!b->kv_start && !b->page_table))
        return fail(MSA_ERR_INVALID, "batch device arrays must not be NULL");
    if (b->page_table && (int64_t)b->pages_per_seq * msa::kBlock < b->max_seq_len)
        return fail(MSA_ERR_INVALID, "pages_per_seq=%d covers fewer than max_seq_len=%d keys", b->pages_per_seq,
                    b->max_seq_len);
    if (b->max_rows < 1 || b->max_seq_len < 1 || b->total_rows < b->n_seqs)
        return fail(MSA_ERR_INVALID, "every sequence needs >= 1 row and >= 1 key");
    if (b->max_rows > b->max_seq_len)
        return fail(MSA_ERR_INVALID, "max_rows=%d > max_seq_len=%d", b->max_rows, b->max_seq_len);
    if ((int64_t)b->max_rows * b->n_seqs < b->total_rows)
        return fail(MSA_ERR_INVALID, "total_rows exceeds n_seqs * max_rows");
    if ((int64_t)b->n_seqs * sh->n_kv_heads > 65535)
        return fail(MSA_ERR_UNSUPPORTED, "n_seqs * n_kv_heads > 65535");
    if ((int64_t)b->total_rows * sh->n_kv_heads * 8 > 0x7fffffffLL)
        return fail(MSA_ERR_UNSUPPORTED, "total_rows * n_kv_heads too large for one launch");
    return MSA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MSA_ERR_HIP, "no usable HIP device: %s", hipGetErrorString(e));
    return MSA_OK;
}

msa::BatchDev to_dev(const msa_batch *b) {
    msa::BatchDev d;
    d.n_seqs = b->n_seqs;
    d.total_rows = b->total_rows;
    d.max_rows = b->max_rows;
    d.max_seq_len = b->max_seq_len;
    d.cu_rows = b->cu_rows;
    d.seq_lens = b->seq_lens;
    d.kv_start = b->kv_start;
    d.page_table = b->page_table;
    d.pages_per_seq = b->page_table ? b->pages_per_seq : 0;
    return d;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MSA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

int check_kv(const void *k, const void *v, int64_t tok, int64_t head, int n_kv_heads) {
    if (!k || !v) return fail(MSA_ERR_INVALID, "k/v must not be NULL");
    if (tok < msa::kHeadDim || head < 0 || (n_kv_heads > 1 && head < msa::kHeadDim))
        return fail(MSA_ERR_INVALID, "kv strides (%lld, %lld) overlap a %d-element row",
                    (long long)tok, (long long)head, msa::kHeadDim);
    if (!aligned16(k) || !aligned16(v) || (tok * 2) % 16 || (head * 2) % 16)
        return fail(MSA_ERR_INVALID, "k/v rows must be 16-byte aligned");
    if (tok > msa::kMaxKvTokStride)   // the kernels address 32 tokens with 32-bit offsets
        return fail(MSA_ERR_UNSUPPORTED, "kv token stride %lld above %lld elements", (long long)tok,
                    (long long)msa::kMaxKvTokStride);
    return MSA_OK;
}

}  // namespace

extern "C" {

const char *msa_version(void) { return "msa-mi355x 0.2 (gfx950)"; }

const char *msa_last_error(void) { return g_last_error; }

const char *msa_status_string(int status) {
    switch (status) {
        case MSA_OK: return "ok";
        case MSA_ERR_INVALID: return "invalid argument";
        case MSA_ERR_UNSUPPORTED: return "unsupported shape";
        case MSA_ERR_WORKSPACE: return "workspace too small";
        case MSA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int msa_index_scores(const msa_shape *shape, const msa_batch *batch, const void *iq, const void *ik,
                     int64_t ik_tok_stride, int64_t ik_head_stride, float *block_scores,
                     int32_t bs_stride, void *stream) {
    int rc;
    bool empty;
    if ((rc = check_shape(shape)) || (rc = check_batch(batch, shape, &empty))) return rc;
    if (empty) return ok();
    if (!iq || !ik || !block_scores) return fail(MSA_ERR_INVALID, "iq/ik/block_scores must not be NULL");
    if (ik_tok_stride < msa::kIndexDim || ik_head_stride < 0 ||
        (ik_head_stride > 0 && ik_head_stride < msa::kIndexDim))
        return fail(MSA_ERR_INVALID, "ik strides (%lld, %lld) overlap a %d-element row",
                    (long long)ik_tok_stride, (long long)ik_head_stride, msa::kIndexDim);
    if (!aligned16(iq) || !aligned16(ik) || (ik_tok_stride * 2) % 16 || (ik_head_stride * 2) % 16)
        return fail(MSA_ERR_INVALID, "iq/ik rows must be 16-byte aligned");
    const int64_t need = ((int64_t)batch->max_seq_len + msa::kBlock - 1) / msa::kBlock;
    if (bs_stride < need)
        return fail(MSA_ERR_INVALID, "bs_stride=%d < ceil(max_seq_len/64)=%lld", bs_stride, (long long)need);
    if ((rc = check_device())) return rc;
    msa::IndexArgs a;
    a.b = to_dev(batch);
    a.H = shape->n_kv_heads;
    a.iq = static_cast<const uint16_t *>(iq);
    a.ik = static_cast<const uint16_t *>(ik);
    a.ik_tok = ik_tok_stride;
    a.ik_head = ik_head_stride;
    a.scores = block_scores;
    a.bs_stride = bs_stride;
    return launched(msa::launch_index_scores(a, static_cast<hipStream_t>(stream)), "index_scores");
}

int msa_select_blocks(const msa_shape *shape, const msa_batch *batch, const float *block_scores,
                      int32_t bs_stride, int32_t *block_idx, void *stream) {
    int rc;
    bool empty;
    if ((rc = check_shape(shape)) || (rc = check_batch(batch, shape, &empty))) return rc;
    if (empty) return ok();
    if (!block_scores || !block_idx) return fail(MSA_ERR_INVALID, "block_scores/block_idx must not be NULL");
    const int64_t need = ((int64_t)batch->max_seq_len + msa::kBlock - 1) / msa::kBlock;
    if (bs_stride < need)
        return fail(MSA_ERR_INVALID, "bs_stride=%d < ceil(max_seq_len/64)=%lld", bs_stride, (long long)need);
    if (need > msa::kMaxSelectBlocks)
        return fail(MSA_ERR_UNSUPPORTED, "max_seq_len=%d: selection supports at most %d blocks (%d keys)",
                    batch->max_seq_len, msa::kMaxSelectBlocks, msa::kMaxSelectBlocks * msa::kBlock);
    if ((rc = check_device())) return rc;
    msa::SelectArgs a;
    a.b = to_dev(batch);
    a.H = shape->n_kv_heads;
    a.top_k = shape->top_k;
    a.scores = block_scores;
    a.bs_stride = bs_stride;
    a.idx = block_idx;
    return launched(msa::launch_select_blocks(a, static_cast<hipStream_t>(stream)), "select_blocks");
}

size_t msa_index_select_workspace_bytes(const msa_shape *shape, const msa_batch *batch) {
    bool empty = false;
    if (!shape || check_shape(shape) || check_batch(batch, shape, &empty)) return 0;
    if (empty) return msa::kIndexSelectCountBytes;
    return msa::index_select_workspace_bytes(batch->n_seqs, shape->n_kv_heads, batch->total_rows, batch->max_rows,
                                             batch->max_seq_len, shape->top_k);
}

}  // extern "C"

// msa_index_select, and msa_index_select_pack_rows with pk = its batch writer
// (checked by the caller): decode-shaped launches carry the writer's
// workgroups, the others launch it first.
static int index_select_impl(const msa_shape *shape, const msa_batch *batch, const void *iq, const void *ik,
                             int64_t ik_tok_stride, int64_t ik_head_stride, float *block_scores, int32_t bs_stride,
                             int32_t *block_idx, void *workspace, size_t workspace_bytes,
                             const msa::PackRowsArgs *pk, void *stream) {
    int rc;
    bool empty;
    if ((rc = check_shape(shape)) || (rc = check_batch(batch, shape, &empty))) return rc;
    if (empty) return ok();
    if (!iq || !ik || !block_idx) return fail(MSA_ERR_INVALID, "iq/ik/block_idx must not be NULL");
    if (ik_tok_stride < msa::kIndexDim || ik_head_stride < 0 ||
        (ik_head_stride > 0 && ik_head_stride < msa::kIndexDim))
        return fail(MSA_ERR_INVALID, "ik strides (%lld, %lld) overlap a %d-element row",
                    (long long)ik_tok_stride, (long long)ik_head_stride, msa::kIndexDim);
    if (!aligned16(iq) || !aligned16(ik) || (ik_tok_stride * 2) % 16 || (ik_head_stride * 2) % 16)
        return fail(MSA_ERR_INVALID, "iq/ik rows must be 16-byte aligned");
    const int H = shape->n_kv_heads;
    // NULL block_scores: the prompt-chunk kernel, whose scores never reach memory
    const bool chunk = !block_scores;
    if (chunk && !msa::chunk_select_eligible(batch->n_seqs, H, batch->max_rows, shape->top_k))
        return fail(MSA_ERR_INVALID, "block_scores may be NULL only for batches with more than 16 rows in a "
                    "sequence, top_k <= %d and at most %lld (sequence, key head, 256-row tile) units",
                    msa::kChunkMaxTopK, (long long)msa::kIndexSelectCounters);
    const int64_t need = ((int64_t)batch->max_seq_len + msa::kBlock - 1) / msa::kBlock;
    if (!chunk && bs_stride < need)
        return fail(MSA_ERR_INVALID, "bs_stride=%d < ceil(max_seq_len/64)=%lld", bs_stride, (long long)need);
    if (!chunk && need > msa::kMaxSelectBlocks)
        return fail(MSA_ERR_UNSUPPORTED, "max_seq_len=%d: selection supports at most %d blocks (%d keys)",
                    batch->max_seq_len, msa::kMaxSelectBlocks, msa::kMaxSelectBlocks * msa::kBlock);
    const size_t ws_need = msa::index_select_workspace_bytes(batch->n_seqs, H, batch->total_rows,
                                                             batch->max_rows, batch->max_seq_len, shape->top_k);
    if (!workspace || workspace_bytes < ws_need)
        return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, ws_need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(MSA_ERR_INVALID, "workspace must be 256-byte aligned");
    if ((rc = check_device())) return rc;
    msa::IndexArgs a;
    a.b = to_dev(batch);
    a.H = H;
    a.iq = static_cast<const uint16_t *>(iq);
    a.ik = static_cast<const uint16_t *>(ik);
    a.ik_tok = ik_tok_stride;
    a.ik_head = ik_head_stride;
    a.scores = block_scores;
    a.bs_stride = bs_stride;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (chunk) {
        msa::ChunkSelect c{};
        c.top_k = shape->top_k;
        c.idx = block_idx;
        c.count = static_cast<unsigned *>(workspace);
        c.cand = reinterpret_cast<uint64_t *>(static_cast<uint8_t *>(workspace) + msa::kIndexSelectCountBytes);
        c.tiles = msa::chunk_tiles(batch->max_rows);
        msa::chunk_splits(batch->n_seqs, H, batch->max_rows, batch->max_seq_len, &c.splits, &c.per_split);
        if (pk && (rc = launched(msa::launch_pack_kv_rows(*pk, st), "pack_kv_tiled_rows"))) return rc;
        return launched(msa::launch_index_select_chunk(a, c, st), "index_select_chunk");
    }
    if (batch->max_rows > 1) {
        // Several rows per sequence: the last workgroup would select them one
        // after another, which costs more than a second launch that selects
        // every (row, key head) in parallel.
        if ((rc = launched(msa::launch_index_scores(a, st, pk), "index_scores"))) return rc;
        msa::SelectArgs s;
        s.b = a.b;
        s.H = a.H;
        s.top_k = shape->top_k;
        s.scores = block_scores;
        s.bs_stride = bs_stride;
        s.idx = block_idx;
        return launched(msa::launch_select_blocks(s, st), "select_blocks");
    }
    msa::SelectTail t{};
    t.top_k = shape->top_k;
    t.idx = block_idx;
    t.count = static_cast<unsigned *>(workspace);
    t.wmax = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + msa::kIndexSelectCountBytes);
    t.ranges = msa::window_ranges(batch->max_seq_len);
    return launched(msa::launch_index_select(a, t, st, pk), "index_select");
}

extern "C" {

int msa_index_select(const msa_shape *shape, const msa_batch *batch, const void *iq, const void *ik,
                     int64_t ik_tok_stride, int64_t ik_head_stride, float *block_scores, int32_t bs_stride,
                     int32_t *block_idx, void *workspace, size_t workspace_bytes, void *stream) {
    return index_select_impl(shape, batch, iq, ik, ik_tok_stride, ik_head_stride, block_scores, bs_stride,
                             block_idx, workspace, workspace_bytes, nullptr, stream);
}

static int check_kv8(const msa_kv8 *kv, int n_kv_heads) {
    if (!kv) return fail(MSA_ERR_INVALID, "kv is NULL");
    if (!kv->k || !kv->v || !kv->k_scale || !kv->v_scale)
        return fail(MSA_ERR_INVALID, "int8 cache codes and scales must not be NULL");
    if (kv->tok_stride < msa::kHeadDim || kv->head_stride < 0 ||
        (n_kv_heads > 1 && kv->head_stride < msa::kHeadDim))
        return fail(MSA_ERR_INVALID, "code strides (%lld, %lld) overlap a %d-element row",
                    (long long)kv->tok_stride, (long long)kv->head_stride, msa::kHeadDim);
    if (!aligned16(kv->k) || !aligned16(kv->v) || kv->tok_stride % 16 || kv->head_stride % 16)
        return fail(MSA_ERR_INVALID, "int8 code rows must be 16-byte aligned");
    if (kv->tok_stride > msa::kMaxKvTokStride)
        return fail(MSA_ERR_UNSUPPORTED, "kv token stride %lld above %lld elements", (long long)kv->tok_stride,
                    (long long)msa::kMaxKvTokStride);
    if (kv->scale_tok_stride < 1 || kv->scale_head_stride < 0 || (n_kv_heads > 1 && kv->scale_head_stride < 1) ||
        ((uintptr_t)kv->k_scale & 3u) || ((uintptr_t)kv->v_scale & 3u))
        return fail(MSA_ERR_INVALID, "scale strides (%lld, %lld) or scale alignment invalid",
                    (long long)kv->scale_tok_stride, (long long)kv->scale_head_stride);
    return MSA_OK;
}

static int attn_common(const msa_shape *shape, const msa_batch *batch, const void *q, const void *k,
                       const void *v, int64_t kv_tok_stride, int64_t kv_head_stride,
                       const int32_t *block_idx, void *out, float *lse, msa::AttnArgs *a, bool *empty,
                       const msa_kv8 *kv8 = nullptr) {
    int rc;
    if ((rc = check_shape(shape)) || (rc = check_batch(batch, shape, empty))) return rc;
    if (*empty) return MSA_OK;
    if (!q || !block_idx || !out) return fail(MSA_ERR_INVALID, "q/block_idx/out must not be NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(MSA_ERR_INVALID, "q/out must be 16-byte aligned");
    if (kv8) {
        if ((rc = check_kv8(kv8, shape->n_kv_heads))) return rc;
        kv_tok_stride = kv8->tok_stride;
        kv_head_stride = kv8->head_stride;
    } else if ((rc = check_kv(k, v, kv_tok_stride, kv_head_stride, shape->n_kv_heads))) {
        return rc;
    }
    a->b = to_dev(batch);
    a->H = shape->n_kv_heads;
    a->top_k = shape->top_k;
    a->scale_log2 = shape->scale * msa::kLog2e;
    a->q = static_cast<const uint16_t *>(q);
    a->k = static_cast<const uint16_t *>(k);
    a->v = static_cast<const uint16_t *>(v);
    a->kv_tok = kv_tok_stride;
    a->kv_head = kv_head_stride;
    a->idx = block_idx;
    a->out = static_cast<uint16_t *>(out);
    a->lse = lse;
    a->ws_count = nullptr;
    a->ws_part = nullptr;
    a->k8 = kv8 ? kv8->k : nullptr;
    a->v8 = kv8 ? kv8->v : nullptr;
    a->ks = kv8 ? kv8->k_scale : nullptr;
    a->vs = kv8 ? kv8->v_scale : nullptr;
    a->s_tok = kv8 ? kv8->scale_tok_stride : 0;
    a->s_head = kv8 ? kv8->scale_head_stride : 0;
    a->tiled = false;
    return MSA_OK;
}

int msa_prefill(const msa_shape *shape, const msa_batch *batch, const void *q, const void *k,
                const void *v, int64_t kv_tok_stride, int64_t kv_head_stride, const int32_t *block_idx,
                void *out, float *lse, void *stream) {
    msa::AttnArgs a;
    bool empty = false;
    int rc = attn_common(shape, batch, q, k, v, kv_tok_stride, kv_head_stride, block_idx, out, lse, &a,
                         &empty);
    if (rc) return rc;
    if (empty) return ok();
    if ((rc = check_device())) return rc;
    return launched(msa::launch_prefill(a, static_cast<hipStream_t>(stream)), "prefill");
}

size_t msa_decode_workspace_bytes(const msa_shape *shape, int32_t total_rows) {
    if (!shape || check_shape(shape) || total_rows < 0) return 0;
    return msa::decode_workspace_bytes((int64_t)total_rows * shape->n_kv_heads, shape->top_k);
}

// Workspace checks and the decode launch, for arguments attn_common accepted.
static int decode_launch(msa::AttnArgs &a, const msa_batch *batch, const msa_shape *shape, void *workspace,
                         size_t workspace_bytes, void *stream) {
    int rc;
    const int64_t units = (int64_t)batch->total_rows * shape->n_kv_heads;
    const size_t need = msa::decode_workspace_bytes(units, shape->top_k);
    if (!workspace || workspace_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(MSA_ERR_INVALID, "workspace must be 256-byte aligned");
    if ((rc = check_device())) return rc;
    a.ws_count = static_cast<unsigned *>(workspace);
    a.ws_part = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + msa::kDecodeCountBytes);
    return launched(msa::launch_decode(a, static_cast<hipStream_t>(stream)), "decode");
}

static int decode_common(const msa_shape *shape, const msa_batch *batch, const void *q, const void *k,
                         const void *v, int64_t kv_tok_stride, int64_t kv_head_stride, const int32_t *block_idx,
                         void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream,
                         const msa_kv8 *kv8) {
    msa::AttnArgs a;
    bool empty = false;
    int rc = attn_common(shape, batch, q, k, v, kv_tok_stride, kv_head_stride, block_idx, out, lse, &a,
                         &empty, kv8);
    if (rc) return rc;
    if (empty) return ok();
    return decode_launch(a, batch, shape, workspace, workspace_bytes, stream);
}

int msa_decode(const msa_shape *shape, const msa_batch *batch, const void *q, const void *k,
               const void *v, int64_t kv_tok_stride, int64_t kv_head_stride, const int32_t *block_idx,
               void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    return decode_common(shape, batch, q, k, v, kv_tok_stride, kv_head_stride, block_idx, out, lse, workspace,
                         workspace_bytes, stream, nullptr);
}

int msa_decode_kv8(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv8 *kv,
                   const int32_t *block_idx, void *out, float *lse, void *workspace, size_t workspace_bytes,
                   void *stream) {
    if (!kv) return fail(MSA_ERR_INVALID, "kv is NULL");
    return decode_common(shape, batch, q, nullptr, nullptr, 0, 0, block_idx, out, lse, workspace,
                         workspace_bytes, stream, kv);
}

int msa_prefill_kv8(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv8 *kv,
                    const int32_t *block_idx, void *out, float *lse, void *stream) {
    msa::AttnArgs a;
    bool empty = false;
    if (!kv) return fail(MSA_ERR_INVALID, "kv is NULL");
    int rc = attn_common(shape, batch, q, nullptr, nullptr, 0, 0, block_idx, out, lse, &a, &empty, kv);
    if (rc) return rc;
    if (empty) return ok();
    if ((rc = check_device())) return rc;
    return launched(msa::launch_prefill(a, static_cast<hipStream_t>(stream)), "prefill_kv8");
}

static int check_tiles(const void *k, const void *v, int64_t block_stride, int64_t head_stride, int n_kv_heads) {
    if (!k || !v) return fail(MSA_ERR_INVALID, "k/v tiles must not be NULL");
    if (!aligned16(k) || !aligned16(v) || block_stride % 8 || head_stride % 8)
        return fail(MSA_ERR_INVALID, "tiles must be 16-byte aligned");
    if (block_stride < msa::kTileElems || head_stride < 0 || (n_kv_heads > 1 && head_stride < msa::kTileElems))
        return fail(MSA_ERR_INVALID, "tile strides (%lld, %lld) overlap a %d-element tile", (long long)block_stride,
                    (long long)head_stride, msa::kTileElems);
    return MSA_OK;
}

static int tiled_common(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv_tiled *kv,
                        const int32_t *block_idx, void *out, float *lse, msa::AttnArgs *a, bool *empty) {
    int rc;
    if (!kv) return fail(MSA_ERR_INVALID, "kv is NULL");
    if ((rc = check_shape(shape))) return rc;
    if ((rc = check_tiles(kv->k, kv->v, kv->block_stride, kv->head_stride, shape->n_kv_heads))) return rc;
    // the strided checks do not apply to tile strides: give attn_common a
    // valid strided description, then replace it with the tiles
    if ((rc = attn_common(shape, batch, q, kv->k, kv->v, msa::kHeadDim * shape->n_kv_heads, msa::kHeadDim,
                          block_idx, out, lse, a, empty)))
        return rc;
    a->kv_tok = kv->block_stride;
    a->kv_head = kv->head_stride;
    a->tiled = true;
    return MSA_OK;
}

int msa_prefill_tiled(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv_tiled *kv,
                      const int32_t *block_idx, void *out, float *lse, void *stream) {
    msa::AttnArgs a;
    bool empty = false;
    int rc = tiled_common(shape, batch, q, kv, block_idx, out, lse, &a, &empty);
    if (rc) return rc;
    if (empty) return ok();
    if ((rc = check_device())) return rc;
    return launched(msa::launch_prefill(a, static_cast<hipStream_t>(stream)), "prefill_tiled");
}

int msa_decode_tiled(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv_tiled *kv,
                     const int32_t *block_idx, void *out, float *lse, void *workspace, size_t workspace_bytes,
                     void *stream) {
    msa::AttnArgs a;
    bool empty = false;
    int rc = tiled_common(shape, batch, q, kv, block_idx, out, lse, &a, &empty);
    if (rc) return rc;
    if (empty) return ok();
    return decode_launch(a, batch, shape, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- msa_decode_tiled_noalloc: the decode workspace in a static device array ----
//
// `scratch` is this library's decode workspace for callers that cannot
// allocate: one copy per device, held until the process ends.  In host code
// its name is only a stand-in for the symbol; the device address of each
// GPU's copy comes from hipGetSymbolAddress on that device (first call there)
// and is the only thing ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[MSA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[kMaxScratchDevices];     // device address of `scratch` per device
bool g_scratch_clean[kMaxScratchDevices];       // its counters are known to be zero

__global__ void zero_words(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The current device's scratch address (looked up once per device); on the
// first call there, or after a failed launch, its counters are cleared on
// `st` first by a fill kernel (not a memset, so the call can be captured).
int scratch_for_call(hipStream_t st, uint8_t **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MSA_ERR_HIP, "no usable HIP device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(MSA_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<uint8_t *>(ptr);
        g_scratch_clean[dev] = false;
    }
    if (!g_scratch_clean[dev]) {
        constexpr int n = (int)(msa::kDecodeCountBytes / 4);
        hipLaunchKernelGGL(zero_words, dim3(1), dim3(n), 0, st, reinterpret_cast<uint32_t *>(g_scratch_ptr[dev]), n);
        if ((e = hipGetLastError()) != hipSuccess)
            return fail(MSA_ERR_HIP, "clearing the static workspace failed: %s", hipGetErrorString(e));
        g_scratch_clean[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return MSA_OK;
}

void scratch_mark_dirty() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch_clean[dev] = false;
}

}  // namespace

extern "C" {

int msa_decode_tiled_noalloc(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv_tiled *kv,
                             const int32_t *block_idx, void *out, float *lse, void *stream) {
    static_assert(MSA_DECODE_NOALLOC_SCRATCH_BYTES >= msa::kDecodeCountBytes, "scratch below its counters");
    msa::AttnArgs a;
    bool empty = false;
    int rc = tiled_common(shape, batch, q, kv, block_idx, out, lse, &a, &empty);
    if (rc) return rc;
    if (empty) return ok();
    const int64_t units = (int64_t)batch->total_rows * shape->n_kv_heads;
    const size_t need = msa::decode_workspace_bytes(units, shape->top_k);
    if (need > MSA_DECODE_NOALLOC_SCRATCH_BYTES)
        return fail(MSA_ERR_WORKSPACE, "batch needs %zu bytes of decode workspace, above the %zu-byte static one",
                    need, (size_t)MSA_DECODE_NOALLOC_SCRATCH_BYTES);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *ws = nullptr;
    if ((rc = scratch_for_call(st, &ws))) return rc;
    a.ws_count = reinterpret_cast<unsigned *>(ws);
    a.ws_part = reinterpret_cast<float *>(ws + msa::kDecodeCountBytes);
    rc = launched(msa::launch_decode(a, st), "decode_tiled_noalloc");
    if (rc) scratch_mark_dirty();
    return rc;
}

int msa_pack_kv_tiled(const msa_shape *shape, int64_t tok_begin, int64_t tok_end, const void *k, const void *v,
                      int64_t kv_tok_stride, int64_t kv_head_stride, void *k_tiles, void *v_tiles,
                      int64_t block_stride, int64_t head_stride, void *stream) {
    int rc;
    if ((rc = check_shape(shape))) return rc;
    if (tok_begin < 0 || tok_end <= tok_begin)
        return fail(MSA_ERR_INVALID, "token range [%lld, %lld) is empty or negative", (long long)tok_begin,
                    (long long)tok_end);
    const int H = shape->n_kv_heads;
    if ((rc = check_kv(k, v, kv_tok_stride, kv_head_stride, H))) return rc;
    if ((rc = check_tiles(k_tiles, v_tiles, block_stride, head_stride, H))) return rc;
    msa::PackTiledArgs a;
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.tok = kv_tok_stride;
    a.head = kv_head_stride;
    a.kt = static_cast<uint16_t *>(k_tiles);
    a.vt = static_cast<uint16_t *>(v_tiles);
    a.t_blk = block_stride;
    a.t_head = head_stride;
    a.tok_begin = tok_begin;
    a.tok_end = tok_end;
    a.n_blocks = (tok_end - 1) / 64 - tok_begin / 64 + 1;
    a.H = H;
    if (a.n_blocks * H * 2 > (int64_t)0x7fffffff)
        return fail(MSA_ERR_UNSUPPORTED, "token range too large for one call");
    if ((rc = check_device())) return rc;
    return launched(msa::launch_pack_kv_tiled(a, static_cast<hipStream_t>(stream)), "pack_kv_tiled");
}

int msa_pack_kv_tiled_rows(const msa_shape *shape, const msa_batch *batch, const void *k, const void *v,
                           int64_t kv_tok_stride, int64_t kv_head_stride, void *k_tiles, void *v_tiles,
                           int64_t block_stride, int64_t head_stride, void *stream) {
    int rc;
    bool empty = false;
    if ((rc = check_shape(shape)) || (rc = check_batch(batch, shape, &empty))) return rc;
    if (empty) return ok();
    const int H = shape->n_kv_heads;
    if ((rc = check_kv(k, v, kv_tok_stride, kv_head_stride, H))) return rc;
    if ((rc = check_tiles(k_tiles, v_tiles, block_stride, head_stride, H))) return rc;
    if ((int64_t)batch->total_rows * H * 64 / 256 > (int64_t)0x7fffffff)
        return fail(MSA_ERR_UNSUPPORTED, "batch too large for one call");
    if ((rc = check_device())) return rc;
    msa::PackRowsArgs a;
    a.b = to_dev(batch);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.tok = kv_tok_stride;
    a.head = kv_head_stride;
    a.kt = static_cast<uint16_t *>(k_tiles);
    a.vt = static_cast<uint16_t *>(v_tiles);
    a.t_blk = block_stride;
    a.t_head = head_stride;
    a.H = H;
    return launched(msa::launch_pack_kv_rows(a, static_cast<hipStream_t>(stream)), "pack_kv_tiled_rows");
}

int msa_index_select_pack_rows(const msa_shape *shape, const msa_batch *batch, const void *iq, const void *ik,
                               int64_t ik_tok_stride, int64_t ik_head_stride, float *block_scores,
                               int32_t bs_stride, int32_t *block_idx, void *workspace, size_t workspace_bytes,
                               const void *k, const void *v, int64_t kv_tok_stride, int64_t kv_head_stride,
                               void *k_tiles, void *v_tiles, int64_t block_stride, int64_t head_stride,
                               void *stream) {
    int rc;
    bool empty = false;
    if ((rc = check_shape(shape)) || (rc = check_batch(batch, shape, &empty))) return rc;
    if (empty) return ok();
    const int H = shape->n_kv_heads;
    if ((rc = check_kv(k, v, kv_tok_stride, kv_head_stride, H))) return rc;
    if ((rc = check_tiles(k_tiles, v_tiles, block_stride, head_stride, H))) return rc;
    if ((int64_t)batch->total_rows * H * 64 / 256 > (int64_t)0x7fffffff)
        return fail(MSA_ERR_UNSUPPORTED, "batch too large for one call");
    msa::PackRowsArgs p;
    p.b = to_dev(batch);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.tok = kv_tok_stride;
    p.head = kv_head_stride;
    p.kt = static_cast<uint16_t *>(k_tiles);
    p.vt = static_cast<uint16_t *>(v_tiles);
    p.t_blk = block_stride;
    p.t_head = head_stride;
    p.H = H;
    return index_select_impl(shape, batch, iq, ik, ik_tok_stride, ik_head_stride, block_scores, bs_stride,
                             block_idx, workspace, workspace_bytes, &p, stream);
}

int msa_quantize_kv8(const msa_shape *shape, int64_t n_tokens, const void *x, int64_t tok_stride,
                     int64_t head_stride, int8_t *codes, int64_t code_tok_stride, int64_t code_head_stride,
                     float *scales, int64_t scale_tok_stride, int64_t scale_head_stride, void *stream) {
    int rc;
    if ((rc = check_shape(shape))) return rc;
    if (n_tokens < 0) return fail(MSA_ERR_INVALID, "n_tokens < 0");
    if (n_tokens == 0) return ok();
    const int H = shape->n_kv_heads;
    if (!x || !codes || !scales) return fail(MSA_ERR_INVALID, "x/codes/scales must not be NULL");
    if ((rc = check_kv(x, x, tok_stride, head_stride, H))) return rc;
    msa_kv8 kv = {codes, codes, scales, scales, code_tok_stride, code_head_stride, scale_tok_stride,
                  scale_head_stride};
    if ((rc = check_kv8(&kv, H))) return rc;
    if (n_tokens * H > (int64_t)0x7fffffff / 16) return fail(MSA_ERR_UNSUPPORTED, "n_tokens * n_kv_heads too large");
    if ((rc = check_device())) return rc;
    msa::QuantArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.tok = tok_stride;
    a.head = head_stride;
    a.codes = codes;
    a.ctok = code_tok_stride;
    a.chead = code_head_stride;
    a.scales = scales;
    a.stok = scale_tok_stride;
    a.shead = scale_head_stride;
    a.n_tokens = n_tokens;
    a.H = H;
    return launched(msa::launch_quantize_kv8(a, static_cast<hipStream_t>(stream)), "quantize_kv8");
}

}  // extern "C"
