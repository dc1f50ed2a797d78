/*
 * msa.h -- C ABI of the MI355X (gfx950) MiniMax-M3 block-sparse attention
 * (MSA) library, libmsa.so.
 *
 * The method, as the pages describe it in prose (no formulas are given):
 *   - "minimax-m3-sm120" README, section "What this fixes": the MSA model
 *     selects the top-16 blocks per GQA group, scores blocks by max-pooling
 *     and always keeps the local block.
 *   - TensorFold pull request 1388, commit adding the minimax_m3 family: the
 *     lightning indexer produces index scores and a top-16 block selection
 *     per row and key head; decode attends over the kept blocks in 32-key
 *     partials; prompt chunks attend over each tile's kept blocks.
 *   - same pull request, commit on 4,096-row prompt chunks: the 16 query heads
 *     of one key head share that key head's selection, so one fetch of a kept
 *     key/value block serves all sixteen.
 *
 * Notation.  A ragged batch holds n_seqs sequences.  Sequence s has
 * seq_lens[s] keys (every key visible to its last row, the rows' own keys
 * included) and rows_s = cu_rows[s+1] - cu_rows[s] query rows, which are its
 * LAST rows_s positions: row i sits at p = seq_lens[s] - rows_s + i.  Key j of
 * the sequence (0-based) lives at token kv_start[s] + j of the key tensors and
 * is visible to the row at p iff j <= p.
 *
 * Paged layout (page_table != NULL): the key tensors k, v and ik are pools of
 * pages of `block` tokens -- a page is exactly one sparse block -- and key j
 * of sequence s lives at token page_table[s * pages_per_seq + j / block] *
 * block + j % block.  Sequences may share pages (a cached prompt prefix is
 * stored once and referenced by every sequence that extends it; prompt chunks
 * resume on top of it).  The page table is a precondition like cu_rows: every
 * entry a sequence's keys reach must name a page inside the pools.
 * (Serving stacks on the pages share one longest-prefix KV cache between
 * requests -- "minimax-rs", API section -- keep the prompt cache on by default
 * -- "minimax3-on-2-nodes", Performance & tuning -- and keep prompt-cache
 * snapshots at chunk starts -- TensorFold pull request 1388, commit adding the
 * minimax_m3 family.  Pages of one sparse block are this library's layout for
 * that reuse.)  Blocks are `block` consecutive keys;
 * the row's causal block count is nb = floor(p / block) + 1 and its local
 * block is nb - 1.  Query head h belongs to key head floor(h / group).
 *
 * Steps (one entry point each, enqueued on the caller's stream):
 *   msa_index_scores  S[r,g,b] = max_{j in block b, j <= p} sum_d iq[r,g,d]*ik[j,g,d]
 *   msa_select_blocks the local block + the top_k-1 best other blocks by S
 *                     (ties: lower block index), ascending, -1 padded
 *   msa_prefill       exact softmax attention of the group's query heads over
 *                     the kept blocks' visible keys (one pass per row)
 *   msa_decode        the same result, split into 32-key partials that are
 *                     merged with a log-sum-exp combine (for few rows)
 *
 * Dtypes: bf16 tensors are passed as raw 16-bit patterns (void*); scores and
 * lse are fp32; indices int32.  Every pointer argument is DEVICE memory unless
 * marked host.  Element strides are in elements, not bytes.
 *
 * Ownership and threading: the caller allocates and owns every buffer,
 * including the decode workspace.  The library allocates nothing, keeps no
 * state between calls (msa_decode_tiled_noalloc's static workspace, below, is
 * the one exception), never synchronises the device and only enqueues work
 * on `stream` (a hipStream_t; NULL is the default stream).  Calls are
 * thread-safe.
 *
 * Errors: all host-visible arguments are validated before anything is
 * enqueued; a failure returns a negative msa_status, enqueues nothing and sets
 * the calling thread's msa_last_error() text.  A launch failure returns
 * MSA_ERR_HIP.  Device-array contents are preconditions and are not checked
 * on the host: 1 <= rows_s <= seq_lens[s] <= max_seq_len, rows_s <= max_rows,
 * cu_rows non-decreasing with cu_rows[n_seqs] == total_rows, key ranges in
 * bounds of the key tensors, and block_idx entries either -1 or a causal block
 * of their row.  Kernels skip (do not fault on) rows and blocks that violate
 * the row/length preconditions; their outputs are then unspecified.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msa_status {
    MSA_OK = 0,
    MSA_ERR_INVALID = -1,      /* null pointer, negative size, inconsistent sizes */
    MSA_ERR_UNSUPPORTED = -2,  /* a shape the library has no kernel for */
    MSA_ERR_WORKSPACE = -3,    /* decode workspace missing or too small */
    MSA_ERR_HIP = -4           /* HIP runtime error (no device, launch failure) */
} msa_status;

/* Fixed per-model shape.  Supported: group 16, head_dim 128, index_dim 64,
 * block 64, 1 <= top_k <= 32, n_kv_heads >= 1, scale finite and > 0. */
typedef struct msa_shape {
    int32_t n_kv_heads;   /* H_kv: key heads (query heads = H_kv * group) */
    int32_t group;        /* query heads per key head */
    int32_t head_dim;     /* D of q, k, v */
    int32_t index_dim;    /* d_I of iq, ik */
    int32_t block;        /* keys per block */
    int32_t top_k;        /* blocks kept per (row, key head), local block included */
    float scale;          /* softmax scale applied to q.k (1/sqrt(head_dim) usually) */
} msa_shape;

/* Ragged batch.  The four integers are host values; the arrays are device
 * arrays.  No device-to-host copy is ever made. */
typedef struct msa_batch {
    int32_t n_seqs;            /* >= 0; 0 means nothing to do */
    int32_t total_rows;        /* == cu_rows[n_seqs] */
    int32_t max_rows;          /* >= every rows_s */
    int32_t max_seq_len;       /* >= every seq_lens[s] */
    const int32_t *cu_rows;    /* device [n_seqs + 1], prefix sums of rows_s, cu_rows[0] = 0 */
    const int32_t *seq_lens;   /* device [n_seqs] */
    const int64_t *kv_start;   /* device [n_seqs], first token of each sequence in k/v/ik
                                  (contiguous layout; not read when page_table is set) */
    const int32_t *page_table; /* device [n_seqs, pages_per_seq] or NULL: paged layout, below */
    int32_t pages_per_seq;     /* row stride of page_table, >= ceil(max_seq_len / block) */
} msa_batch;

/*
 * Steps 1-2: lightning-indexer scores, max-pooled per block.
 *   iq           bf16 [total_rows, n_kv_heads, index_dim], contiguous
 *   ik           bf16, element (token t, key head g, dim d) at
 *                ik[t*ik_tok_stride + g*ik_head_stride + d]; the dim axis is
 *                contiguous; ik_head_stride == 0 means one index key shared by
 *                every key head.  Rows of 128 bytes must be 16-byte aligned.
 *   block_scores fp32 [total_rows, n_kv_heads, bs_stride], written in full:
 *                S[r,g,b] for b < nb(r), -INFINITY for nb(r) <= b < bs_stride.
 *   bs_stride    >= ceil(max_seq_len / block)
 * Cost: reads every causally visible index key once per row tile; the
 * contraction runs on bf16 MFMA with fp32 accumulation.
 */
int msa_index_scores(const msa_shape *shape, const msa_batch *batch,
                     const void *iq, const void *ik,
                     int64_t ik_tok_stride, int64_t ik_head_stride,
                     float *block_scores, int32_t bs_stride, void *stream);

/*
 * Step 3: per (row, key head), keep the local block and the top_k-1 highest
 * block scores among the earlier blocks; equal scores prefer the lower block
 * index (-0.0 and +0.0 are equal).  Rows with nb <= top_k keep blocks
 * 0..nb-1.  Output is ascending and padded with -1.
 *   block_scores fp32 [total_rows, n_kv_heads, bs_stride] (as written above)
 *   block_idx    int32 [total_rows, n_kv_heads, top_k]
 * Scores must not be NaN.  max_seq_len may be at most 1,048,576 keys (16,384
 * blocks; larger returns MSA_ERR_UNSUPPORTED): a row's scores are staged in
 * on-chip memory.
 */
int msa_select_blocks(const msa_shape *shape, const msa_batch *batch,
                      const float *block_scores, int32_t bs_stride,
                      int32_t *block_idx, void *stream);

/*
 * Steps 1-3 in one call: the index scores and max-pool of msa_index_scores,
 * then the selection of msa_select_blocks, with block_idx bit-identical to
 * those two calls.  The computation is the one of steps 1-3 (TensorFold pull
 * request 1388, commit adding the minimax_m3 family: index scores and a
 * top-16 block selection per row and key head); the pages keep the block
 * scores as a buffer of their own between the two steps (a later commit of
 * the same pull request shares its memory with other buffers, so that
 * 4,096-row chunks fit).  Doing both in one launch is this library's
 * addition.  Three cases:
 *   - block_scores == NULL (batches with more than 16 rows in a sequence and
 *     top_k <= 16: prompt chunks): one launch in which the scores never reach
 *     memory.  The candidate blocks of every (sequence, key head, 256-row
 *     tile) are split over a few workgroups; each keeps, per row, a sorted
 *     list of its 16 best (score, block) pairs, publishes it in `workspace`,
 *     and the last workgroup of the tile merges the lists (every kept block
 *     is in its own split's list with the same tie order) and writes the
 *     selection.
 *   - block_scores != NULL, one row per sequence (decode steps): one launch;
 *     the key axis of every (sequence, key head) is spread over many
 *     workgroups, the last of which (an arrival counter in `workspace`)
 *     selects the row from the scores, which it reads back while they are
 *     still in the caches.  block_scores is written as by msa_index_scores
 *     (it is the exchange buffer).
 *   - block_scores != NULL, several rows in a sequence: the two launches of
 *     msa_index_scores and msa_select_blocks (selecting the rows in parallel
 *     is faster than a last workgroup selecting them one by one).
 *   workspace   device, 256-byte aligned, msa_index_select_workspace_bytes()
 *               bytes for the batch: a fixed 256 KiB region of arrival
 *               counters, then (for batches the NULL-score case can take) the
 *               candidate lists, 128 bytes per (row, key head, split).  The
 *               counters must be zero before the first call (allocate it
 *               zeroed); every completed call leaves them zero, whatever the
 *               batch, so one workspace serves every batch it is large
 *               enough for.  Calls that share a workspace must not overlap in
 *               time.  Required (and checked) for every batch.
 * Errors: as msa_index_scores and msa_select_blocks; NULL block_scores for a
 * batch outside the first case -> MSA_ERR_INVALID; a missing or short
 * workspace -> MSA_ERR_WORKSPACE.  msa_index_select_workspace_bytes returns 0
 * for an invalid shape or batch (host fields only are read).
 */
size_t msa_index_select_workspace_bytes(const msa_shape *shape, const msa_batch *batch);
int msa_index_select(const msa_shape *shape, const msa_batch *batch,
                     const void *iq, const void *ik, int64_t ik_tok_stride, int64_t ik_head_stride,
                     float *block_scores, int32_t bs_stride, int32_t *block_idx,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Step 4 for prompt chunks: out[r, h, :] = softmax over the kept, visible keys
 * of scale * q[r,h,:].k[j,g,:], applied to v[j,g,:], g = h / group.  One pass
 * per row; the group's query heads share the row's selection, so one fetch of
 * a kept block serves every head of the group.  Keys are walked in ascending block
 * order, so a row's bits do not depend on the other rows in the batch.
 *   q, out    bf16 [total_rows, n_kv_heads*group, head_dim], contiguous
 *   k, v      bf16, element (token t, key head g, dim d) at
 *             k[t*kv_tok_stride + g*kv_head_stride + d]; 16-byte aligned rows;
 *             kv_tok_stride <= 2^24 elements (else MSA_ERR_UNSUPPORTED)
 *   block_idx int32 [total_rows, n_kv_heads, top_k] (from msa_select_blocks)
 *   lse       fp32 [total_rows, n_kv_heads*group] natural-log log-sum-exp of
 *             the scaled scores, or NULL.  A row with no kept visible key gets
 *             out = 0 and lse = -INFINITY.
 */
int msa_prefill(const msa_shape *shape, const msa_batch *batch,
                const void *q, const void *k, const void *v,
                int64_t kv_tok_stride, int64_t kv_head_stride,
                const int32_t *block_idx, void *out, float *lse, void *stream);

/*
 * int8 key/value cache (opt-in; it changes the arithmetic, so it is checked
 * against its own reference, not against the bf16 path).  Keys and values are
 * int8 codes with one fp32 scale per (token, key head): the element value is
 * code * scale.  Attention over it scales each key's score by the key's scale
 * and each weight by the value's scale before the weighted sum (the softmax
 * sum uses the unscaled weights), so the codes feed the matrix cores as exact
 * bf16.  (TensorFold pull request 1388, commit adding the minimax_m3 family,
 * describes such a cache: int8 keys and values with one scale per position
 * and key head, a little over half the bytes of bf16, with the key scales
 * applied to the scores and the value scales to the weights in prompt
 * chunks.  A later commit of the same pull request
 * removed the int8 cache because it changes the model's arithmetic; here it
 * is an alternative entry point and the bf16 path is unchanged.)
 * Index keys stay bf16.  The paged layout applies to the codes and scales as
 * to k and v.
 */
typedef struct msa_kv8 {
    const int8_t *k, *v;            /* codes, element (token t, key head g, dim d) at
                                       t*tok_stride + g*head_stride + d; rows 16-byte aligned */
    const float *k_scale, *v_scale; /* scales, element (t, g) at t*scale_tok_stride + g*scale_head_stride */
    int64_t tok_stride, head_stride;            /* elements (= bytes) */
    int64_t scale_tok_stride, scale_head_stride;  /* elements */
} msa_kv8;

/*
 * Write the int8 cache rows of n_tokens tokens from a bf16 tensor x (k or v,
 * one call each), per (token, key head) row of head_dim values, in fp32:
 * scale = max|x| / 127, code = round-half-even(x / scale) clamped to +-127
 * (IEEE division); an all-zero row gets scale 0.  x must be finite.  This rule
 * is this library's reading: the pages give the scale's granularity only.
 */
int msa_quantize_kv8(const msa_shape *shape, int64_t n_tokens,
                     const void *x, int64_t tok_stride, int64_t head_stride,
                     int8_t *codes, int64_t code_tok_stride, int64_t code_head_stride,
                     float *scales, int64_t scale_tok_stride, int64_t scale_head_stride, void *stream);

/* msa_prefill over an int8 cache (other arguments and errors as msa_prefill). */
int msa_prefill_kv8(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv8 *kv,
                    const int32_t *block_idx, void *out, float *lse, void *stream);

/* msa_decode over an int8 cache (other arguments, workspace and errors as msa_decode). */
int msa_decode_kv8(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv8 *kv,
                   const int32_t *block_idx, void *out, float *lse, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Tiled bf16 key/value cache (opt-in layout; the same values as the strided
 * bf16 cache, and msa_prefill_tiled / msa_decode_tiled return bit for bit
 * what msa_prefill / msa_decode return on it).  The pages leave the cache
 * layout to the kernel; this one stores each key/value block in the order the
 * attention's matrix-core operands read it, so every 64-lane load of a kept
 * block reads 1 KiB of contiguous memory.  Tile (block t, key head g) holds
 * key head g of tokens 64t .. 64t+63: a K tile at k + t*block_stride +
 * g*head_stride and a V tile at the same offset from v, 8,192 bf16 each.
 * Within a tile, chunk c = 0, 1 (keys 32c .. 32c+31 of the block) fills
 * elements 4096c .. 4096c+4095 as 512 pieces of 8 elements, piece q at 8q:
 *   K: q = 256*mt + 64*s + l -> key 32c + 16*mt + l%16, dims 32*s + 8*(l/16) + 0..7
 *   V: q = 64*dt + l         -> dim 16*dt + l%16 of keys 32c + 4*(l/16) + 0..3,
 *                               then of keys 32c + 16 + 4*(l/16) + 0..3
 * (mt < 2, s < 4, dt < 8, l < 64).  Tokens are numbered as for the strided
 * cache (kv_start or the page table), and a block must start a tile: in the
 * contiguous layout every kv_start[s] is a multiple of 64 (a precondition,
 * like cu_rows); in the paged layout page p is tile p.  Keys of a tile that
 * no row can see need not be written (they are never used, NaN included).
 */
typedef struct msa_kv_tiled {
    const void *k, *v;       /* tiles, 16-byte aligned */
    int64_t block_stride;    /* elements between tiles of consecutive blocks: a multiple of 8, >= 8192 */
    int64_t head_stride;     /* elements between key heads' tiles: a multiple of 8, >= 8192 if n_kv_heads > 1 */
} msa_kv_tiled;

/*
 * Write tokens tok_begin .. tok_end-1 of a strided bf16 cache (k and v as in
 * msa_prefill) into their tiles (blocks tok_begin/64 .. (tok_end-1)/64 of
 * k_tiles / v_tiles, strides as in msa_kv_tiled);
 * other keys of those tiles keep their contents, so a cache is extended a
 * prompt chunk or a decode token at a time.  Errors: MSA_ERR_INVALID for a
 * NULL pointer, an empty or negative range, or strides as msa_prefill and
 * msa_kv_tiled reject them.
 */
int msa_pack_kv_tiled(const msa_shape *shape, int64_t tok_begin, int64_t tok_end,
                      const void *k, const void *v, int64_t kv_tok_stride, int64_t kv_head_stride,
                      void *k_tiles, void *v_tiles, int64_t block_stride, int64_t head_stride,
                      void *stream);

/*
 * Write the batch's own keys -- the key at every row's position p, i.e. each
 * sequence's last rows_s tokens, numbered through kv_start or the page table
 * as in msa_prefill -- from a strided bf16 cache into their tiles, in one
 * launch for the whole batch (a decode step's new keys, one per sequence).
 * Strides and errors as msa_pack_kv_tiled; batch errors as msa_prefill.
 */
int msa_pack_kv_tiled_rows(const msa_shape *shape, const msa_batch *batch,
                           const void *k, const void *v, int64_t kv_tok_stride, int64_t kv_head_stride,
                           void *k_tiles, void *v_tiles, int64_t block_stride, int64_t head_stride,
                           void *stream);

/*
 * A decode step's first two calls in one: msa_pack_kv_tiled_rows (the batch's
 * own keys into their tiles; arguments k .. head_stride as there) and
 * msa_index_select (arguments iq .. workspace_bytes as there), with results
 * bit-identical to those two calls.  Each computes what its own declaration
 * cites; the pages' step kernels write a step's keys and values into the
 * cache that its attention then reads (TensorFold pull request 1388, the
 * commit that drops the int8 cache: the prep and decode kernels and the cache
 * layout).  The tiles are read by the attention only, never by the index
 * scores or the selection, so the writes ride in the selection's first launch
 * as extra workgroups (the index-score launch, or the one launch of one-row
 * batches) instead of a launch of their own; only the NULL-block_scores
 * prompt-chunk path takes the writer's launch first.  Each wave writes one
 * (row, key head) key; a prompt chunk whose new keys are one token range per
 * sequence writes them faster with msa_pack_kv_tiled.
 * Errors: the union of the two calls'; on any error nothing is launched.
 */
int msa_index_select_pack_rows(const msa_shape *shape, const msa_batch *batch,
                               const void *iq, const void *ik, int64_t ik_tok_stride, int64_t ik_head_stride,
                               float *block_scores, int32_t bs_stride, int32_t *block_idx,
                               void *workspace, size_t workspace_bytes,
                               const void *k, const void *v, int64_t kv_tok_stride, int64_t kv_head_stride,
                               void *k_tiles, void *v_tiles, int64_t block_stride, int64_t head_stride,
                               void *stream);

/* msa_prefill over a tiled cache (other arguments and errors as msa_prefill). */
int msa_prefill_tiled(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv_tiled *kv,
                      const int32_t *block_idx, void *out, float *lse, void *stream);

/* msa_decode over a tiled cache (other arguments, workspace and errors as msa_decode). */
int msa_decode_tiled(const msa_shape *shape, const msa_batch *batch, const void *q, const msa_kv_tiled *kv,
                     const int32_t *block_idx, void *out, float *lse, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Bytes of device workspace msa_decode needs for total_rows rows (host
 * function; 0 for an invalid shape).  Batches of 80 or more (row, key head)
 * units need only the 512-byte counter region; below that, 512 bytes plus
 * 8,320 bytes per partial (ceil(top_k/4) partials per unit): at most about
 * 5.3 MB for any batch. */
size_t msa_decode_workspace_bytes(const msa_shape *shape, int32_t total_rows);

/*
 * msa_decode_tiled for callers that cannot allocate device memory (code
 * under stream capture, serving loops that forbid allocation): the same
 * kernels and the same results, bit for bit, with the decode workspace
 * taken from a static device array of MSA_DECODE_NOALLOC_SCRATCH_BYTES
 * inside the library instead of a caller buffer.  Each device holds its own
 * copy from the library's load until the process ends.  The call allocates
 * nothing; on its first call on a device (and after a failed launch) it
 * clears the array's counters with a small kernel on `stream` (a kernel, not
 * a memset).
 *   Limit: a batch whose msa_decode_workspace_bytes exceeds the array is
 *   rejected with MSA_ERR_WORKSPACE (with the current kernels no batch
 *   does: the most any batch needs is about 5.3 MB).
 *   Concurrency: every call on one device shares that device's array, which
 *   keeps the last call's contents; calls that overlap in time on one device
 *   (other streams, other threads) race and give undefined results.
 * Other arguments and errors as msa_decode_tiled.
 */
#define MSA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int msa_decode_tiled_noalloc(const msa_shape *shape, const msa_batch *batch, const void *q,
                             const msa_kv_tiled *kv, const int32_t *block_idx, void *out, float *lse,
                             void *stream);

/*
 * Step 4 for decode steps and verify windows: the same result as msa_prefill
 * (within rounding), computed as split-K over the kept keys.  Each kept block
 * (two 32-key pieces) is folded into a state of its own; the states of block
 * slots 4w..4w+3 combine into partial w (max, sum, weighted values), and the
 * partials merge in slot order with log-sum-exp weights.  With fewer than 80
 * (row, key head) units in the batch, each unit's slots are spread over
 * ceil(top_k/4) workgroups that publish their partials in `workspace`, and the
 * last to finish merges them; with more, one workgroup per unit does it all on
 * chip.  Both compute the same tree in the same order, and the tree depends
 * only on top_k, so a row's bits do not depend on the other rows: a verify
 * window equals the same rows decoded one at a time, bit for bit.
 *   workspace        device memory of >= msa_decode_workspace_bytes() bytes,
 *                    256-byte aligned.  Its first 512 bytes hold the
 *                    arrival counters: they must be zero before the first
 *                    call that uses this workspace (allocate it zeroed), and
 *                    every completed call leaves them zero again, whatever
 *                    the batch size, so one workspace serves batches of any
 *                    size it covers.  If a launch fails, zero it again before
 *                    reuse.  Calls that share a workspace must not run
 *                    concurrently.
 * Other arguments as msa_prefill.
 */
int msa_decode(const msa_shape *shape, const msa_batch *batch,
               const void *q, const void *k, const void *v,
               int64_t kv_tok_stride, int64_t kv_head_stride,
               const int32_t *block_idx, void *out, float *lse,
               void *workspace, size_t workspace_bytes, void *stream);

/* Static text for a status code. */
const char *msa_status_string(int status);

/* Detail of the calling thread's last failure ("" if none). */
const char *msa_last_error(void);

/* Library version string (static). */
const char *msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
