// msa_launch.h -- library-internal kernel argument blocks and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

struct BatchDev {
    int n_seqs, total_rows, max_rows, max_seq_len;
    const int32_t *cu_rows;
    const int32_t *seq_lens;
    const int64_t *kv_start;     // contiguous layout
    const int32_t *page_table;   // paged layout (null: contiguous)
    int pages_per_seq;
};

// First token of sequence s in the key tensors (contiguous layout; 0 when paged).
__device__ __forceinline__ int64_t seq_token0(const BatchDev &b, int s) {
    return b.page_table ? 0 : b.kv_start[s];
}

// Token of the first key of logical block blk of sequence s, whose contiguous
// start is kv0 (from seq_token0).  Keys blk*64 + i (i < 64) follow at + i.
__device__ __forceinline__ int64_t block_token0(const BatchDev &b, int s, int64_t kv0, int blk) {
    return b.page_table ? (int64_t)b.page_table[(int64_t)s * b.pages_per_seq + blk] * 64
                        : kv0 + (int64_t)blk * 64;
}

struct IndexArgs {
    BatchDev b;
    int H;                       // key heads
    const uint16_t *iq;          // [total_rows, H, 64]
    const uint16_t *ik;          // strided, dims contiguous
    int64_t ik_tok, ik_head;     // element strides
    float *scores;               // [total_rows, H, bs_stride]
    int bs_stride;
};

struct SelectArgs {
    BatchDev b;
    int H, top_k;
    const float *scores;
    int bs_stride;
    int32_t *idx;                // [total_rows, H, top_k]
};

struct AttnArgs {
    BatchDev b;
    int H, top_k;
    float scale_log2;            // softmax scale * log2(e)
    const uint16_t *q;           // [total_rows, H*16, 128]
    const uint16_t *k, *v;       // strided, dims contiguous; or tiled (below)
    int64_t kv_tok, kv_head;     // tiled: elements between tiles of consecutive blocks / key heads
    bool tiled;                  // k, v are tiled caches (tile of block t0 / 64, operand order)
    const int32_t *idx;          // [total_rows, H, top_k]
    uint16_t *out;               // [total_rows, H*16, 128]
    float *lse;                  // [total_rows, H*16] or null
    unsigned *ws_count;          // decode: one arrival counter per (row, key head)
    float *ws_part;              // decode: one partial per workgroup of a (row, key head)
    // int8 cache (k8 non-null): codes with the kv_tok / kv_head strides, one
    // fp32 scale per (token, key head) with the s_tok / s_head strides
    const int8_t *k8, *v8;
    const float *ks, *vs;
    int64_t s_tok, s_head;
};

// Selection fused after the decode-shaped indexer (one-row batches).
struct SelectTail {
    int top_k;
    int32_t *idx;                // [total_rows, H, top_k]
    unsigned *count;             // one arrival counter per (sequence, key-head group); zero between calls
    float *wmax;                 // [n_seqs, H, ranges]: the best candidate score of each 4-block range
    int ranges;                  // row stride of wmax: ceil(ceil(max_seq_len / 64) / 4)
};
constexpr int kWindowBlocks = 4;   // blocks per wave of the decode-shaped indexer
inline int window_ranges(int max_seq_len) { return ((max_seq_len + 63) / 64 + kWindowBlocks - 1) / kWindowBlocks; }

// Selection fused into the prompt-chunk indexer: the candidate blocks of each
// (sequence, key head, 256-row tile) are split over `splits` workgroups of
// `per_split` blocks; each keeps a sorted list of its kChunkList best
// (score, block) pairs per row and publishes it, and the last workgroup of
// the tile merges the lists and writes the selection.
constexpr int kChunkRowsWg = 256;
constexpr int kChunkList = 16;          // list length: top_k - 1 <= 15 candidates plus one spare
constexpr int kChunkMaxTopK = 16;
constexpr int kChunkMaxPerSplit = 192;  // blocks a workgroup's page lookups cover
struct ChunkSelect {
    int top_k;
    int32_t *idx;                // [total_rows, H, top_k]
    unsigned *count;             // one counter per (sequence, key head, row tile); zero between calls
    uint64_t *cand;              // [total_rows, H, splits, kChunkList] packed (key, block) pairs
    int splits, per_split, tiles;
};
// Workspace of msa_index_select: a fixed region of arrival counters (one per
// (sequence, key head) for one-row batches, per (sequence, key head, row
// tile) for prompt chunks), then the prompt chunks' candidate lists.  The
// counters' place does not depend on the batch, so one zeroed workspace
// serves batches of any size it covers.
constexpr size_t kIndexSelectCountBytes = 256 * 1024;
constexpr int64_t kIndexSelectCounters = kIndexSelectCountBytes / 4;
inline int chunk_tiles(int max_rows) { return (max_rows + kChunkRowsWg - 1) / kChunkRowsWg; }
// Splits of the key range: about 512 workgroups in all (two per CU), at most
// one per 16 blocks, at most kChunkMaxPerSplit blocks each.
inline void chunk_splits(int n_seqs, int H, int max_rows, int max_seq_len, int *splits, int *per_split) {
    const int64_t tiles = chunk_tiles(max_rows);
    const int nbk = (max_seq_len + 63) / 64;
    const int64_t units = (int64_t)n_seqs * H * tiles;
    int S = (int)((512 + units - 1) / units);
    S = S < 1 ? 1 : S;
    const int s_max = (nbk + 15) / 16 > 0 ? (nbk + 15) / 16 : 1;
    S = S > s_max ? s_max : S;
    int per = (nbk + S - 1) / S;
    while (per > kChunkMaxPerSplit) {
        ++S;
        per = (nbk + S - 1) / S;
    }
    *splits = S;
    *per_split = per > 0 ? per : 1;
}
// Whether msa_index_select can run a batch through the fused prompt-chunk kernel.
inline bool chunk_select_eligible(int n_seqs, int H, int max_rows, int top_k) {
    return max_rows > 16 && top_k <= kChunkMaxTopK && (int64_t)n_seqs * H * chunk_tiles(max_rows) <= kIndexSelectCounters;
}
inline size_t index_select_workspace_bytes(int n_seqs, int H, int total_rows, int max_rows, int max_seq_len,
                                           int top_k) {
    size_t b = kIndexSelectCountBytes;
    if (chunk_select_eligible(n_seqs, H, max_rows, top_k)) {
        int S, per;
        chunk_splits(n_seqs, H, max_rows, max_seq_len, &S, &per);
        b += (size_t)total_rows * H * S * kChunkList * sizeof(uint64_t);
    } else if (max_rows == 1) {   // the range maxima of the one-row path
        b += ((size_t)n_seqs * H * window_ranges(max_seq_len) * sizeof(float) + 255) / 256 * 256;
    }
    return b;
}

// Decode partial: m[16], l[16], acc[16][128] (fp32) for one workgroup's kept blocks.
constexpr int kPartialFloats = 16 + 16 + 16 * 128;
inline int decode_wg_per_unit(int top_k) { return (top_k + 3) / 4; }
// Units from which a decode launch takes one workgroup per unit (no
// workspace); below it, a unit's slots are split over several workgroups that
// exchange partials through the workspace.
constexpr int64_t kDecodeUnitKernelMin = 80;
// Workspace: a fixed region of arrival counters (one uint32 per unit of the
// split kernel), then the partials.  The counters' place does not depend on
// the batch, so a workspace reused by batches of other sizes keeps its
// zeroed counters apart from every partial.
constexpr size_t kDecodeCountBytes = 512;
static_assert(kDecodeUnitKernelMin * 4 <= (int64_t)kDecodeCountBytes, "counter region too small");
inline size_t decode_workspace_bytes(int64_t units, int top_k) {
    if (units >= kDecodeUnitKernelMin) return kDecodeCountBytes;
    return kDecodeCountBytes + (size_t)units * decode_wg_per_unit(top_k) * kPartialFloats * sizeof(float);
}

// int8 cache writer: one bf16 [tokens, H, 128] tensor -> codes + scales.
struct QuantArgs {
    const uint16_t *x;
    int64_t tok, head;           // element strides of x
    int8_t *codes;
    int64_t ctok, chead;         // element strides of codes
    float *scales;
    int64_t stok, shead;         // element strides of scales
    int64_t n_tokens;
    int H;
};

// Tiled cache writer: tokens [tok_begin, tok_end) of strided k / v into the
// tiles of blocks tok_begin / 64 .. (tok_end - 1) / 64 (n_blocks of them).
constexpr int kTileElems = 64 * 128;   // one key head's K (or V) of one block

struct PackTiledArgs {
    const uint16_t *k, *v;
    int64_t tok, head;           // element strides of k / v
    uint16_t *kt, *vt;
    int64_t t_blk, t_head;       // element strides of the tiles
    int64_t tok_begin, tok_end, n_blocks;
    int H;
};

// Tiled cache writer for a batch's own keys (key p of every row).
struct PackRowsArgs {
    BatchDev b;
    const uint16_t *k, *v;
    int64_t tok, head;
    uint16_t *kt, *vt;
    int64_t t_blk, t_head;
    int H;
};

// Sets the message msa_last_error() returns (empty for success) and returns status.
int report(int status, const char *msg);

hipError_t launch_quantize_kv8(const QuantArgs &a, hipStream_t st);
hipError_t launch_pack_kv_tiled(const PackTiledArgs &a, hipStream_t st);
hipError_t launch_pack_kv_rows(const PackRowsArgs &a, hipStream_t st);
// pk (optional): the batch's own keys into the tiled cache in the same launch
// (extra workgroups for decode-shaped batches, else a launch of its own first).
hipError_t launch_index_scores(const IndexArgs &a, hipStream_t st, const PackRowsArgs *pk = nullptr);
hipError_t launch_select_blocks(const SelectArgs &a, hipStream_t st);
hipError_t launch_index_select(const IndexArgs &a, SelectTail t, hipStream_t st, const PackRowsArgs *pk = nullptr);
hipError_t launch_index_select_chunk(const IndexArgs &a, const ChunkSelect &c, hipStream_t st);
hipError_t launch_prefill(const AttnArgs &a, hipStream_t st);
hipError_t launch_decode(const AttnArgs &a, hipStream_t st);

}  // namespace msa
