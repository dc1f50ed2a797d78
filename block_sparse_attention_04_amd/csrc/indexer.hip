// indexer.hip -- lightning-indexer scores max-pooled per 64-key block.
//
// S[r, g, b] = max over the causally visible keys j of block b of
//              sum_d iq[r, g, d] * ik[j, g, d]
// (TensorFold pull request 1388, commit adding the minimax_m3 family: index
// scores per row and key head; "minimax-m3-sm120", What this fixes: blocks
// are scored by max-pooling.  The plain dot product is this library's
// reading of the unspecified score form.)
//
// The contraction runs on v_mfma_f32_16x16x32_bf16 with keys on the M axis and
// query rows on the N axis (S^T = IK * IQ^T): each lane's accumulator then
// holds 4 keys of one row, so the 64-key max-pool is 15 in-lane maxima per
// lane and, for four such maxima at once (four row tiles, or four blocks),
// three cross-lane swaps that leave each lane group with one of them; no
// score ever leaves the registers.
//
// Two tilings of the same computation:
//   index_scores_tiled  prompt chunks: a workgroup owns 256 rows x a key range;
//                       each 64-key tile of ik is staged once in LDS (a ring
//                       of four, one barrier per two tiles) and reused by the 4
//                       waves' 64 rows each.
//   index_scores_window decode steps and windows (<= 16 rows per sequence):
//                       the 16-row tile is the wave's whole row set, so ik is
//                       streamed straight from HBM into MFMA operand registers
//                       and the key axis is spread over the whole chip.
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"
#include "msa_pack.h"
#include "msa_select.h"

namespace msa {

// k-assignment shared by both operands: k-step s, lane group lg -> index dims
// 16*lg + 8*s + (0..7), i.e. each lane reads 32 contiguous bytes of a vector.

// The lane's part of the block max of one 16-row x 64-key MFMA result (4
// M-tiles): its 16 keys of its row, causal-masked (kMask) against the lane's
// row position; blocks left of the wave's first row take the plain max tree.
// The 4 lane groups' parts are combined by max_scatter_lane_groups.
template <bool kMask>
__device__ __forceinline__ float lane_max_64(const floatx4 (&acc)[4], int key0, int p_row) {
    float m;
    if constexpr (kMask) {
        const int lg = (threadIdx.x & 63) >> 4;
        m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m = fmaxf(m, key0 + 16 * mt + 4 * lg + i > p_row ? -INFINITY : acc[mt][i]);
    } else {
        // 16 values in 8 three-input maxima (v_max3_f32): five triples, two
        // triples of those (with the 16th value), one last pair
        const float u0 = fmaxf(fmaxf(acc[0][0], acc[0][1]), acc[0][2]);
        const float u1 = fmaxf(fmaxf(acc[0][3], acc[1][0]), acc[1][1]);
        const float u2 = fmaxf(fmaxf(acc[1][2], acc[1][3]), acc[2][0]);
        const float u3 = fmaxf(fmaxf(acc[2][1], acc[2][2]), acc[2][3]);
        const float u4 = fmaxf(fmaxf(acc[3][0], acc[3][1]), acc[3][2]);
        m = fmaxf(fmaxf(fmaxf(u0, u1), u2), fmaxf(fmaxf(u3, u4), acc[3][3]));
    }
    return m;
}

constexpr int kTiledWaves = 4;
constexpr int kTiledBlocks = 16;   // blocks per workgroup key range (at most)
constexpr int64_t kTiledFillWgs = 512;   // workgroups below which ranges shrink
constexpr int64_t kMaxGridZ = 65535;     // the launch grid's z extent, at most
constexpr int kLdsRow = 144;   // bytes per staged key (128 + 16 pad: conflict-free b128 reads)

// Slices z >= z_index (msa_index_select_pack_rows) carry the batch's own keys
// into the tiled cache, one (row, key head) per wave: nothing in this launch
// reads the tiles, and the attention that does comes after it on the stream.
template <int NT>
__global__ __launch_bounds__(256) void index_scores_tiled(IndexArgs a, int blocks_per_wg, PackRowsArgs pk,
                                                          int z_index) {
    constexpr int kRowsWave = 16 * NT;
    constexpr int kRowsWg = kRowsWave * kTiledWaves;
    __shared__ __attribute__((aligned(16))) uint8_t lds[4][kBlock * kLdsRow];
    __shared__ float otile[kTiledWaves][kRowsWave * kTiledBlocks];

    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    if ((int)blockIdx.z >= z_index) {
        const int64_t wg = ((int64_t)(blockIdx.z - z_index) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        pack_row_key(pk, wg * 4 + wave, lane);
        return;
    }
    const int lg = lane >> 4, lr = lane & 15;
    const int s = blockIdx.z / a.H, g = blockIdx.z % a.H;
    if (s >= a.b.n_seqs) return;
    const int row0 = a.b.cu_rows[s];
    const int rows_s = a.b.cu_rows[s + 1] - row0;
    const int L = a.b.seq_lens[s];
    if (rows_s <= 0 || rows_s > L || L > a.b.max_seq_len) return;
    const int tile0 = blockIdx.y * kRowsWg;
    if (tile0 >= rows_s) return;
    const int tile_rows = min(kRowsWg, rows_s - tile0);
    const int p_base = L - rows_s;                       // position of row 0 of the sequence
    const int nb_tile = (p_base + tile0 + tile_rows - 1) / kBlock + 1;
    const int b_begin = blockIdx.x * blocks_per_wg;
    const int b_end = min(b_begin + blocks_per_wg, a.bs_stride);
    if (b_begin >= b_end) return;
    const int b_cmp_end = min(b_end, nb_tile);
    const int64_t kv0 = seq_token0(a.b, s);

    // This wave's rows and their indexer queries (the B operand, kept in VGPRs).
    const int wrow0 = tile0 + wave * kRowsWave;
    u32x4 bq[NT][2];
    int prow[NT];
    bool rvalid[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rl = wrow0 + nt * 16 + lr;
        rvalid[nt] = rl < rows_s;
        prow[nt] = p_base + rl;
        if (rvalid[nt]) {
            const uint16_t *src = a.iq + ((int64_t)(row0 + rl) * a.H + g) * kIndexDim + 16 * lg;
            bq[nt][0] = load16(src);
            bq[nt][1] = load16(src + 8);
        } else {
            bq[nt][0] = zero16();
            bq[nt][1] = zero16();
        }
    }
    const int wave_p_min = p_base + wrow0;

    // Staging: thread t copies 32 bytes (piece t&3) of key t>>2 of the tile.
    // Four LDS slots and two register sets: step i computes block i from slot
    // i%4, stores block i+2 (requested two steps earlier) into slot (i+2)%4
    // and requests block i+4.  A slot is written two steps before it is read
    // and two steps after its previous read, so one barrier every two steps
    // (after the odd ones) orders both.
    const int st_key = threadIdx.x >> 2, st_piece = threadIdx.x & 3;
    const uint16_t *ik_g = a.ik + (int64_t)g * a.ik_head + 16 * st_piece;
    struct Stage {
        u32x4 x0, x1;
    };
    // Keys past the sequence end read its last key instead (always in
    // bounds); they lie past every row's position, so the max-pool masks them.
    // First token of each of the workgroup's blocks, looked up once: lane q
    // holds block b_begin + q (clamped to the blocks with visible keys), so
    // the loop's loads never wait on a page-table read.
    const int64_t blk_tok = block_token0(a.b, s, kv0, max(min(b_begin + (lane & 15), b_cmp_end - 1), 0));
    const int blk_tok_lo = (int)(uint32_t)blk_tok, blk_tok_hi = (int)(uint32_t)((uint64_t)blk_tok >> 32);
    auto gload = [&](int b, Stage &r) {
        // b is in [b_begin, b_cmp_end) when the range has visible blocks, else
        // b_cmp_end - 1 < b_begin, which every lane holds (the clamp above)
        const int q = max(b - b_begin, 0);
        const int64_t tok0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(blk_tok_hi, q) << 32) |
                                       (uint32_t)__builtin_amdgcn_readlane(blk_tok_lo, q));
        const int j = min(b * kBlock + st_key, L - 1);    // stays in block b (b holds a visible key)
        const uint16_t *src = ik_g + (tok0 + (j - b * kBlock)) * a.ik_tok;
        r.x0 = load16(src);
        r.x1 = load16(src + 8);
    };
    auto sstore = [&](int buf, const Stage &r) {
        uint8_t *dst = &lds[buf][st_key * kLdsRow + 32 * st_piece];
        *reinterpret_cast<u32x4 *>(dst) = r.x0;
        *reinterpret_cast<u32x4 *>(dst + 16) = r.x1;
    };

    // Block maxima go to an LDS tile [blocks of the range][wave rows] and
    // leave in one flush at the end, so no global store sits between the
    // loop's prefetch loads.  The cross-lane step of the NT = 4 row tiles is
    // one reduce-and-scatter that leaves lane l with row l (tile l/16): one
    // full-wave, conflict-free write per block.
    static_assert(NT * 16 == kWave, "one wave row per lane");
    float *out_tile = otile[wave];
    auto emit = [&](int b, float v) { out_tile[(b - b_begin) * kRowsWave + lane] = v; };
    const int nblk = b_cmp_end - b_begin;
    auto step = [&](int i, Stage &r, bool sync) {
        const int b = b_begin + i;
        const uint8_t *buf = lds[i & 3];
        // A operands of the block's 4 key tiles (both k-steps), read once.
        u32x4 av[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const uint8_t *src = buf + (16 * mt + lr) * kLdsRow + 32 * lg;
            av[mt][0] = *reinterpret_cast<const u32x4 *>(src);
            av[mt][1] = *reinterpret_cast<const u32x4 *>(src + 16);
        }
        const bool need_mask = b * kBlock + kBlock - 1 > wave_p_min;
        // Row tile by row tile: the MFMAs of tile nt are independent of the
        // max-pool of tile nt-1, so the pool fills the MFMA pipeline's gaps.
        // The mask decision is taken once per block, so each variant is
        // straight-line code the scheduler can interleave.
        float m[NT];
        auto tiles = [&](auto masked) {
            constexpr bool kMask = decltype(masked)::value;
            floatx4 prev[4];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                floatx4 cur[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    floatx4 c = {0.f, 0.f, 0.f, 0.f};
                    c = mfma_16x16x32(av[mt][0], bq[nt][0], c);
                    cur[mt] = mfma_16x16x32(av[mt][1], bq[nt][1], c);
                }
                if (nt == 1) {
                    // Unconditional (clamped) so every step issues the same two
                    // loads and the compiler can wait for exactly the older set:
                    // block i+2 was requested two steps ago; slot (i+2)%4 is
                    // not read this step.
                    sstore((i + 2) & 3, r);
                    gload(min(b + 4, b_cmp_end - 1), r);
                }
                if (nt > 0) m[nt - 1] = lane_max_64<kMask>(prev, b * kBlock, prow[nt - 1]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) prev[mt] = cur[mt];
            }
            m[NT - 1] = lane_max_64<kMask>(prev, b * kBlock, prow[NT - 1]);
        };
        if (__builtin_expect(need_mask, 0)) tiles(std::true_type{});
        else tiles(std::false_type{});
        const float v = max_scatter_lane_groups(m[0], m[1], m[2], m[3]);
        if (sync) __syncthreads();
        emit(b, v);
    };

    Stage r0, r1;
    if (nblk > 0) {
        gload(b_begin, r0);
        gload(min(b_begin + 1, b_cmp_end - 1), r1);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {  // iq operands complete before the loop
        force_ready(bq[nt][0]);
        force_ready(bq[nt][1]);
    }
    if (nblk > 0) {
        sstore(0, r0);
        sstore(1, r1);
    }
    gload(min(b_begin + 2, b_cmp_end - 1), r0);
    gload(min(b_begin + 3, b_cmp_end - 1), r1);
    __syncthreads();
    // Both halves unconditional inside the loop (the odd last block after
    // it), so every path into a step has the same loads outstanding and each
    // step waits only for its own register set, never for the prefetch.
    int i = 0;
    for (; i + 1 < nblk; i += 2) {
        step(i, r0, false);
        step(i + 1, r1, true);
    }
    if (i < nblk) step(i, r0, false);
    for (int b = b_cmp_end; b < b_end; ++b) emit(b, -INFINITY);
    wave_lds_sync();
    // Flush: lane l writes its row's blocks, 4 at a time (one 16-byte store
    // when the range is whole and rows are 16-byte aligned).
    const int nb_here = b_end - b_begin;
    const bool vec = nb_here == kTiledBlocks && (a.bs_stride & 3) == 0 && ((uintptr_t)a.scores & 15) == 0;
    const int rl = wrow0 + lane;
    if (rl < rows_s) {
        float *dst = a.scores + ((int64_t)(row0 + rl) * a.H + g) * a.bs_stride + b_begin;
#pragma unroll
        for (int c4 = 0; c4 < kTiledBlocks; c4 += 4) {
            floatx4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = out_tile[(c4 + q) * kRowsWave + lane];
            if (vec) {
                *reinterpret_cast<floatx4 *>(dst + c4) = v;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (c4 + q < nb_here) dst[c4 + q] = v[q];
            }
        }
    }
}

// ---- Selection fused into the prompt-chunk indexer ----
//
// The candidate blocks of a (sequence, key head, 256-row tile) -- every block
// below the tile's last row's local block -- are split over c.splits
// workgroups.  Each computes its blocks' maxima as index_scores_tiled does
// (the same operands, products and order, so the same bits) and, instead of
// storing them, folds each 16 of them into a sorted list of the 16 best
// (score, block) pairs of every row, in registers.  The lists are published
// with agent-scope stores; the last workgroup of the tile to count in merges
// each row's lists and writes its selection.  Each row's kept set is the top
// top_k-1 of the union of the lists: every block of the row's top top_k-1 is
// in the top of its own split with the same tie order, so the result equals
// one pass over all blocks (and msa_select_blocks on the stored scores).
//
// A candidate is one 64-bit value: the score's order key in the high word and
// 0x7fffffff minus the block in the low word, so a larger value is a better
// candidate (higher score, then lower block: the selection's tie rule), and 0
// (an empty slot) is below every real one.
__device__ __forceinline__ uint64_t cand_pack(uint32_t key, int blk) {
    return ((uint64_t)key << 32) | (uint32_t)(0x7fffffff - blk);
}
__device__ __forceinline__ int cand_block(uint64_t c) { return 0x7fffffff - (int)(uint32_t)c; }

// Compare-exchange leaving a >= b (kDesc) or a <= b.
template <bool kDesc, typename T>
__device__ __forceinline__ void cex(T &a, T &b) {
    const bool sw = kDesc ? a < b : b < a;
    const T x = sw ? b : a, y = sw ? a : b;
    a = x;
    b = y;
}

// Bitonic sort of 16 values, descending (kDesc) or ascending.
template <bool kDesc, typename T>
__device__ __forceinline__ void sort16(T (&v)[16]) {
#pragma unroll
    for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    if (((i & k) == 0) != kDesc) cex<false>(v[i], v[l]);
                    else cex<true>(v[i], v[l]);
                }
            }
}

// r (descending) becomes the 16 largest of r and q, descending; q is given
// ascending.  The elementwise maxima of a descending and an ascending
// sequence hold the 16 largest of both as a bitonic sequence, which the
// four-stage half-cleaner cascade sorts.
__device__ __forceinline__ void merge_top16(uint64_t (&r)[16], const uint64_t (&q_asc)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = r[i] < q_asc[i] ? q_asc[i] : r[i];
#pragma unroll
    for (int j = 8; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) cex<true>(r[i], r[l]);
        }
}

template <int NT>
__global__ __launch_bounds__(256) void index_select_tiled(IndexArgs a, ChunkSelect c) {
    constexpr int kRowsWave = 16 * NT;
    constexpr int kRowsWg = kRowsWave * kTiledWaves;
    static_assert(kRowsWg == kChunkRowsWg && kChunkList == 16, "tile and list sizes");
    static_assert(NT * 16 == kWave, "one wave row per lane");
    __shared__ __attribute__((aligned(16))) uint8_t lds[4][kBlock * kLdsRow];
    __shared__ float otile[kTiledWaves][kRowsWave * 16];
    __shared__ int is_last;

    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int lg = lane >> 4, lr = lane & 15;
    const int s = blockIdx.z / a.H, g = blockIdx.z % a.H;
    if (s >= a.b.n_seqs) return;
    const int row0 = a.b.cu_rows[s];
    const int rows_s = a.b.cu_rows[s + 1] - row0;
    const int L = a.b.seq_lens[s];
    // a malformed sequence, or a tile past its rows: every split of the tile
    // returns alike, so no counter is touched
    if (rows_s <= 0 || rows_s > L || L > a.b.max_seq_len) return;
    const int tile = blockIdx.y, tile0 = tile * kRowsWg;
    if (tile0 >= rows_s) return;
    const int tile_rows = min(kRowsWg, rows_s - tile0);
    const int p_base = L - rows_s;                       // position of row 0 of the sequence
    const int l_last = (p_base + tile0 + tile_rows - 1) / kBlock;   // candidates lie below it
    const int split = blockIdx.x;
    const int b_begin = split * c.per_split;
    const int b_end = min(b_begin + c.per_split, l_last);
    const int nblk = max(b_end - b_begin, 0);
    const int64_t kv0 = seq_token0(a.b, s);

    // This wave's rows (B operand in VGPRs); after the reduce-and-scatter,
    // lane l holds row wrow0 + l.
    const int wrow0 = tile0 + wave * kRowsWave;
    u32x4 bq[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rl = wrow0 + nt * 16 + lr;
        if (rl < rows_s) {
            const uint16_t *src = a.iq + ((int64_t)(row0 + rl) * a.H + g) * kIndexDim + 16 * lg;
            bq[nt][0] = load16(src);
            bq[nt][1] = load16(src + 8);
        } else {
            bq[nt][0] = zero16();
            bq[nt][1] = zero16();
        }
    }
    const int my_row = wrow0 + lane;
    const bool my_valid = my_row < rows_s;
    const int my_p = p_base + my_row;
    const int my_l = my_p / kBlock;                      // the row's local block (not a candidate)

    // First token of the workgroup's blocks, three windows of 64 (lane q of
    // window w: block b_begin + 64w + q, clamped to the sequence's blocks),
    // looked up once so the loop's loads never wait on a page-table read.
    const int last_blk = (L - 1) / kBlock;
    const int64_t tw0 = block_token0(a.b, s, kv0, min(b_begin + lane, last_blk));
    const int64_t tw1 = block_token0(a.b, s, kv0, min(b_begin + 64 + lane, last_blk));
    const int64_t tw2 = block_token0(a.b, s, kv0, min(b_begin + 128 + lane, last_blk));
    const int st_key = threadIdx.x >> 2, st_piece = threadIdx.x & 3;
    const uint16_t *ik_g = a.ik + (int64_t)g * a.ik_head + 16 * st_piece;
    struct Stage {
        u32x4 x0, x1;
    };
    auto gload = [&](int b, Stage &r) {
        const int q = b - b_begin;                       // 0 <= q < per_split <= 192
        const int w = q >> 6, qq = q & 63;
        auto at = [&](int64_t t) {                       // lane qq's value of t (wave-uniform)
            return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)((uint64_t)t >> 32), qq) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)t, qq));
        };
        const int64_t tok0 = w == 0 ? at(tw0) : (w == 1 ? at(tw1) : at(tw2));
        const int j = min(b * kBlock + st_key, L - 1);
        const uint16_t *src = ik_g + (tok0 + (j - b * kBlock)) * a.ik_tok;
        r.x0 = load16(src);
        r.x1 = load16(src + 8);
    };
    auto sstore = [&](int buf, const Stage &r) {
        uint8_t *dst = &lds[buf][st_key * kLdsRow + 32 * st_piece];
        *reinterpret_cast<u32x4 *>(dst) = r.x0;
        *reinterpret_cast<u32x4 *>(dst + 16) = r.x1;
    };

    float *out_tile = otile[wave];
    // Every candidate block lies wholly below the row's position, so its
    // maximum needs no causal mask; blocks at or past a row's local block are
    // computed like the others and dropped by the row's filter.
    auto step = [&](int i, Stage &r, bool sync) {
        const int b = b_begin + i;
        const uint8_t *buf = lds[i & 3];
        u32x4 av[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const uint8_t *src = buf + (16 * mt + lr) * kLdsRow + 32 * lg;
            av[mt][0] = *reinterpret_cast<const u32x4 *>(src);
            av[mt][1] = *reinterpret_cast<const u32x4 *>(src + 16);
        }
        float m[NT];
        floatx4 prev[4];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            floatx4 cur[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma_16x16x32(av[mt][0], bq[nt][0], acc);
                cur[mt] = mfma_16x16x32(av[mt][1], bq[nt][1], acc);
            }
            if (nt == 1) {
                sstore((i + 2) & 3, r);
                gload(min(b + 4, b_end - 1), r);
            }
            if (nt > 0) m[nt - 1] = lane_max_64<false>(prev, 0, 0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) prev[mt] = cur[mt];
        }
        m[NT - 1] = lane_max_64<false>(prev, 0, 0);
        const float v = max_scatter_lane_groups(m[0], m[1], m[2], m[3]);
        if (sync) __syncthreads();
        out_tile[(i & 15) * kRowsWave + lane] = v;
    };

    // The row's running list: the 16 best candidates so far, descending.
    uint64_t best[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) best[q] = 0ull;
    // Fold the batch of n (<= 16) maxima in the tile slots (blocks base ..
    // base+n-1) into the list.
    auto fold_batch = [&](int base, int n) {
        wave_lds_sync();
        uint64_t x[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int blk = base + q;
            const float v = out_tile[q * kRowsWave + lane];
            x[q] = (q < n && blk < my_l) ? cand_pack(order_key(v), blk) : 0ull;
        }
        wave_lds_sync();   // the slots are read before the next batch overwrites them
        sort16<false>(x);
        merge_top16(best, x);
    };

    Stage r0, r1;
    if (nblk > 0) {
        gload(b_begin, r0);
        gload(min(b_begin + 1, b_end - 1), r1);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        force_ready(bq[nt][0]);
        force_ready(bq[nt][1]);
    }
    if (nblk > 0) {
        sstore(0, r0);
        sstore(1, r1);
        gload(min(b_begin + 2, b_end - 1), r0);
        gload(min(b_begin + 3, b_end - 1), r1);
    }
    __syncthreads();
    int i = 0;
    for (; i + 1 < nblk; i += 2) {
        step(i, r0, false);
        step(i + 1, r1, true);
        if (((i + 1) & 15) == 15 || i + 1 == nblk - 1) fold_batch(b_begin + ((i + 1) & ~15), ((i + 1) & 15) + 1);
    }
    if (i < nblk) {
        step(i, r0, false);
        fold_batch(b_begin + (i & ~15), (i & 15) + 1);
    }

    // Publish the list (agent-scope stores: written through this XCD's L2),
    // wait for the stores, then count the workgroup in.  The language's model
    // orders none of this; gfx950's sc1 stores and loads and its
    // device-level atomic add do (see decode_kernel).
    uint64_t *mine = c.cand + (((int64_t)(row0 + my_row) * a.H + g) * c.splits + split) * kChunkList;
    if (my_valid) {
#pragma unroll
        for (int q = 0; q < 16; ++q) __hip_atomic_store(mine + q, best[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    unsigned *counter = c.count + ((int64_t)s * a.H + g) * c.tiles + tile;
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last) return;
    if (threadIdx.x == 0)   // leave the counter at zero for the next call
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!my_valid) return;

    // The last workgroup: each lane merges its row's lists from every split.
    const uint64_t *lists = c.cand + ((int64_t)(row0 + my_row) * a.H + g) * c.splits * kChunkList;
    for (int sp = 0; sp < c.splits; ++sp) {
        if (sp == split) continue;
        uint64_t q_asc[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
            q_asc[15 - q] = __hip_atomic_load(lists + sp * kChunkList + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        merge_top16(best, q_asc);
    }
    const int top_k = c.top_k, nb = my_l + 1;
    int32_t *out = c.idx + ((int64_t)(row0 + my_row) * a.H + g) * top_k;
    int f[16];
    if (nb <= top_k) {          // every causal block
#pragma unroll
        for (int q = 0; q < 16; ++q) f[q] = q < nb ? q : -1;
    } else {                    // the best top_k-1, then the local block, ascending
#pragma unroll
        for (int q = 0; q < 15; ++q) f[q] = q < top_k - 1 ? cand_block(best[q]) : 0x7fffffff;
        f[15] = my_l;
        sort16<false>(f);
    }
    if (top_k == 16 && ((uintptr_t)c.idx & 15u) == 0) {
#pragma unroll
        for (int q = 0; q < 16; q += 4) *reinterpret_cast<int4 *>(out + q) = make_int4(f[q], f[q + 1], f[q + 2], f[q + 3]);
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if (q < top_k) out[q] = f[q];
    }
}

// tok0: token of the block's first key; keys past the sequence end read its
// last key (in the same block) and are masked.
__device__ __forceinline__ void window_load_block(u32x4 (&av)[4][2], const uint16_t *ik_g, int64_t tok0,
                                                  int64_t tok, int b, int L, int lr) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int j = min(b * kBlock + 16 * mt + lr, L - 1);
        const uint16_t *src = ik_g + (tok0 + (j - b * kBlock)) * tok;
        av[mt][0] = load16(src);
        av[mt][1] = load16(src + 8);
    }
}

// The lane's part of block b's max for its row (prow), masked when the block
// reaches past the window's first row p_first (wave-uniform).
__device__ __forceinline__ float window_lane_max(const u32x4 (&av)[4][2], u32x4 bq0, u32x4 bq1, int b, int prow,
                                                 int p_first) {
    floatx4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        floatx4 c = {0.f, 0.f, 0.f, 0.f};
        c = mfma_16x16x32(av[mt][0], bq0, c);
        acc[mt] = mfma_16x16x32(av[mt][1], bq1, c);
    }
    const int key0 = b * kBlock;
    return __builtin_expect(key0 + kBlock - 1 > p_first, 0) ? lane_max_64<true>(acc, key0, prow)
                                                           : lane_max_64<false>(acc, key0, prow);
}

// Each wave owns kWindowBlocks = 4 consecutive blocks: all their loads go
// out before the first MFMA (a block past the sequence re-reads its last
// computed block and is discarded), and lane group lg ends up holding block
// b_begin + lg.

// The selection of one one-row unit by the wave that finished last, from the
// range maxima and scores every wave published (agent-scope loads).  The
// range maxima give T0, a lower bound on the (top_k-1)-th best candidate
// score T: the top_k-1 largest range maxima belong to distinct ranges, each
// holding a candidate at least that large.  Every candidate >= T then lies in
// a range whose maximum is >= T0, so only those ranges' scores are read
// (usually top_k-1 of them, at most 64 here).  Among their blocks only those
// >= T0 can be kept (at least top_k-1 blocks reach T0): they are listed in
// ascending block order, one per lane, and top_keep keeps the top top_k-1 of
// the list with ties to the lower block (by rank for short lists, by a
// bitwise search for the cut otherwise).  More than 64 candidate ranges, or
// more than 64 blocks at or above T0 (mass ties), take an exact search over
// every candidate score instead, streamed from memory.
struct WindowTailLds {
    int32_t cr[2 * kWave];    // candidate ranges; [kWave, 2 kWave): per-lane discard slots
    uint2 kb[2 * kWave];      // blocks >= T0: (order key, block); discard slots as above
};

// Exclusive prefix over the lanes of cnt (0 <= cnt < 2^kBits), and the total.
template <int kBits>
__device__ __forceinline__ int lane_prefix(int cnt, int &total) {
    int pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < kBits; ++bit) {
        const uint64_t bm = __ballot((cnt >> bit) & 1);
        pre += lanes_below(bm) << bit;
        tot += (int)__popcll(bm) << bit;
    }
    total = tot;
    return pre;
}

__device__ __forceinline__ void window_select_tail(const float *scores, const float *wmax, int n, int top_k,
                                                   int32_t *out, WindowTailLds &sh) {
    const int lane = threadIdx.x & 63;
    const int nb = n + 1, need = top_k - 1;
    if (nb <= top_k || need == 0) {
        if (lane < top_k) out[lane] = nb <= top_k ? (lane < nb ? lane : -1) : n;
        return;
    }
    auto ld = [](const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    const int nw = (n + kWindowBlocks - 1) / kWindowBlocks;       // ranges holding candidates
    // pass 1: T0 from the per-lane maxima of the range maxima (16 per lane per
    // round; the first round's values stay in registers for pass 2)
    float x0[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x0[j] = ld(wmax + min(lane + kWave * j, nw - 1));
    uint32_t lmax = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (lane + kWave * j < nw) lmax = max(lmax, order_key(x0[j]));
    for (int w0 = 16 * kWave; w0 < nw; w0 += 16 * kWave) {
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = ld(wmax + min(w0 + lane + kWave * j, nw - 1));
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (w0 + lane + kWave * j < nw) lmax = max(lmax, order_key(x[j]));
    }
    const uint32_t t0 = kth_largest_wave<16>(lmax, need);
    // pass 2: the ranges with a maximum >= T0 into cr[0, c) in ascending
    // order: the 16 masks first, then each one's place from the running count
    int c = 0;
    for (int w0 = 0; w0 < nw; w0 += 16 * kWave) {
        float x[16];
        if (w0 == 0) {
#pragma unroll
            for (int j = 0; j < 16; ++j) x[j] = x0[j];
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) x[j] = ld(wmax + min(w0 + lane + kWave * j, nw - 1));
        }
        uint64_t bm[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) bm[j] = __ballot(w0 + lane + kWave * j < nw && order_key(x[j]) >= t0);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const bool f = (bm[j] >> lane) & 1ull;
            const int pos = c + lanes_below(bm[j]);
            sh.cr[f && pos < kWave ? pos : kWave + lane] = w0 + lane + kWave * j;
            c += (int)__popcll(bm[j]);
        }
    }
    bool done = false;   // wave-uniform
    if (c <= kWave) {
        wave_lds_sync();
        // lane l: the 4 blocks of candidate range l; those >= T0 into kb[0, m)
        const int w = lane < c ? sh.cr[lane] : 0;
        float sv[kWindowBlocks];
#pragma unroll
        for (int j = 0; j < kWindowBlocks; ++j) sv[j] = ld(scores + min(kWindowBlocks * w + j, n - 1));
        uint32_t fb = 0u;
#pragma unroll
        for (int j = 0; j < kWindowBlocks; ++j)
            fb |= (lane < c && kWindowBlocks * w + j < n && order_key(sv[j]) >= t0 ? 1u : 0u) << j;
        int m;
        int pos = lane_prefix<3>(__popc(fb), m);
#pragma unroll
        for (int j = 0; j < kWindowBlocks; ++j) {
            const bool f = (fb >> j) & 1u;
            sh.kb[f && pos < kWave ? pos : kWave + lane] =
                make_uint2(order_key(sv[j]), (uint32_t)(kWindowBlocks * w + j));
            pos += f ? 1 : 0;
        }
        if (m <= kWave) {
            wave_lds_sync();
            // lane l: block l of the list (ascending blocks)
            const uint2 me = lane < m ? sh.kb[lane] : make_uint2(0u, 0u);
            const bool take = top_keep(me.x, m, need);
            const uint64_t tm = __ballot(take);
            if (take) out[lanes_below(tm)] = (int32_t)me.y;
            done = true;
        }
    }
    if (!done) {
        // exact fallback (more than 64 candidate ranges, or more than 64
        // blocks at or above T0: ties): bitwise search for T over every
        // candidate score, then one pass in block order
        uint32_t t = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cb = t | (1u << bit);
            int cnt = 0;
            for (int j = lane; j < n; j += kWave) cnt += order_key(ld(scores + j)) >= cb;
            if (wave_sum_int(cnt) >= need) t = cb;
        }
        int cnt = 0;
        for (int j = lane; j < n; j += kWave) cnt += order_key(ld(scores + j)) > t;
        const int need_eq = need - wave_sum_int(cnt);
        int taken = 0, eq_seen = 0;
        for (int j0 = 0; j0 < n; j0 += kWave) {
            const int j = j0 + lane;
            const uint32_t v = j < n ? order_key(ld(scores + j)) : 0u;
            const bool eq = j < n && v == t;
            const uint64_t em = __ballot(eq);
            const bool tk = (j < n && v > t) || (eq && eq_seen + lanes_below(em) < need_eq);
            const uint64_t tm = __ballot(tk);
            if (tk) out[taken + lanes_below(tm)] = j;
            taken += __popcll(tm);
            eq_seen += __popcll(em);
        }
    }
    if (lane == 0) out[need] = n;
}

// kSelect: the fused index-and-select variant (launched for one-row
// sequences).  Every wave stores its scores and its range's best candidate
// score with agent-scope stores; once a workgroup's stores have completed it
// counts itself in on the counter of its (sequence, key-head group); the last
// workgroup's waves select the group's heads, one head per wave.
// Workgroup columns from x_index on (sequence slice z = 0 only) carry the
// batch's own keys into the tiled cache, one (row, key head) per wave
// (msa_index_select_pack_rows): nothing in this launch reads the tiles, and
// the attention that does comes after it on the stream.
// kDeep: a wave requests all 4 of its blocks at once (4 register sets), for
// launches small enough that every workgroup is resident together: its walk
// then waits for one round trip to memory instead of three.
template <bool kSelect, bool kDeep>
__global__ __launch_bounds__(256) void index_scores_window(IndexArgs a, SelectTail t, PackRowsArgs pk,
                                                           int x_index) {
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    if ((int)blockIdx.x >= x_index) {
        if (blockIdx.z == 0) pack_row_key(pk, (int64_t)(blockIdx.x - x_index) * 4 + wave, lane);
        return;
    }
    const int lg = lane >> 4, lr = lane & 15;
    // With a multiple of 4 key heads, a workgroup's 4 waves are 4 heads of one
    // 4-block key range (blockIdx.x = key range * H/4 + head group), so index
    // keys of neighbouring heads, side by side in token-major caches, are
    // read by one CU at the same time.  Otherwise a workgroup is one head's
    // 16 blocks (blockIdx.x = key range * H + head), the heads of a key range
    // dispatched together.
    const bool heads_wg = a.H % 4 == 0;
    const int s = blockIdx.z;
    const int n_groups = heads_wg ? a.H / 4 : a.H;          // workgroups per key range
    const int g0 = heads_wg ? (blockIdx.x % n_groups) * 4 : blockIdx.x % a.H;   // the workgroup's first head
    const int g = heads_wg ? g0 + wave : g0;
    const int xr = blockIdx.x / n_groups;
    if (s >= a.b.n_seqs) return;
    const int row0 = a.b.cu_rows[s];
    const int rows_s = a.b.cu_rows[s + 1] - row0;
    const int L = a.b.seq_lens[s];
    if (rows_s <= 0 || rows_s > 16 || rows_s > L || L > a.b.max_seq_len) return;   // whole (s, g) alike
    if (kSelect && rows_s != 1) return;                                            // launched for one-row batches
    const int range = heads_wg ? xr : xr * 4 + wave;        // this wave's 4-block range
    const int b_begin = range * kWindowBlocks;
    const int b_end = min(b_begin + kWindowBlocks, a.bs_stride);
    const int p_first = L - rows_s;
    if (b_begin < b_end) {
        const int nb_seq = (L - 1) / kBlock + 1;
        const int nblk = min(b_end, nb_seq) - b_begin;    // blocks with visible keys
        const int64_t kv0 = seq_token0(a.b, s);
        const bool rvalid = lr < rows_s;
        const int prow = p_first + lr;
        float mine = -INFINITY;
        if (nblk > 0) {
            u32x4 bq0 = zero16(), bq1 = zero16();
            if (rvalid) {
                const uint16_t *src = a.iq + ((int64_t)(row0 + lr) * a.H + g) * kIndexDim + 16 * lg;
                bq0 = load16(src);
                bq1 = load16(src + 8);
            }
            const uint16_t *ik_g = a.ik + (int64_t)g * a.ik_head + 16 * lg;
            // Two register sets: block q+2 is requested as soon as block q
            // is computed (past the last visible block, that block again).
            auto ld = [&](int q, u32x4 (&av)[4][2]) {
                const int bq = b_begin + min(q, nblk - 1);
                window_load_block(av, ik_g, block_token0(a.b, s, kv0, bq), a.ik_tok, bq, L, lr);
            };
            static_assert(kWindowBlocks == 4, "the register sets below cover four blocks");
            float m0, m1, m2, m3;
            if constexpr (kDeep) {
                u32x4 ra[4][2], rb[4][2], rc[4][2], rd[4][2];
                ld(0, ra);
                ld(1, rb);
                ld(2, rc);
                ld(3, rd);
                m0 = window_lane_max(ra, bq0, bq1, b_begin, prow, p_first);
                m1 = window_lane_max(rb, bq0, bq1, b_begin + 1, prow, p_first);
                m2 = window_lane_max(rc, bq0, bq1, b_begin + 2, prow, p_first);
                m3 = window_lane_max(rd, bq0, bq1, b_begin + 3, prow, p_first);
            } else {
                u32x4 ra[4][2], rb[4][2];
                ld(0, ra);
                ld(1, rb);
                m0 = window_lane_max(ra, bq0, bq1, b_begin, prow, p_first);
                ld(2, ra);
                m1 = window_lane_max(rb, bq0, bq1, b_begin + 1, prow, p_first);
                ld(3, rb);
                m2 = window_lane_max(ra, bq0, bq1, b_begin + 2, prow, p_first);
                m3 = window_lane_max(rb, bq0, bq1, b_begin + 3, prow, p_first);
            }
            // lane group lg ends with block b_begin + lg (past the visible
            // blocks: a re-read, discarded)
            const float v = max_scatter_lane_groups(m0, m1, m2, m3);
            if (lg < nblk) mine = v;
        }
        const int blk = b_begin + lg;
        if (rvalid && blk < b_end) {
            float *dst = a.scores + ((int64_t)(row0 + lr) * a.H + g) * a.bs_stride + blk;
            if constexpr (kSelect)   // agent-scope store (written through the XCD's L2)
                __hip_atomic_store(dst, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                *dst = mine;
        }
        if constexpr (kSelect) {
            // the range's best candidate (blocks below the row's local block)
            const int n_cand = p_first / kBlock;
            const float cm = max_over_lane_groups(lr == 0 && lg < nblk && blk < n_cand ? mine : -INFINITY);
            if (lane == 0 && b_begin < n_cand)
                __hip_atomic_store(t.wmax + ((int64_t)s * a.H + g) * t.ranges + range, cm, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if constexpr (kSelect) {
        // Every store above is agent-scoped (compiled with sc1: written
        // through the XCD's L2 to the device-coherent level), so publishing
        // them needs only their completion: wait for this wave's stores, meet
        // at the barrier, then count the workgroup in (the atomic add is
        // performed at that level).  The last workgroup reads them with
        // agent-scope loads (sc1: not served from a copy in its own L2).  The
        // language's model orders none of this; an agent-scope release fence
        // would, but writes back the whole L2 in each of the many workgroups.
        __shared__ WindowTailLds tail_lds[4];
        __shared__ int is_last;
        const int unit = s * n_groups + (heads_wg ? g0 / 4 : g0);   // (sequence, head group)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned prev = __hip_atomic_fetch_add(t.count + unit, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            is_last = prev == x_index / n_groups - 1;
        }
        __syncthreads();
        if (!is_last) return;
        if (threadIdx.x == 0)   // leave the counter at zero for the next call
            __hip_atomic_store(t.count + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!heads_wg && wave != 0) return;          // one head: its first wave selects
        const int gs = heads_wg ? g0 + wave : g0;
        const int64_t u = (int64_t)row0 * a.H + gs;
        window_select_tail(a.scores + u * a.bs_stride, t.wmax + ((int64_t)s * a.H + gs) * t.ranges, p_first / kBlock,
                           t.top_k, t.idx + u * t.top_k, tail_lds[wave]);
    }
}

// index_scores_window's grid: with heads in fours, a workgroup per (4-block
// key range, group of 4 heads); else per (16-block range, head).  With a
// batch writer `pk`, one more column per 4 (row, key head) units.
// The deep variant while the index workgroups fit the chip at once: 3 per
// compute unit at its register use, 256 compute units.
constexpr int64_t kDeepWindowWgs = 3 * 256;
static bool window_deep(int x_index, int n_seqs) { return (int64_t)x_index * n_seqs <= kDeepWindowWgs; }

static dim3 window_grid(const IndexArgs &a, const PackRowsArgs *pk, int *x_index) {
    int x = 0;
    if (a.H % 4 == 0) {
        x = (a.bs_stride + kWindowBlocks - 1) / kWindowBlocks * (a.H / 4);
    } else {
        const int per_wg = kWindowBlocks * 4;
        x = (a.bs_stride + per_wg - 1) / per_wg * a.H;
    }
    *x_index = x;
    const int64_t pack_wgs = pk ? ((int64_t)pk->b.total_rows * pk->H + 3) / 4 : 0;
    return dim3((unsigned)(x + pack_wgs), 1, a.b.n_seqs);
}

hipError_t launch_index_scores(const IndexArgs &a, hipStream_t st, const PackRowsArgs *pk) {
    const int gz = a.b.n_seqs * a.H;
    if (a.b.max_rows <= 16) {
        int x_index = 0;
        const dim3 grid = window_grid(a, pk, &x_index);
        if (window_deep(x_index, a.b.n_seqs))
            hipLaunchKernelGGL((index_scores_window<false, true>), grid, dim3(256), 0, st, a, SelectTail{},
                               pk ? *pk : PackRowsArgs{}, x_index);
        else
            hipLaunchKernelGGL((index_scores_window<false, false>), grid, dim3(256), 0, st, a, SelectTail{},
                               pk ? *pk : PackRowsArgs{}, x_index);
    } else {
        constexpr int NT = 4;
        const int rows_wg = 16 * NT * kTiledWaves;
        const int tiles = (a.b.max_rows + rows_wg - 1) / rows_wg;
        // 16 blocks per workgroup; fewer (8, 4, 2, 1) while the grid would
        // leave most of the chip idle (a 2,048-row prefill has 8 row tiles x
        // 2 ranges of 16 blocks).  Scores do not depend on it.
        int per = kTiledBlocks;
        while (per > 1 && (int64_t)gz * tiles * ((a.bs_stride + per - 1) / per) < kTiledFillWgs) per /= 2;
        dim3 grid((a.bs_stride + per - 1) / per, tiles, gz);
        if (pk) {   // the writer's workgroups: whole slices after the indexer's
            const int64_t pack_wgs = ((int64_t)pk->b.total_rows * pk->H + 3) / 4;
            const int64_t per_slice = (int64_t)grid.x * grid.y;
            const int64_t slices = (pack_wgs + per_slice - 1) / per_slice;
            if (gz + slices <= kMaxGridZ) {
                grid.z += (unsigned)slices;
            } else {   // past the grid's z limit: the writer's own launch first
                const hipError_t e = launch_pack_kv_rows(*pk, st);
                if (e != hipSuccess) return e;
                pk = nullptr;
            }
        }
        hipLaunchKernelGGL(index_scores_tiled<NT>, grid, dim3(256), 0, st, a, per, pk ? *pk : PackRowsArgs{}, gz);
    }
    return hipGetLastError();
}

hipError_t launch_index_select_chunk(const IndexArgs &a, const ChunkSelect &c, hipStream_t st) {
    const dim3 grid((unsigned)c.splits, (unsigned)c.tiles, (unsigned)(a.b.n_seqs * a.H));
    hipLaunchKernelGGL(index_select_tiled<4>, grid, dim3(256), 0, st, a, c);
    return hipGetLastError();
}

// The fused one-row selection always takes the deep variant: beside a
// prompt chunk's indexer (the chunk's workgroups leave no room for a scan
// wave on their SIMDs, so the scan takes compute units as they free up) a
// workgroup that waits for one round trip instead of three holds its unit
// for less time (262,144-key row beside the chunk: step 564.0 -> 562.6 us;
// alone 41.3 -> 41.2 us).  The scores-only launch keeps the residency rule
// (verify windows: 62.1 us, 63.4 us with the deep variant).
hipError_t launch_index_select(const IndexArgs &a, SelectTail t, hipStream_t st, const PackRowsArgs *pk) {
    int x_index = 0;
    const dim3 grid = window_grid(a, pk, &x_index);
    hipLaunchKernelGGL((index_scores_window<true, true>), grid, dim3(256), 0, st, a, t, pk ? *pk : PackRowsArgs{},
                       x_index);
    return hipGetLastError();
}

}  // namespace msa
