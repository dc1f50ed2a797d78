// msa_pack.h -- device code that writes a batch's own keys into the tiled
// cache, shared by the batch writer (pack_kv_rows_kernel) and the selection
// launches that carry the write (msa_index_select_pack_rows).  The tile layout
// is the one kvcache.hip describes.
#pragma once

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// Key p of unit `unit` = (row, key head) into its tile, by one wave (`lane` =
// 0..63): lanes 0..15 copy the key's 16 K pieces, and every lane stores 2 of
// its 128 V elements (2-byte stores: the 8 keys of a V piece can belong to
// different rows).  Units past the batch, and rows of a sequence the batch
// checks reject, write nothing.
__device__ __forceinline__ void pack_row_key(const PackRowsArgs &a, int64_t unit, int lane) {
    if (unit >= (int64_t)a.b.total_rows * a.H) return;
    const int r = (int)(unit / a.H), g = (int)(unit % a.H);
    const int s = locate_seq(a.b.cu_rows, a.b.n_seqs, r);
    const int rows_s = a.b.cu_rows[s + 1] - a.b.cu_rows[s];
    const int L = a.b.seq_lens[s];
    if (rows_s <= 0 || rows_s > L || L > a.b.max_seq_len) return;
    const int p = L - rows_s + (r - a.b.cu_rows[s]);
    const int64_t t = block_token0(a.b, s, seq_token0(a.b, s), p / 64) + p % 64;
    const int j = (int)(t & 63), jj = j & 31;                 // key of the tile, of its chunk
    const int64_t tile = (t >> 6) * a.t_blk + (int64_t)g * a.t_head + 4096 * (j >> 5);
    const int64_t src = t * a.tok + (int64_t)g * a.head;
    if (lane < 16) {
        const int s4 = lane >> 2, lg = lane & 3;
        const int q = 256 * (jj >> 4) + 64 * s4 + 16 * lg + (jj & 15);
        *reinterpret_cast<u32x4 *>(a.kt + tile + 8 * q) = load16(a.k + src + 32 * s4 + 8 * lg);
    }
    const int lg = (jj & 15) >> 2, e = 4 * (jj >> 4) + (jj & 3);   // V: lane group and element of the key
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int d = 2 * lane + h;
        const int q = 64 * (d >> 4) + 16 * lg + (d & 15);
        a.vt[tile + 8 * q + e] = a.v[src + d];
    }
}

}  // namespace msa
