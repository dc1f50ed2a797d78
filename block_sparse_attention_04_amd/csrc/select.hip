// select.hip -- top-k block selection with a forced local block.
//
// Per (row, key head): keep the row's local block and the top_k-1 highest
// block scores among the earlier blocks; equal scores keep the lower block
// index; rows with at most top_k causal blocks keep all of them.  Output is
// ascending and padded with -1.  ("minimax-m3-sm120", What this fixes:
// top-16 block selection per GQA group with a forced local block; TensorFold
// pull request 1388, commit adding the minimax_m3 family: the selection is
// per row and key head.  Tie order and the local block counting inside the
// 16 are this library's readings.)
//
// One wave per (row, key head).  Scores become order-preserving 32-bit keys
// (so every comparison is exact integer work); the (top_k-1)-th largest key T
// is found with ballot counts:
//   1. T0 = the (top_k-1)-th largest of the 64 per-lane maxima, decided on
//      their top 16 bits -- a lower bound on T, since top_k-1 lanes hold a
//      value >= T0;
//   2. the candidates >= T0 (usually a few dozen) are compacted into LDS, one
//      key per lane in block order; up to 16 of them are kept by their rank
//      (keys above, plus equal keys earlier in the list), more by a 32-step
//      bitwise search for T and then every key > T and the first
//      (lowest-index) keys == T; if more than 64 candidates tie above T0, the
//      search runs over all scores instead;
//   3. the kept blocks are written in ascending block order until top_k-1 are
//      kept; the local block closes the list.
#include "msa_launch.h"
#include "msa_select.h"

namespace msa {

struct SelUnit {
    int64_t unit;
    int n;        // candidate blocks 0..n-1 (n = nb - 1); the local block is n
    bool direct;  // nb <= top_k: keep everything, no scores needed
    bool ok;
};

__device__ __forceinline__ SelUnit sel_unit(const SelectArgs &a, int64_t unit) {
    SelUnit u;
    u.unit = unit;
    const int r = (int)(unit / a.H);
    const int s = locate_seq(a.b.cu_rows, a.b.n_seqs, r);
    const int rows_s = a.b.cu_rows[s + 1] - a.b.cu_rows[s];
    const int L = a.b.seq_lens[s];
    u.ok = rows_s > 0 && rows_s <= L && L <= a.b.max_seq_len;
    const int p = L - rows_s + (r - a.b.cu_rows[s]);
    const int nb = p / kBlock + 1;
    u.n = nb - 1;
    u.direct = nb <= a.top_k;
    return u;
}

template <bool kMulti>
__global__ __launch_bounds__(256) void select_blocks_kernel(SelectArgs a, int cap) {
    extern __shared__ uint32_t dyn[];
    __shared__ SelScratch sc;
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int64_t units = (int64_t)a.b.total_rows * a.H;
    const int64_t unit = kMulti ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * 4 + wave;
    if (unit >= units) return;
    // Stage the unit's scores before its metadata arrives, so both go out in one
    // round of loads.  min(cap, bs_stride) entries stay inside the unit's row and
    // cover every causal block; entries past the row's count are never read.
    {
        const float *S = a.scores + unit * a.bs_stride;
        const int n_stage = min(cap, a.bs_stride);
        if (kMulti) stage_keys(dyn, S, n_stage, threadIdx.x, 256);
        else stage_keys(dyn + wave * cap, S, n_stage, lane, kWave);
    }
    const SelUnit u = sel_unit(a, unit);
    if (!u.ok) return;
    int32_t *out = a.idx + unit * a.top_k;
    if (kMulti) select_unit_wg(dyn, u.n + 1, a.top_k, out, sc);
    else select_unit_wave(dyn + wave * cap, u.n + 1, a.top_k, out, sc.ck[wave], sc.ci[wave]);
}

hipError_t launch_select_blocks(const SelectArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.b.total_rows * a.H;
    const int nb_max = (a.b.max_seq_len + kBlock - 1) / kBlock;
    const int cap = ((nb_max + 63) / 64) * 64;      // staged keys per unit (<= kMaxSelectBlocks)
    // One wave per unit when there are many units and their 4 stages fit 64 KiB;
    // otherwise one workgroup per unit (its stage is at most 64 KiB).
    const bool multi = cap * 16 > 64 * 1024 || (units <= 1024 && nb_max > 256);
    if (multi) {
        hipLaunchKernelGGL(select_blocks_kernel<true>, dim3((unsigned)units), dim3(256),
                           (size_t)cap * sizeof(uint32_t), st, a, cap);
    } else {
        hipLaunchKernelGGL(select_blocks_kernel<false>, dim3((unsigned)((units + 3) / 4)), dim3(256),
                           (size_t)4 * cap * sizeof(uint32_t), st, a, cap);
    }
    return hipGetLastError();
}

}  // namespace msa
