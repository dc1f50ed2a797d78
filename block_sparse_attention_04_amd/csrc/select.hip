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
//   1. T0 = the (top_k-1)-th largest of the 64 per-lane maxima -- a lower
//      bound on T, since top_k-1 lanes hold a value >= T0;
//   2. the candidates >= T0 (usually a few dozen) are compacted into LDS and
//      T is found among them by a 32-step bitwise search over one key per
//      lane; if more than 64 candidates tie above T0, the same search runs
//      over all scores instead;
//   3. one pass in ascending block order keeps every key > T and the first
//      (lowest-index) keys == T until top_k-1 are kept; the local block
//      closes the list.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// Monotone map float -> uint32 (x < y  <=>  key(x) < key(y)); -0 maps as +0.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Largest T with #{lanes: v >= T} >= k (the k-th largest of 64 values).
__device__ __forceinline__ uint32_t kth_largest_wave(uint32_t v, int k) {
    uint32_t t = 0u;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = t | (1u << bit);
        if (__popcll(__ballot(v >= c)) >= k) t = c;
    }
    return t;
}

// Scores of the unit live in LDS (one burst of independent loads) when they
// fit the per-wave capacity `cap`; otherwise every pass reads them from global
// memory (L2-resident after the first).
template <bool kStaged>
__device__ __forceinline__ void select_unit(const SelectArgs &a, const float *S, float *lds, int n,
                                            int need, int32_t *out, uint32_t *cand) {
    const int lane = threadIdx.x & 63;
    auto key_at = [&](int b) -> uint32_t { return order_key(kStaged ? lds[b] : S[b]); };

    uint32_t lmax = 0u;
#pragma unroll 8
    for (int b = lane; b < n; b += kWave) lmax = max(lmax, key_at(b));
    const uint32_t t0 = kth_largest_wave(lmax, need);

    int c = 0;
    for (int b0 = 0; b0 < n; b0 += kWave) {
        const int b = b0 + lane;
        const uint32_t v = b < n ? key_at(b) : 0u;
        const bool f = b < n && v >= t0;
        const uint64_t mk = __ballot(f);
        const int pos = c + lanes_below(mk);
        if (f && pos < kWave) cand[pos] = v;
        c += __popcll(mk);
    }

    uint32_t t;
    int n_gt;
    if (c <= kWave) {
        wave_lds_sync();
        const uint32_t cv = lane < c ? cand[lane] : 0u;
        t = kth_largest_wave(cv, need);
        n_gt = __popcll(__ballot(cv > t));
    } else {
        t = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cb = t | (1u << bit);
            int cnt = 0;
#pragma unroll 8
            for (int b = lane; b < n; b += kWave) cnt += key_at(b) >= cb;
            if (wave_sum_int(cnt) >= need) t = cb;
        }
        int cnt = 0;
#pragma unroll 8
        for (int b = lane; b < n; b += kWave) cnt += key_at(b) > t;
        n_gt = wave_sum_int(cnt);
    }

    const int need_eq = need - n_gt;
    int taken = 0, eq_seen = 0;
    for (int b0 = 0; b0 < n; b0 += kWave) {
        const int b = b0 + lane;
        const bool valid = b < n;
        const uint32_t v = valid ? key_at(b) : 0u;
        const bool gt = valid && v > t;
        const bool eq = valid && v == t;
        const uint64_t em = __ballot(eq);
        const bool take = gt || (eq && eq_seen + lanes_below(em) < need_eq);
        const uint64_t tm = __ballot(take);
        if (take) out[taken + lanes_below(tm)] = b;
        taken += __popcll(tm);
        eq_seen += __popcll(em);
    }
    if (lane == 0) out[need] = n;  // the local block, largest index, last
}

__global__ __launch_bounds__(256) void select_blocks_kernel(SelectArgs a, int cap) {
    extern __shared__ float dyn[];             // [4 waves][cap] staged scores
    __shared__ uint32_t cand[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave;
    if (unit >= (int64_t)a.b.total_rows * a.H) return;
    const int r = (int)(unit / a.H);
    int32_t *out = a.idx + unit * a.top_k;

    const int s = locate_seq(a.b.cu_rows, a.b.n_seqs, r);
    const int rows_s = a.b.cu_rows[s + 1] - a.b.cu_rows[s];
    const int L = a.b.seq_lens[s];
    if (rows_s <= 0 || rows_s > L || L > a.b.max_seq_len) return;
    const int p = L - rows_s + (r - a.b.cu_rows[s]);
    const int nb = p / kBlock + 1;

    if (nb <= a.top_k) {
        if (lane < a.top_k) out[lane] = lane < nb ? lane : -1;
        return;
    }
    const float *S = a.scores + unit * a.bs_stride;
    const int n = nb - 1;          // candidates: blocks 0 .. nb-2
    const int need = a.top_k - 1;  // how many of them to keep
    if (n <= cap) {
        float *lds = dyn + wave * cap;
#pragma unroll 8
        for (int b = lane; b < n; b += kWave) lds[b] = S[b];
        wave_lds_sync();
        select_unit<true>(a, S, lds, n, need, out, cand[wave]);
    } else {
        select_unit<false>(a, S, nullptr, n, need, out, cand[wave]);
    }
}

hipError_t launch_select_blocks(const SelectArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.b.total_rows * a.H;
    // stage up to 4,096 candidate blocks (262,144 keys) per unit in LDS
    const int need = (a.b.max_seq_len + kBlock - 1) / kBlock;
    const int cap = ((min(need, 4096) + 63) / 64) * 64;
    dim3 grid((unsigned)((units + 3) / 4));
    hipLaunchKernelGGL(select_blocks_kernel, grid, dim3(256), (size_t)4 * cap * sizeof(float), st, a, cap);
    return hipGetLastError();
}

}  // namespace msa
