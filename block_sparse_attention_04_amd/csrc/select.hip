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

// Largest T with #{lanes: v >= T} >= k (the k-th largest of 64 values),
// two bits per step: three independent ballots decide bits (b+1, b).
__device__ __forceinline__ uint32_t kth_largest_wave(uint32_t v, int k) {
    uint32_t t = 0u;
#pragma unroll
    for (int shift = 30; shift >= 0; shift -= 2) {
        const uint32_t c1 = t | (1u << shift), c2 = t | (2u << shift), c3 = t | (3u << shift);
        const int n3 = __popcll(__ballot(v >= c3));
        const int n2 = __popcll(__ballot(v >= c2));
        const int n1 = __popcll(__ballot(v >= c1));
        t = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : t;
    }
    return t;
}

// Top-`need` of keys[0..n) (order keys in LDS, n > need) for one wave, ties
// to the lower index.  idx_of(j) gives element j's block index; emit(pos, key,
// idx) receives the kept elements with pos = 0..need-1 in index order.
// ck/ci: this wave's 64-entry LDS scratch for candidates.
template <class IdxOf, class Emit>
__device__ __forceinline__ void wave_top(const uint32_t *keys, int n, int need, IdxOf idx_of, Emit emit,
                                         uint32_t *ck, int32_t *ci) {
    const int lane = threadIdx.x & 63;
    if (n <= kWave) {
        // one key per lane, already in index order: T directly
        const uint32_t cv = lane < n ? keys[lane] : 0u;
        const uint32_t t = kth_largest_wave(cv, need);
        const int need_eq = need - __popcll(__ballot(cv > t));
        const uint64_t em = __ballot(lane < n && cv == t);
        const bool take = cv > t || (lane < n && cv == t && lanes_below(em) < need_eq);
        const uint64_t tm = __ballot(take);
        if (take) emit(lanes_below(tm), cv, idx_of(lane));
        return;
    }
    uint32_t lmax = 0u;
#pragma unroll 8
    for (int j = lane; j < n; j += kWave) lmax = max(lmax, keys[j]);
    const uint32_t t0 = kth_largest_wave(lmax, need);

    int c = 0;
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int j = j0 + lane;
        const uint32_t v = j < n ? keys[j] : 0u;
        const bool f = j < n && v >= t0;
        const uint64_t mk = __ballot(f);
        const int pos = c + lanes_below(mk);
        if (f && pos < kWave) {
            ck[pos] = v;
            ci[pos] = idx_of(j);
        }
        c += __popcll(mk);
    }

    if (c <= kWave) {
        // every key >= T (the need-th largest) is a candidate, kept in index order
        wave_lds_sync();
        const uint32_t cv = lane < c ? ck[lane] : 0u;
        const int civ = lane < c ? ci[lane] : -1;
        const uint32_t t = kth_largest_wave(cv, need);
        const int need_eq = need - __popcll(__ballot(cv > t));
        const uint64_t em = __ballot(lane < c && cv == t);
        const bool take = cv > t || (lane < c && cv == t && lanes_below(em) < need_eq);
        const uint64_t tm = __ballot(take);
        if (take) emit(lanes_below(tm), cv, civ);
        return;
    }
    // Many ties above T0: bitwise search for T over all keys, then one pass in
    // index order.
    uint32_t t = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cb = t | (1u << bit);
        int cnt = 0;
#pragma unroll 8
        for (int j = lane; j < n; j += kWave) cnt += keys[j] >= cb;
        if (wave_sum_int(cnt) >= need) t = cb;
    }
    int cnt = 0;
#pragma unroll 8
    for (int j = lane; j < n; j += kWave) cnt += keys[j] > t;
    const int need_eq = need - wave_sum_int(cnt);
    int taken = 0, eq_seen = 0;
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int j = j0 + lane;
        const bool valid = j < n;
        const uint32_t v = valid ? keys[j] : 0u;
        const bool eq = valid && v == t;
        const uint64_t em = __ballot(eq);
        const bool take = (valid && v > t) || (eq && eq_seen + lanes_below(em) < need_eq);
        const uint64_t tm = __ballot(take);
        if (take) emit(taken + lanes_below(tm), v, idx_of(j));
        taken += __popcll(tm);
        eq_seen += __popcll(em);
    }
}

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

// Stage order keys of scores S[0..n) into LDS (a burst of independent loads).
__device__ __forceinline__ void stage_keys(uint32_t *dst, const float *S, int n, int from, int step) {
#pragma unroll 16
    for (int j = from; j < n; j += step) dst[j] = order_key(S[j]);
}

// kMulti = false: a workgroup of 4 waves takes 4 units, one wave each (many
// units).  kMulti = true: the 4 waves share one unit (few, long units): each
// selects the top top_k-1 of its quarter of the candidates, then wave 0
// selects among those 4*(top_k-1) -- every kept block is in its quarter's
// top, with the same tie order, so the result is the same.
template <bool kMulti>
__global__ __launch_bounds__(256) void select_blocks_kernel(SelectArgs a, int cap) {
    extern __shared__ uint32_t dyn[];
    __shared__ uint32_t ck[4][64];
    __shared__ int32_t ci[4][64];
    __shared__ uint32_t mk[4 * kMaxTopK];
    __shared__ int32_t mi[4 * kMaxTopK];
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
    const int need = a.top_k - 1;
    if (u.direct || need == 0) {            // all causal blocks, or only the local one
        if ((!kMulti || wave == 0) && lane < a.top_k) out[lane] = u.direct ? (lane <= u.n ? lane : -1) : u.n;
        return;
    }
    auto to_out = [&](int pos, uint32_t, int idx) { out[pos] = idx; };
    if (!kMulti) {
        uint32_t *keys = dyn + wave * cap;      // cap >= every row's candidate count
        wave_lds_sync();
        wave_top(keys, u.n, need, [](int j) { return j; }, to_out, ck[wave], ci[wave]);
        if (lane == 0) out[need] = u.n;
        return;
    }
    uint32_t *keys = dyn;
    __syncthreads();
    const int seg = (u.n + 3) / 4;
    const int j0 = wave * seg, n_seg = max(0, min(seg, u.n - j0));
    uint32_t *mkw = mk + wave * need;
    int32_t *miw = mi + wave * need;
    if (n_seg <= need) {
        for (int j = lane; j < need; j += kWave) {
            mkw[j] = j < n_seg ? keys[j0 + j] : 0u;     // 0 sorts below every score
            miw[j] = j < n_seg ? j0 + j : -1;
        }
    } else {
        wave_top(keys + j0, n_seg, need, [j0](int j) { return j0 + j; },
                 [&](int pos, uint32_t k, int idx) { mkw[pos] = k; miw[pos] = idx; }, ck[wave], ci[wave]);
    }
    __syncthreads();
    if (wave != 0) return;
    wave_top(mk, 4 * need, need, [&](int j) { return mi[j]; }, to_out, ck[0], ci[0]);
    if (lane == 0) out[need] = u.n;
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
