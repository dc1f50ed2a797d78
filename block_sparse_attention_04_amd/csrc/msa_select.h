// msa_select.h -- device code of the top-k block selection, shared by the
// selection kernel and the fused index-and-select kernel.
//
// Per (row, key head): keep the row's local block and the top_k-1 highest
// block scores among the earlier blocks; equal scores keep the lower block
// index; rows with at most top_k causal blocks keep all of them.  Output is
// ascending and padded with -1.  Scores become order-preserving 32-bit keys,
// so every comparison is exact integer work.
#pragma once

#include "msa_device.h"

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

// Largest T with #{lanes: v >= T} >= k (the k-th largest of 64 values), one
// bit per step (one ballot each: fewer vector instructions than wider steps).
// With kLowBit > 0 only bits 31..kLowBit are decided: the result is the k-th
// largest of the values with their low kLowBit bits cleared -- a lower bound
// on the exact one, in fewer steps.
template <int kLowBit = 0>
__device__ __forceinline__ uint32_t kth_largest_wave(uint32_t v, int k) {
    uint32_t t = 0u;
#pragma unroll
    for (int bit = 31; bit >= kLowBit; --bit) {
        const uint32_t c = t | (1u << bit);
        t = __popcll(__ballot(v >= c)) >= k ? c : t;
    }
    return t;
}

// Whether this lane's entry of a list of n <= 64 order keys (lane l holds
// entry l, in index order; 0 past the list) is among the top `need`, ties to
// the lower index.  Short lists: its rank -- the keys above it, plus equal
// keys earlier in the list -- is below `need`, each lane counting over the
// list on its own (n steps, none of them a cross-lane round).  Longer lists:
// T, the need-th largest key, by one ballot per bit (32 cross-lane rounds),
// then the keys above T and the first equal ones.  The same entries either way
// (the ranks measured faster up to 16 entries: chunk selection 21.3 -> 20.9 us;
// at 24-32 the 2,048-row prefill's 31-entry lists lost 0.3-0.6 us a step).
constexpr int kRankListMax = 16;
__device__ __forceinline__ bool top_keep(uint32_t v, int n, int need) {
    const int lane = threadIdx.x & 63;
    if (n <= kRankListMax) {
        int rank = 0;
#pragma unroll 4
        for (int i = 0; i < n; ++i) {
            const uint32_t k = (uint32_t)__builtin_amdgcn_readlane((int)v, i);
            rank += k > v || (k == v && i < lane) ? 1 : 0;
        }
        return lane < n && rank < need;
    }
    const uint32_t t = kth_largest_wave(v, need);
    const int need_eq = need - __popcll(__ballot(v > t));
    const uint64_t em = __ballot(lane < n && v == t);
    return v > t || (lane < n && v == t && lanes_below(em) < need_eq);
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
        // one key per lane, already in index order
        const uint32_t cv = lane < n ? keys[lane] : 0u;
        const bool take = top_keep(cv, n, need);
        const uint64_t tm = __ballot(take);
        if (take) emit(lanes_below(tm), cv, idx_of(lane));
        return;
    }
    uint32_t lmax = 0u;
#pragma unroll 8
    for (int j = lane; j < n; j += kWave) lmax = max(lmax, keys[j]);
    // T0: a lower bound on T (need lanes hold a key >= it), decided on the
    // top 16 bits only; keys in T0's 2^16-wide bucket just add candidates.
    const uint32_t t0 = kth_largest_wave<16>(lmax, need);

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
        const bool take = top_keep(cv, c, need);
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

// Stage order keys of scores S[0..n) into LDS (a burst of independent loads;
// nontemporal: every score is read once, and the caches are better left to
// the attention that follows).
__device__ __forceinline__ void stage_keys(uint32_t *dst, const float *S, int n, int from, int step) {
#pragma unroll 16
    for (int j = from; j < n; j += step) dst[j] = order_key(__builtin_nontemporal_load(S + j));
}

// As stage_keys, reading the scores with device-scoped loads (scores stored
// by other workgroups of the same launch with device-scoped stores).
// Loads go out in bursts of 16 before any of them is used.
__device__ __forceinline__ void stage_keys_coherent(uint32_t *dst, const float *S, int n, int from, int step) {
    for (int j0 = from; j0 < n; j0 += 16 * step) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int j = min(j0 + q * step, n - 1);     // past the end: re-read the last score
            v[q] = __hip_atomic_load(S + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if (j0 + q * step < n) dst[j0 + q * step] = order_key(v[q]);
    }
}

// LDS scratch of the workgroup-mode selection.
struct SelScratch {
    uint32_t ck[4][64];
    int32_t ci[4][64];
    uint32_t mk[4 * kMaxTopK];
    int32_t mi[4 * kMaxTopK];
};

// One unit with nb causal blocks whose first nb-1 order keys are staged in
// keys[] (LDS, visible to the workgroup once the caller's stores are done),
// selected by all 4 waves of the workgroup: each wave takes the top top_k-1 of
// its quarter, then wave 0 selects among those 4*(top_k-1) -- every kept block
// is in its quarter's top, with the same tie order, so the result is the same
// as one pass over all blocks.  Writes out[0..top_k).  Called by every thread.
__device__ __forceinline__ void select_unit_wg(const uint32_t *keys, int nb, int top_k, int32_t *out,
                                               SelScratch &sc) {
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int n = nb - 1, need = top_k - 1;
    if (nb <= top_k || need == 0) {       // all causal blocks, or only the local one
        if (wave == 0 && lane < top_k) out[lane] = nb <= top_k ? (lane < nb ? lane : -1) : n;
        return;
    }
    __syncthreads();
    const int seg = (n + 3) / 4;
    const int j0 = wave * seg, n_seg = max(0, min(seg, n - j0));
    uint32_t *mkw = sc.mk + wave * need;
    int32_t *miw = sc.mi + wave * need;
    if (n_seg <= need) {
        for (int j = lane; j < need; j += kWave) {
            mkw[j] = j < n_seg ? keys[j0 + j] : 0u;     // 0 sorts below every score
            miw[j] = j < n_seg ? j0 + j : -1;
        }
    } else {
        wave_top(keys + j0, n_seg, need, [j0](int j) { return j0 + j; },
                 [&](int pos, uint32_t k, int idx) { mkw[pos] = k; miw[pos] = idx; }, sc.ck[wave], sc.ci[wave]);
    }
    __syncthreads();
    if (wave == 0) {
        wave_top(sc.mk, 4 * need, need, [&](int j) { return sc.mi[j]; },
                 [&](int pos, uint32_t, int idx) { out[pos] = idx; }, sc.ck[0], sc.ci[0]);
        if (lane == 0) out[need] = n;
    }
}

// One unit selected by one wave (keys staged by this wave).  Writes out[0..top_k).
__device__ __forceinline__ void select_unit_wave(const uint32_t *keys, int nb, int top_k, int32_t *out,
                                                 uint32_t *ck, int32_t *ci) {
    const int lane = threadIdx.x & 63;
    const int n = nb - 1, need = top_k - 1;
    if (nb <= top_k || need == 0) {
        if (lane < top_k) out[lane] = nb <= top_k ? (lane < nb ? lane : -1) : n;
        return;
    }
    wave_lds_sync();
    wave_top(keys, n, need, [](int j) { return j; }, [&](int pos, uint32_t, int idx) { out[pos] = idx; }, ck, ci);
    if (lane == 0) out[need] = n;
}

}  // namespace msa
