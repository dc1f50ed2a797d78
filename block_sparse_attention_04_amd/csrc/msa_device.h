// msa_device.h -- device-side helpers shared by the library's kernels
// (gfx950 / CDNA4, wave64).  Library-internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace msa {

constexpr int kWave = 64;
constexpr int kGroup = 16;      // query heads per key head
constexpr int kHeadDim = 128;   // q/k/v head dim
constexpr int kIndexDim = 64;   // indexer dim
constexpr int kBlock = 64;      // keys per block
constexpr int kMaxTopK = 32;
constexpr int64_t kMaxKvTokStride = int64_t(1) << 24;   // elements between consecutive tokens of k/v
constexpr int kMaxSelectBlocks = 16384;  // selection stages a row's block scores in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even, on the
// hardware converter (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const floatx2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// D = A * B + C on one 16x16x32 bf16 MFMA.
// Lane layout (wave64): A supplies row (lane % 16) and the 8 k-values of
// lane group (lane / 16); B supplies column (lane % 16) and the same 8
// k-values of its lane group; D lane holds column (lane % 16), rows
// 4*(lane/16) + 0..3.  A and B share the k assignment, so any consistent
// relabelling of k across the two operands computes the same contraction.
__device__ __forceinline__ floatx4 mfma_16x16x32(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x4 zero16() {
    u32x4 z = {0u, 0u, 0u, 0u};
    return z;
}

// Sequence owning global row r: the last s with cu_rows[s] <= r.
__device__ __forceinline__ int locate_seq(const int32_t *cu_rows, int n_seqs, int r) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu_rows[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Reductions across the four lanes l, l^16, l^32, l^48 that share a column
// of an MFMA result, on the VALU: v_permlane16_swap pairs lane rows (l, l^16)
// and v_permlane32_swap pairs halves (l, l^32); with both operands equal, the
// two results of each swap hold the pair's two values on every lane.
__device__ __forceinline__ float max_over_lane_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Four values reduced over the 4 lane groups at once and scattered: lane
// group g receives the maximum of a_g over the groups (for its lane % 16).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, v_permlane16_swap the odd 16-lane rows of the
// first with the even rows of the second.
__device__ __forceinline__ float max_scatter_lane_groups(float a0, float a1, float a2, float a3) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a2), false, false);
    const float m02 = fmaxf(__uint_as_float(s02[0]), __uint_as_float(s02[1]));   // groups 0,1: a0; 2,3: a2
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a1), __float_as_uint(a3), false, false);
    const float m13 = fmaxf(__uint_as_float(s13[0]), __uint_as_float(s13[1]));   // groups 0,1: a1; 2,3: a3
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(m02), __float_as_uint(m13), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float sum_over_lane_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Make the compiler complete the loads that produced x here (an empty asm
// that reads x): a software-pipelined loop that later uses x then never
// waits on it, which would also wait for the loop's own prefetches.
__device__ __forceinline__ void force_ready(const u32x4 &x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void force_ready(int x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Make LDS writes of this wave visible to its own later LDS reads (and keep
// the compiler from moving LDS accesses across this point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace msa
