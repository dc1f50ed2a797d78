// peaks.hip -- measurement kernels (include/msa_peaks.h): the HBM read rate
// and the bf16 MFMA rate the device sustains, reported beside the published
// peaks.  Not part of the method.
#include <stdarg.h>
#include <stdio.h>

#include "msa.h"
#include "msa_device.h"
#include "msa_launch.h"
#include "msa_peaks.h"

namespace msa {

// Grid-stride read of n16 16-byte words, four independent loads in flight per
// thread per iteration; the words are folded into one value that is stored
// only if it happens to equal a constant, so no load can be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *p, int64_t n16, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) + (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const u32x4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// The same read with the knobs a streaming kernel has: U loads in flight per
// thread per iteration, loads of W = sizeof(T) bytes, plain or nontemporal
// loads (the grid is the caller's).  Swept by the benchmark to find the best
// read rate the device sustains.
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fold_word(uint32_t x) { return x; }
__device__ __forceinline__ uint32_t fold_word(u32x2v x) { return x.x ^ x.y; }
__device__ __forceinline__ uint32_t fold_word(u32x4 x) { return x.x ^ x.y ^ x.z ^ x.w; }

template <int U, typename T, bool NT>
__device__ __forceinline__ T read_word(const T *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int U, typename T, bool NT>
__global__ __launch_bounds__(256) void stream_read_variant_kernel(const T *p, int64_t n, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        T v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = read_word<U, T, NT>(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc += fold_word(v[u]);
    }
    for (; i < n; i += stride) acc ^= fold_word(read_word<U, T, NT>(p + i));
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Four independent accumulation chains per wave, so the MFMA pipeline never
// waits on a result; operands depend on the lane so nothing folds away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float *sink, int iters) {
    const uint32_t t = threadIdx.x & 63;
    const uint32_t one = 0x3f803f80u;                   // two bf16 ones
    const u32x4 a = {one, one ^ (t << 3), one, one};    // lane-dependent low bits: small values
    const u32x4 b = {one, one, one ^ (t << 2), one};
    floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int i = 0; i < iters; ++i) {
        c0 = mfma_16x16x32(a, b, c0);
        c1 = mfma_16x16x32(b, a, c1);
        c2 = mfma_16x16x32(a, a, c2);
        c3 = mfma_16x16x32(b, b, c3);
    }
    const float s = c0[0] + c1[1] + c2[2] + c3[3];
    if (s == 1234.5f) sink[threadIdx.x] = s;
}

}  // namespace msa

namespace {
int peaks_fail(int code, const char *fmt, ...) {
    char msg[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    return msa::report(code, msg);
}
int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return peaks_fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return msa::report(MSA_OK, "");
}
}  // namespace

extern "C" int msa_peaks_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink) return peaks_fail(MSA_ERR_INVALID, "stream_read: NULL buffer");
    if (bytes <= 0 || (bytes & 15) != 0 || ((uintptr_t)buf & 15u) != 0)
        return peaks_fail(MSA_ERR_INVALID, "stream_read: bytes=%lld must be > 0, a multiple of 16, 16-byte aligned",
                          (long long)bytes);
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 256 * 16 ? blocks : 256 * 16);   // 16 workgroups per CU
    hipLaunchKernelGGL(msa::stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(buf), n16, sink);
    return launched(hipGetLastError(), "stream_read");
}

namespace {
template <int U, typename T>
void launch_variant(const void *buf, int64_t n, uint32_t *sink, bool nt, unsigned grid, hipStream_t st) {
    if (nt) hipLaunchKernelGGL((msa::stream_read_variant_kernel<U, T, true>), dim3(grid), dim3(256), 0, st,
                               static_cast<const T *>(buf), n, sink);
    else hipLaunchKernelGGL((msa::stream_read_variant_kernel<U, T, false>), dim3(grid), dim3(256), 0, st,
                            static_cast<const T *>(buf), n, sink);
}
template <typename T>
void launch_unroll(int unroll, const void *buf, int64_t n, uint32_t *sink, bool nt, unsigned grid, hipStream_t st) {
    switch (unroll) {
        case 1: launch_variant<1, T>(buf, n, sink, nt, grid, st); break;
        case 2: launch_variant<2, T>(buf, n, sink, nt, grid, st); break;
        case 4: launch_variant<4, T>(buf, n, sink, nt, grid, st); break;
        case 8: launch_variant<8, T>(buf, n, sink, nt, grid, st); break;
        default: launch_variant<16, T>(buf, n, sink, nt, grid, st); break;
    }
}
}  // namespace

extern "C" int msa_peaks_stream_read_variant(const void *buf, int64_t bytes, uint32_t *sink, int32_t unroll,
                                             int32_t width, int32_t nontemporal, int32_t wg_per_cu, void *stream) {
    if (!buf || !sink) return peaks_fail(MSA_ERR_INVALID, "stream_read_variant: NULL buffer");
    if (bytes <= 0 || (bytes & 15) != 0 || ((uintptr_t)buf & 15u) != 0)
        return peaks_fail(MSA_ERR_INVALID, "stream_read_variant: bytes=%lld must be > 0, a multiple of 16, "
                          "16-byte aligned", (long long)bytes);
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)
        return peaks_fail(MSA_ERR_INVALID, "stream_read_variant: unroll=%d not 1, 2, 4, 8 or 16", unroll);
    if (width != 4 && width != 8 && width != 16)
        return peaks_fail(MSA_ERR_INVALID, "stream_read_variant: width=%d not 4, 8 or 16", width);
    if (wg_per_cu < 1 || wg_per_cu > 64)
        return peaks_fail(MSA_ERR_INVALID, "stream_read_variant: wg_per_cu=%d outside [1, 64]", wg_per_cu);
    const int64_t n = bytes / width;
    const int64_t blocks = (n + 255) / 256;
    const int64_t cap = 256LL * wg_per_cu;
    const unsigned grid = (unsigned)(blocks < cap ? blocks : cap);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const bool nt = nontemporal != 0;
    if (width == 4) launch_unroll<uint32_t>(unroll, buf, n, sink, nt, grid, st);
    else if (width == 8) launch_unroll<msa::u32x2v>(unroll, buf, n, sink, nt, grid, st);
    else launch_unroll<u32x4>(unroll, buf, n, sink, nt, grid, st);
    return launched(hipGetLastError(), "stream_read_variant");
}

extern "C" int msa_peaks_mfma(float *sink, int32_t workgroups, int32_t iters, void *stream) {
    if (!sink) return peaks_fail(MSA_ERR_INVALID, "mfma: NULL sink");
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20))
        return peaks_fail(MSA_ERR_INVALID, "mfma: workgroups=%d iters=%d outside [1, 2^20]", workgroups, iters);
    hipLaunchKernelGGL(msa::mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), sink, iters);
    return launched(hipGetLastError(), "mfma");
}
