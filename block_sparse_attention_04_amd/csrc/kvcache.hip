// kvcache.hip -- writing the int8 key/value cache.
//
// The cache keeps keys and values as int8 codes with one fp32 scale per
// (token, key head) (TensorFold pull request 1388, commit adding the
// minimax_m3 family: keys and values cached as int8 with a scale a position
// and head).  The rule that makes a row's codes is this library's reading (the
// pages name the scale, not its rule), taken in fp32:
//   scale  = max_d |x_d| / 127
//   code_d = round_half_even(x_d / scale), clamped to [-127, 127]
// A row of zeros gets scale 0 and codes 0.  The divisions are IEEE
// (correctly rounded), so the codes are a function of the bf16 row alone.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// 16 lanes per (token, key head) row: lane q of the row holds dims 8q..8q+7.
__global__ __launch_bounds__(256) void quantize_kv8_kernel(QuantArgs a) {
    const int q = threadIdx.x & 15;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;   // token * H + head
    const bool valid = row < a.n_tokens * a.H;
    const int64_t t = valid ? row / a.H : 0;
    const int g = valid ? (int)(row % a.H) : 0;
    const u32x4 x = valid ? load16(a.x + t * a.tok + (int64_t)g * a.head + 8 * q) : zero16();
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(x[i] << 16);
        f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));   // the row's 16 lanes
    const float sc = amax / 127.0f;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float c = 0.f;
        if (sc != 0.f) c = fminf(fmaxf(rintf(f[i] / sc), -127.f), 127.f);
        w[i >> 2] |= (uint32_t)(uint8_t)(int8_t)(int)c << (8 * (i & 3));
    }
    if (!valid) return;
    *reinterpret_cast<uint2 *>(a.codes + t * a.ctok + (int64_t)g * a.chead + 8 * q) = make_uint2(w[0], w[1]);
    if (q == 0) a.scales[t * a.stok + (int64_t)g * a.shead] = sc;
}

hipError_t launch_quantize_kv8(const QuantArgs &a, hipStream_t st) {
    const int64_t rows = a.n_tokens * a.H;
    hipLaunchKernelGGL(quantize_kv8_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace msa
