// kvcache.hip -- writing the int8 and the tiled key/value caches.
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

// Tiled cache writer.  A tile is one key head's 64 keys of one block (K or V,
// 8,192 elements); chunk c = 0, 1 (keys 32c .. 32c + 31) fills elements
// 4096c .. 4096c + 4095 as 512 pieces of 8 elements, piece q at 8q:
//   K: q = 256*mt + 64*s + lane -> key 32c + 16*mt + lane%16,
//      dims 32*s + 8*(lane/16) + 0..7 (the attention's QK^T A operands);
//   V: q = 64*dt + lane -> dim 16*dt + lane%16 of keys 32c + 4*(lane/16) + 0..3,
//      then 32c + 16 + 4*(lane/16) + 0..3 (its PV A operands).
// One thread per 16-byte piece of the tiles the token range touches; pieces
// (or, for V, elements) of tokens outside the range are left as they are.
__global__ __launch_bounds__(256) void pack_kv_tiled_kernel(PackTiledArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int piece = (int)(i % 2048);                 // 0..1023 K, 1024..2047 V
    const int64_t bh = i / 2048;
    if (bh >= a.n_blocks * a.H) return;
    const int g = (int)(bh % a.H);
    const int64_t tb = a.tok_begin / 64 + bh / a.H;    // the tile's block
    const int q = piece & 1023, c = q >> 9, lane = q & 63, lg = lane >> 4, lr = lane & 15;
    const int64_t key0 = tb * 64 + 32 * c;             // token of the chunk's first key
    const int64_t dst = tb * a.t_blk + (int64_t)g * a.t_head + 8 * q;
    if (piece < 1024) {
        const int mt = (q >> 8) & 1, s = (q >> 6) & 3;
        const int64_t t = key0 + 16 * mt + lr;
        if (t < a.tok_begin || t >= a.tok_end) return;
        *reinterpret_cast<u32x4 *>(a.kt + dst) = load16(a.k + t * a.tok + (int64_t)g * a.head + 32 * s + 8 * lg);
        return;
    }
    const int dim = 16 * ((q >> 6) & 7) + lr;
    const int64_t t_lo = key0 + 4 * lg, t_hi = key0 + 16 + 4 * lg;   // keys of elements 0..3, 4..7
    const bool all_in = t_lo >= a.tok_begin && t_hi + 3 < a.tok_end;
    const bool none_in = t_hi + 3 < a.tok_begin || t_lo >= a.tok_end ||
                         (t_lo + 3 < a.tok_begin && t_hi >= a.tok_end);
    if (none_in) return;
    u32x4 w = all_in ? zero16() : load16(a.vt + dst);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t t = (e < 4 ? t_lo : t_hi) + (e & 3);
        if (t < a.tok_begin || t >= a.tok_end) continue;
        const uint32_t x = a.v[t * a.tok + (int64_t)g * a.head + dim];
        const int sh = 16 * (e & 1);
        w[e >> 1] = (w[e >> 1] & ~(0xffffu << sh)) | (x << sh);
    }
    *reinterpret_cast<u32x4 *>(a.vt + dst) = w;
}

hipError_t launch_pack_kv_tiled(const PackTiledArgs &a, hipStream_t st) {
    const int64_t threads = a.n_blocks * a.H * 2048;
    hipLaunchKernelGGL(pack_kv_tiled_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_quantize_kv8(const QuantArgs &a, hipStream_t st) {
    const int64_t rows = a.n_tokens * a.H;
    hipLaunchKernelGGL(quantize_kv8_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace msa
