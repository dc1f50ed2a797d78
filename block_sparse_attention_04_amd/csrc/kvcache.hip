// kvcache.hip -- writing the int8 and the tiled key/value caches.
//
// The cache keeps keys and values as int8 codes with one fp32 scale per
// (token, key head) (TensorFold pull request 1388, commit adding the
// minimax_m3 family, which describes an int8 key/value cache scaled per
// position and key head).  The rule that makes a row's codes is this library's reading (the
// pages name the scale, not its rule), taken in fp32:
//   scale  = max_d |x_d| / 127
//   code_d = round_half_even(x_d / scale), clamped to [-127, 127]
// A row of zeros gets scale 0 and codes 0.  The divisions are IEEE
// (correctly rounded), so the codes are a function of the bf16 row alone.
#include "msa_device.h"
#include "msa_launch.h"
#include "msa_pack.h"

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
// One workgroup per (block, key head, 32-key chunk).  K pieces are 16-byte
// copies; the chunk's V rows are first staged in LDS with coalesced 16-byte
// loads, then each V piece gathers its 8 keys of one dim from there.  Pieces
// (for V, elements) of tokens outside the range are left as they are.
constexpr int kPackRow = 128 + 8;   // staged V row (elements), padded against bank conflicts

__global__ __launch_bounds__(256) void pack_kv_tiled_kernel(PackTiledArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vs[32 * kPackRow];
    const int c = blockIdx.x & 1;                             // the chunk of the tile
    const int64_t bh = blockIdx.x >> 1;
    const int g = (int)(bh % a.H);
    const int64_t tb = a.tok_begin / 64 + bh / a.H;           // the tile's block
    const int64_t key0 = tb * 64 + 32 * c;                    // token of the chunk's first key
    const int64_t chunk = tb * a.t_blk + (int64_t)g * a.t_head + 4096 * c;
    auto in_range = [&](int64_t t) { return t >= a.tok_begin && t < a.tok_end; };
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i = r * 256 + threadIdx.x;
        // V row `key` of the chunk, 16-byte unit pc, into LDS
        const int key = i >> 4, pc = i & 15;
        if (in_range(key0 + key))
            *reinterpret_cast<u32x4 *>(vs + key * kPackRow + 8 * pc) =
                load16(a.v + (key0 + key) * a.tok + (int64_t)g * a.head + 8 * pc);
        // K piece i of the chunk: operand (mt, s), lane
        const int mt = (i >> 8) & 1, s = (i >> 6) & 3, lane = i & 63;
        const int64_t tk = key0 + 16 * mt + (lane & 15);
        if (in_range(tk))
            *reinterpret_cast<u32x4 *>(a.kt + chunk + 8 * i) =
                load16(a.k + tk * a.tok + (int64_t)g * a.head + 32 * s + 8 * (lane >> 4));
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        // V piece q of the chunk: d-tile dt, lane
        const int q = r * 256 + threadIdx.x;
        const int lane = q & 63, lg = lane >> 4;
        const int dim = 16 * ((q >> 6) & 7) + (lane & 15);
        const int k_lo = 4 * lg, k_hi = k_lo + 16;              // keys of elements 0..3 and 4..7
        const bool lo_in = in_range(key0 + k_lo) && in_range(key0 + k_lo + 3);
        const bool hi_in = in_range(key0 + k_hi) && in_range(key0 + k_hi + 3);
        auto meets = [&](int k) { return key0 + k < a.tok_end && key0 + k + 3 >= a.tok_begin; };
        if (!meets(k_lo) && !meets(k_hi)) continue;
        uint16_t *dst = a.vt + chunk + 8 * q;
        u32x4 w = lo_in && hi_in ? zero16() : load16(dst);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = (e < 4 ? k_lo : k_hi) + (e & 3);
            if (!in_range(key0 + key)) continue;
            const uint32_t x = vs[key * kPackRow + dim];
            const int sh = 16 * (e & 1);
            w[e >> 1] = (w[e >> 1] & ~(0xffffu << sh)) | (x << sh);
        }
        *reinterpret_cast<u32x4 *>(dst) = w;
    }
}

hipError_t launch_pack_kv_tiled(const PackTiledArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(pack_kv_tiled_kernel, dim3((unsigned)(a.n_blocks * a.H * 2)), dim3(256), 0, st, a);
    return hipGetLastError();
}

// The batch's own keys (key p of every row) into their tiles: one wave per
// (row, key head), pack_row_key's work.
__global__ __launch_bounds__(256) void pack_kv_rows_kernel(PackRowsArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    pack_row_key(a, gid >> 6, (int)(gid & 63));
}

hipError_t launch_pack_kv_rows(const PackRowsArgs &a, hipStream_t st) {
    const int64_t threads = (int64_t)a.b.total_rows * a.H * 64;
    hipLaunchKernelGGL(pack_kv_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_quantize_kv8(const QuantArgs &a, hipStream_t st) {
    const int64_t rows = a.n_tokens * a.H;
    hipLaunchKernelGGL(quantize_kv8_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace msa
