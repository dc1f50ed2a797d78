// attention.hip -- exact softmax attention over the kept blocks.
//
// For query head h of key head g = h / 16 and a row at position p:
//   out[h] = sum_j softmax_j(scale * q[h].k[j]) v[j]  over the kept blocks'
//   keys j <= p;  lse[h] = log sum_j exp(scale * q[h].k[j]).
// The 16 query heads of a key head share the row's selection, so a wave holds
// all 16 heads of one (row, key head) and reads every kept key/value once for
// all of them (TensorFold pull request 1388, commit on 4,096-row prompt
// chunks).  Decode splits the kept keys into partials merged by a log-sum-exp
// combine (same pull request, commit adding the minimax_m3 family, which cuts
// them in 32-key pieces; here a partial covers 4 kept blocks).
//
// Per kept 64-key block (bf16 caches), on v_mfma_f32_16x16x32_bf16:
//   S^T[key][head] = K Q^T      4 key tiles x 4 k-steps over the 128 dims
//   O^T[d][head]  += V^T P^T    8 d-tiles x two 32-key k-steps
// (the int8 cache folds 32-key chunks: 2 key tiles, one k-step).  With S^T, a
// lane holds one head's scores for 4 keys of each key tile, which is exactly
// the P^T operand layout of the second product, so probabilities go from the
// softmax straight into the MFMA without leaving registers, and the running
// max / sum / rescale of a head stay inside its 4 lanes.  A strided cache's V
// is written to LDS row-major (one 256-byte row per key, 32-byte column blocks
// XOR-swizzled by key mod 8) and each V^T operand is gathered by two
// transposing LDS reads (ds_read_b64_tr_b16); a tiled cache stores the
// operands ready.  Softmax runs in base 2 on scale*log2(e)-prescaled scores.
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

struct Softmax {
    floatx4 o[8];   // O^T: head (lane % 16), d = 16*dt + 4*(lane/16) + i
    float m;        // running max (log2 units); equal on the 4 lanes of a head
    float l;        // this lane's share of the running sum
};

__device__ __forceinline__ void softmax_init(Softmax &st) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
}

// V tile of one 32-key chunk in LDS: key k's 256-byte row at k*256, its
// 16-byte column unit u (dims 8u..8u+7) at unit u ^ (2 * (k % 8)).  With this
// swizzle the stores below and the transposing reads in fold_rows touch
// distinct banks.
__device__ __forceinline__ int v_unit(int key, int u) { return u ^ (2 * (key & 7)); }

// ds_read_b64_tr_b16: in each 16-lane group, lane 4a + c receives element c
// of the 4-element (8-byte) pieces addressed by lanes a, a+4, a+8, a+12.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t *p) {
    typedef short short4v __attribute__((ext_vector_type(4)));
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v *)(p));
    return make_uint2((uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16),
                      (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16));
}

// Query B operand of the 4 k-steps s: head (lane % 16) and 8 dims that depend
// on the key operand's layout, which the two must share:
//   interleaved (bf16 keys): dims 32*s + 8*(lane/16) -- one key load of a
//                k-step covers 64 contiguous bytes of each key's row;
//   blocked (int8 keys):     dims 32*(lane/16) + 8*s -- one 32-byte code load
//                per lane covers all 4 k-steps.
template <bool kBlocked>
__device__ __forceinline__ void load_q(u32x4 (&qb)[4], const uint16_t *qrow_head0) {
    const int lane = threadIdx.x & 63;
    const uint16_t *src = qrow_head0 + (lane & 15) * kHeadDim + (kBlocked ? 32 : 8) * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = load16(src + (kBlocked ? 8 : 32) * s);
}

// 2^x with the hardware instruction (v_exp_f32, ~1 ulp).  Results below the
// smallest normal float may flush to zero; a softmax weight that small is
// below fp32 resolution of the sum it joins, so nothing is lost.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// q of one row in LDS: 16 heads x 128 dims bf16, head rows padded to 272 B so
// the 16 heads of one operand read fall in different banks.
constexpr int kQRowBytes = 272;
constexpr float kLazyLog2 = 8.f;   // weights stay <= 256 between rescales
constexpr int kQTileBytes = kGroup * kQRowBytes;

// The row's q (16 heads) from global memory into registers (16-byte piece
// s * 64 + lane of 256 in qv[s]), then into its LDS tile.
__device__ __forceinline__ void load_q_tile(u32x4 (&qv)[4], const uint16_t *qrow_head0) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int e = s * kWave + lane;
        qv[s] = load16(qrow_head0 + (e >> 4) * kHeadDim + 8 * (e & 15));
    }
}

__device__ __forceinline__ void store_q_tile(uint8_t *qt, const u32x4 (&qv)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int e = s * kWave + lane;
        *reinterpret_cast<u32x4 *>(qt + (e >> 4) * kQRowBytes + (e & 15) * 16) = qv[s];
    }
}


// The query B operand (as load_q) from an LDS tile.
template <bool kBlocked>
__device__ __forceinline__ void read_q(u32x4 (&qb)[4], const uint8_t *qt) {
    const int lane = threadIdx.x & 63;
    const uint8_t *src = qt + (lane & 15) * kQRowBytes + (kBlocked ? 64 : 16) * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = *reinterpret_cast<const u32x4 *>(src + (kBlocked ? 16 : 64) * s);
}

// Write 32 keys' V rows into an 8 KiB LDS tile: v[2*kk + hf] holds key
// 4*(lane/8) + kk, 16-byte unit lane%8 + 8*hf (load_block_v's half).
__device__ __forceinline__ void stage_v_rows(const u32x4 (&v)[8], uint8_t *vt) {
    const int lane = threadIdx.x & 63;
    const int kg = lane >> 3, dc = lane & 7;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int key = 4 * kg + kk;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            *reinterpret_cast<u32x4 *>(vt + key * 256 + 16 * v_unit(key, dc + 8 * hf)) = v[2 * kk + hf];
    }
}

// Raw registers of one 32-key chunk of an int8 cache: K codes (key kbase +
// 16*mt + lane%16, dims 32*(lane/16) + 16*h .. +15), V codes (key kbase +
// 4*(lane/8) + kk, dims 8*(lane%8 + 8*hf) .. +7) and one scale per lane:
// lanes 0..31 the key scale of key kbase + lane, lanes 32..63 the value scale
// of key kbase + lane - 32.  Keys past p read key p instead (always in
// bounds): their scores are masked, so their weights are 0.
struct ChunkRegs8 {
    u32x4 ka[2][2];
    uint2 vr[4][2];
    float sc;
};

// kc / vc: the chunk's first key (head g) in the code arrays; ksc / vsc: its
// first key's scale; tok / stok: element strides between tokens.
__device__ __forceinline__ void load_chunk8(ChunkRegs8 &c, const int8_t *kc, const int8_t *vc, const float *ksc,
                                            const float *vsc, int64_t tok, int64_t stok, int last) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    const uint32_t t = (uint32_t)tok;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int8_t *src = kc + (uint32_t)min(16 * mt + lr, last) * t + 32u * lg;
        c.ka[mt][0] = *reinterpret_cast<const u32x4 *>(src);
        c.ka[mt][1] = *reinterpret_cast<const u32x4 *>(src + 16);
    }
    const int kg = lane >> 3, dc = lane & 7;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int8_t *src = vc + (uint32_t)min(4 * kg + kk, last) * t + 8u * dc;
        c.vr[kk][0] = *reinterpret_cast<const uint2 *>(src);
        c.vr[kk][1] = *reinterpret_cast<const uint2 *>(src + 64);
    }
    const float *sp = lane < 32 ? ksc : vsc;
    c.sc = sp[(int64_t)min(lane & 31, last) * stok];
}

// 8 int8 codes -> 8 bf16 (exact: |code| <= 127 needs 7 significant bits).
__device__ __forceinline__ float i8_at(uint32_t w, int k) { return (float)(int8_t)(uint8_t)(w >> (8 * k)); }
__device__ __forceinline__ u32x4 i8x8_to_bf16(uint32_t w0, uint32_t w1) {
    return u32x4{pack_bf16x2(i8_at(w0, 0), i8_at(w0, 1)), pack_bf16x2(i8_at(w0, 2), i8_at(w0, 3)),
                 pack_bf16x2(i8_at(w1, 0), i8_at(w1, 1)), pack_bf16x2(i8_at(w1, 2), i8_at(w1, 3))};
}

// K operands of an int8 chunk, as ChunkRegs::ka holds them for bf16.
__device__ __forceinline__ void k_operands8(const ChunkRegs8 &c, u32x4 (&ka)[2][4]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ka[mt][2 * h] = i8x8_to_bf16(c.ka[mt][h][0], c.ka[mt][h][1]);
            ka[mt][2 * h + 1] = i8x8_to_bf16(c.ka[mt][h][2], c.ka[mt][h][3]);
        }
}

// V codes as bf16 into the V tile (stage_v's layout); the scales into the
// wave's 64-float scale tile (keys' scales, then values').
__device__ __forceinline__ void stage_v8(const ChunkRegs8 &c, uint8_t *vt, float *sct) {
    const int lane = threadIdx.x & 63;
    const int kg = lane >> 3, dc = lane & 7;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int key = 4 * kg + kk;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            *reinterpret_cast<u32x4 *>(vt + key * 256 + 16 * v_unit(key, dc + 8 * hf)) =
                i8x8_to_bf16(c.vr[kk][hf].x, c.vr[kk][hf].y);
    }
    sct[lane] = c.sc;
}

// Fold the chunk [kbase, kbase + 32) (keys <= p visible) into row `row`
// (wave-uniform) of a group of RW rows' states: K operands from registers,
// V^T from the LDS tile (already staged and synced).  The scores and softmax
// run once, with the row's max and sum picked by selects; only the rare
// rescale and the 8 PV MFMAs sit under a branch on the row.  (The int8 cache's
// fold; the bf16 caches fold whole blocks, softmax_pv_block below.)
// KV8 (int8 cache): every key's score is scaled by its key scale and every
// weight by its value scale before the PV product (the sum of weights is
// unscaled), with the scales from the wave's scale tile `sct`.
template <int RW, bool KV8>
__device__ __forceinline__ void fold_rows(Softmax (&st)[RW], int row, const u32x4 (&qb)[4],
                                          const u32x4 (&ka)[2][4], int kbase, int p, float scale_log2,
                                          const uint8_t *vt, const float *sct) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    floatx4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_16x16x32(ka[mt][s], qb[s], acc);
        sacc[mt] = acc;
    }
    floatx4 ksc[2], vsc[2];
    if constexpr (KV8) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            ksc[mt] = *reinterpret_cast<const floatx4 *>(sct + 16 * mt + 4 * lg);
            vsc[mt] = *reinterpret_cast<const floatx4 *>(sct + 32 + 16 * mt + 4 * lg);
        }
    }
    // Online softmax over this lane's 8 keys of head lr.  Only the chunk that
    // holds position p has keys to mask.  The max is taken on the unscaled
    // scores and scaled once (scaling by a positive constant is monotone, so
    // this is the max of the scaled scores bit for bit); each weight is one
    // FMA and one exp2.
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = sacc[mt][i];
            if constexpr (KV8) v *= ksc[mt][i];
            z[mt][i] = v;
        }
    if (__builtin_expect(kbase + 31 > p, 0)) {   // uniform: the chunk reaching past p
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kbase + 16 * mt + 4 * lg + i > p) z[mt][i] = -INFINITY;
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[mt][i]);
    mx = max_over_lane_groups(mx) * scale_log2;   // finite: key kbase <= p is visible
    float m_cur = st[0].m, l_cur = st[0].l;
#pragma unroll
    for (int i = 1; i < RW; ++i) {
        m_cur = row == i ? st[i].m : m_cur;
        l_cur = row == i ? st[i].l : l_cur;
    }
    // The reference max moves only when a head's scores exceed it by more
    // than kLazyLog2 (always on the first chunk): until then the weights are
    // exp2(z - m) <= 2^kLazyLog2 and the accumulators need no rescale.  The
    // result is the same softmax; m is the reference, not necessarily the max.
    if (__ballot(mx > m_cur + kLazyLog2) != 0) {
        const float m_new = fmaxf(m_cur, mx);
        const float alpha = fast_exp2(m_cur - m_new);    // 0 on the first chunk
        l_cur *= alpha;
#pragma unroll
        for (int i = 0; i < RW; ++i)
            if (row == i) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) st[i].o[dt] *= alpha;
            }
        m_cur = m_new;
    }
    float pr[2][4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[mt][i] = fast_exp2(fmaf(z[mt][i], scale_log2, -m_cur));
            // the first weight starts the sum (0 + w == w for every w >= +0)
            psum = mt == 0 && i == 0 ? pr[0][0] : psum + pr[mt][i];
            if constexpr (KV8) pr[mt][i] *= vsc[mt][i];
        }
    l_cur += psum;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        st[i].m = row == i ? m_cur : st[i].m;
        st[i].l = row == i ? l_cur : st[i].l;
    }
    const u32x4 pb = {pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                      pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};
    // V^T operand of d-tile dt: lane (lg, lr) needs dim 16*dt + lr of keys
    // 4*lg + 0..3 and 16 + 4*lg + 0..3 (the P^T k-order).  Lane t of group lg
    // addresses the 8-byte piece (dims 16*dt + 4*(t%4) .. +3) of key 4*lg + t/4
    // (and key + 16); the swizzle only flips address bits 5..7, so the piece
    // for d-tile dt sits at the dt = 0 offset XOR (dt << 5).
    u32x4 va[8];
    const int vkey = 4 * lg + (lr >> 2);
    const int rd0 = vkey * 256 + 8 * (lr & 3) + 32 * (vkey & 7);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const int rd = rd0 ^ (dt << 5);
        const uint2 lo = lds_read_tr16(vt + rd);
        const uint2 hi = lds_read_tr16(vt + rd + 16 * 256);
        va[dt] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
        if (row == i) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) st[i].o[dt] = mfma_16x16x32(va[dt], pb, st[i].o[dt]);
        }
}

// ---- 64-key block folds (bf16 caches) ----
//
// A block's fold for one row: S^T = K Q^T over its 4 key tiles, one
// online-softmax step over its 64 keys, then O^T += V^T P^T over its two
// 32-key halves.  Per key it costs the same MFMAs as two 32-key folds, but
// the fold's fixed chain (q read, max and its cross-lane step, the reference
// test, the row's state selects) runs once per 64 keys, and the QK^T products
// form 4 independent chains instead of 2.

// S^T of one block for one row's 16 heads: sacc[mt] holds keys 16*mt + 4*lg
// + i (i < 4) of head lr.
__device__ __forceinline__ void qk_block(floatx4 (&sacc)[4], const u32x4 (&qb)[4], const u32x4 (&ka)[4][4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_16x16x32(ka[mt][s], qb[s], acc);
        sacc[mt] = acc;
    }
}

// The rest of a block's fold into row `row` of a group of RW rows' states
// (keys past p masked; kbase: the block's first key).  kVR: the V^T operands
// of half h are vr[h][0..7] (tiled cache); else they are gathered from the
// wave's LDS V tile (half h at vt + 8192 * h, stage_v_rows' layout) as
// fold_rows does for a chunk.
template <int RW, bool kVR>
__device__ __forceinline__ void softmax_pv_block(Softmax (&st)[RW], int row, const floatx4 (&sacc)[4],
                                                 const u32x4 (&vr)[2][8], const uint8_t *vt, int kbase, int p,
                                                 float scale_log2) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    float z[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[mt][i] = sacc[mt][i];
    if (__builtin_expect(kbase + 63 > p, 0)) {   // uniform: the block reaching past p
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kbase + 16 * mt + 4 * lg + i > p) z[mt][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[mt][i]);
    mx = max_over_lane_groups(mx) * scale_log2;   // finite: key kbase <= p is visible
    float m_cur = st[0].m, l_cur = st[0].l;
#pragma unroll
    for (int i = 1; i < RW; ++i) {
        m_cur = row == i ? st[i].m : m_cur;
        l_cur = row == i ? st[i].l : l_cur;
    }
    // The reference max moves only when a head's scores exceed it by more
    // than kLazyLog2 (always on the first block), as in fold_rows.
    if (__ballot(mx > m_cur + kLazyLog2) != 0) {
        const float m_new = fmaxf(m_cur, mx);
        const float alpha = fast_exp2(m_cur - m_new);    // 0 on the first block
        l_cur *= alpha;
#pragma unroll
        for (int i = 0; i < RW; ++i)
            if (row == i) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) st[i].o[dt] *= alpha;
            }
        m_cur = m_new;
    }
    float pr[4][4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[mt][i] = fast_exp2(fmaf(z[mt][i], scale_log2, -m_cur));
            // the first weight starts the sum (0 + w == w for every w >= +0)
            psum = mt == 0 && i == 0 ? pr[0][0] : psum + pr[mt][i];
        }
    l_cur += psum;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        st[i].m = row == i ? m_cur : st[i].m;
        st[i].l = row == i ? l_cur : st[i].l;
    }
    // P^T operand of half h: keys 32*h + 4*lg + 0..3 and 32*h + 16 + 4*lg + 0..3
    // (the k-order of a chunk's P^T in fold_rows).
    u32x4 pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        pb[h] = u32x4{pack_bf16x2(pr[2 * h][0], pr[2 * h][1]), pack_bf16x2(pr[2 * h][2], pr[2 * h][3]),
                      pack_bf16x2(pr[2 * h + 1][0], pr[2 * h + 1][1]),
                      pack_bf16x2(pr[2 * h + 1][2], pr[2 * h + 1][3])};
    u32x4 va[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if constexpr (kVR) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) va[h][dt] = vr[h][dt];
        } else {
            const int vkey = 4 * lg + (lr >> 2);
            const int rd0 = vkey * 256 + 8 * (lr & 3) + 32 * (vkey & 7);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int rd = 8192 * h + (rd0 ^ (dt << 5));
                const uint2 lo = lds_read_tr16(vt + rd);
                const uint2 hi = lds_read_tr16(vt + rd + 16 * 256);
                va[h][dt] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
        if (row == i) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                st[i].o[dt] = mfma_16x16x32(va[0][dt], pb[0], st[i].o[dt]);
                st[i].o[dt] = mfma_16x16x32(va[1][dt], pb[1], st[i].o[dt]);
            }
        }
}

// Clear the V elements of keys past `last` (an offset within one 32-key half;
// below 0: the whole half) in that half's V^T operands from a tiled cache:
// such keys may never have been written, and 0 times an unwritten NaN would
// not be 0.
__device__ __forceinline__ void clear_tail_v_half(u32x4 (&v)[8], int last) {
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    if (last < 31) {
        // dword w of a V^T operand: keys k0 (low half) and k0 + 1 (high half)
        uint32_t m[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int k0 = (w < 2 ? 4 * lg : 16 + 4 * lg) + 2 * (w & 1);
            m[w] = (k0 <= last ? 0x0000ffffu : 0u) | (k0 + 1 <= last ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int w = 0; w < 4; ++w) v[dt][w] &= m[w];
    }
}

// K operands and V^T operands of a block from a tiled cache (kt, vt: the
// block's 8,192-element K and V tiles of one key head; 32-key half h at
// 4096 * h).  A half's K tile holds its 8 QK^T A operands (key tile mt, k-step
// s) in order and its V tile the 8 V^T operands of the PV product (d-tile dt),
// each as 64 lane-ordered 16-byte pieces, so every load reads 1 KiB of
// contiguous memory.  Keys past the block's largest position may never have
// been written: their scores are masked and their V elements cleared
// (clear_tail_v_half) before the PV products, at fold time, so that a
// prefetch never waits for its own loads.
// Addressing: each load's 1 KiB piece has a wave-uniform base and every load
// shares one per-lane byte offset, 16 * lane.
__device__ __forceinline__ u32x4 load_tile_piece(const uint16_t *piece, uint32_t lane_bytes) {
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(piece) + lane_bytes);
}

__device__ __forceinline__ void load_block_k_tiled(u32x4 (&ka)[4][4], const uint16_t *kt) {
    const uint32_t lb = 16u * (uint32_t)(threadIdx.x & 63);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int s = 0; s < 4; ++s) ka[2 * h + mt][s] = load_tile_piece(kt + 4096 * h + 512 * (4 * mt + s), lb);
}

__device__ __forceinline__ void load_block_v_tiled(u32x4 (&v)[2][8], const uint16_t *vt) {
    const uint32_t lb = 16u * (uint32_t)(threadIdx.x & 63);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) v[h][dt] = load_tile_piece(vt + 4096 * h + 512 * dt, lb);
}

// K operands of a block from a strided cache (kblk: its first key; tok:
// elements between consecutive keys): tile mt holds keys 16*mt + lane%16,
// dims 32*s + 8*(lane/16) (the interleaved layout q's operands share).  Keys past `last`
// (the block's largest visible key offset, 0..63) read key `last` instead, so
// every read stays inside the keys that exist.
__device__ __forceinline__ void load_block_k(u32x4 (&ka)[4][4], const uint16_t *kblk, int64_t tok, int last) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    const uint32_t tok_bytes = (uint32_t)tok * 2u;
    const char *kb = reinterpret_cast<const char *>(kblk);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const uint32_t off = (uint32_t)min(16 * mt + lr, last) * tok_bytes + 16u * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[mt][s] = *reinterpret_cast<const u32x4 *>(kb + off + 64 * s);
    }
}

// V rows of a block from a strided cache, half h in v[h] (keys 32*h +
// 4*(lane/8) + kk in v[h][2*kk + 0/1], 16-byte units lane%8 and lane%8 + 8:
// stage_v_rows' input); keys past `last` read key `last`.
__device__ __forceinline__ void load_block_v(u32x4 (&v)[2][8], const uint16_t *vblk, int64_t tok, int last) {
    const int lane = threadIdx.x & 63, kg = lane >> 3, dc = lane & 7;
    const uint32_t tok_bytes = (uint32_t)tok * 2u;
    const char *vb = reinterpret_cast<const char *>(vblk);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint32_t off = (uint32_t)min(32 * h + 4 * kg + kk, last) * tok_bytes + 16u * dc;
            v[h][2 * kk] = *reinterpret_cast<const u32x4 *>(vb + off);
            v[h][2 * kk + 1] = *reinterpret_cast<const u32x4 *>(vb + off + 128);
        }
}

// Fold one loaded int8 chunk into a single state st (stage and convert V, fold,
// release the tile).
__device__ __forceinline__ void fold_chunk(Softmax &st, const u32x4 (&qb)[4], const ChunkRegs8 &c,
                                           int kbase, int p, float scale_log2, uint8_t *vt, float *sct) {
    stage_v8(c, vt, sct);
    wave_lds_sync();
    u32x4 ka[2][4];
    k_operands8(c, ka);
    fold_rows<1, true>(*reinterpret_cast<Softmax(*)[1]>(&st), 0, qb, ka, kbase, p, scale_log2, vt, sct);
    wave_lds_sync();
}

// Unit (row r, key head g) of a head-major enumeration: consecutive units are
// consecutive rows of one key head, so neighbouring waves share local blocks.
struct Unit {
    int r, g, s, p;
    bool ok;
};

// Row r of key head g: its sequence, position and whether the batch metadata
// is consistent for it.
__device__ __forceinline__ Unit row_unit(const AttnArgs &a, int r, int g) {
    Unit u;
    u.g = g;
    u.r = r;
    u.s = locate_seq(a.b.cu_rows, a.b.n_seqs, r);
    const int rows_s = a.b.cu_rows[u.s + 1] - a.b.cu_rows[u.s];
    const int L = a.b.seq_lens[u.s];
    u.ok = rows_s > 0 && rows_s <= L && L <= a.b.max_seq_len;
    u.p = L - rows_s + (r - a.b.cu_rows[u.s]);
    return u;
}

__device__ __forceinline__ Unit make_unit(const AttnArgs &a, int64_t unit) {
    return row_unit(a, (int)(unit % a.b.total_rows), (int)(unit / a.b.total_rows));
}

// Prefill.  One wave per group of RW rows of one key head (which rows: see
// group_rows below).  For each row it holds the 16 query heads (so every
// kept block is fetched once for the whole group) and an online-softmax state.  The
// rows' kept blocks are merged into one list sorted by block index and walked
// one block at a time (32-key chunks with the int8 cache), the next block's
// K/V loads in flight while the current one is folded.  A block kept by several of the rows (their shared local
// block, or any block on correlated rows) is loaded once and folded into each
// of them.  Each row still sees its own blocks in ascending order, so its bits
// depend only on its blocks.  Walking the merged
// list keeps every resident wave of a key head near the same key position at
// the same time, so rows that keep the same block read it while it is still
// in L2: with independent per-row walks, two rows reach a shared block at
// different ranks of their own lists, long after L2 has turned over.
constexpr int kInvalidKey = 1 << 25;   // above every block index of an int32 position

// Which rows share a wave.  A resident wave's key position at a given time is
// set by its merged list: if the lists of some waves crowd into a part of the
// key range and others spread out, the waves drift apart, the band of blocks
// in use at once outgrows L2, and rows that keep the same block no longer read
// it while it is cached.  With rows that keep unrelated blocks, the rows of
// each key head are therefore grouped per window of 64 consecutive rows: the
// window's rows are ranked by the mean of their kept blocks, ranks are paired
// from both ends (k with 63-k), and a wave of 4 rows takes two such pairs from
// the two halves (ranks w, 63-w, 16+w, 47-w), so every wave's list covers the
// key range about evenly and all of them advance through it together (chunk
// attention with i.i.d. selections: L2 hits 0.61 -> 0.79).  Where neighbouring
// rows keep mostly the same blocks, the consecutive grouping is worth more (the
// wave loads a shared block once for all its rows), so a window whose
// neighbouring rows match in more than 35% of their blocks keeps it.  The
// grouping decides only which wave computes a row: a row's result depends on
// its own blocks alone.
constexpr int kGroupWindow = 64;

// Position of rank rho among the W rows of a window under the pairing above:
// pair k = (rank k, rank W-1-k), pairs of the lower half (k < h) at even pair
// positions and of the upper half at odd ones; with odd W the highest rank
// takes the last position.  A bijection of [0, W).
__device__ __forceinline__ int paired_position(int rho, int W) {
    if (W & 1) {
        if (rho == W - 1) return W - 1;
        --W;
    }
    const int P = W >> 1, h = (P + 1) >> 1;
    const int k = min(rho, W - 1 - rho), s = rho > W - 1 - rho ? 1 : 0;
    const int sp = k < h ? 2 * k : 2 * (k - h) + 1;
    return 2 * sp + s;
}

// The rows of group r0 / RW of key head g (wave-uniform).  Groups past the
// batch's end get row total_rows - 1 (the caller marks them not ok).
template <int RW>
__device__ __forceinline__ void group_rows(const AttnArgs &a, int g, int r0, int (&rows)[RW]) {
    const int n = a.b.total_rows;
#pragma unroll
    for (int i = 0; i < RW; ++i) rows[i] = min(r0 + i, n - 1);
    if constexpr (RW > 1) {
        const int lane = threadIdx.x & 63;
        const int w0 = r0 & ~(kGroupWindow - 1), wn = min(kGroupWindow, n - w0);
        // lane l: row w0 + l, its sort key (mean kept block, lane as the tie
        // break) and a 128-bit hashed set of its kept blocks
        uint32_t ukey = 0x80000000u | (uint32_t)lane;   // lanes past the batch rank last
        uint32_t hs[4] = {0u, 0u, 0u, 0u};
        if (lane < wn) {
            constexpr int kT = RW == 4 ? 16 : kMaxTopK;   // top_k's bound at RW rows per wave
            const int32_t *ix = a.idx + ((int64_t)(w0 + lane) * a.H + g) * a.top_k;
            int v[kT];
#pragma unroll
            for (int t = 0; t < kT; ++t) v[t] = ix[min(t, a.top_k - 1)];   // all in flight together
            uint32_t sum = 0, cnt = 0;
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                const int b = v[t];
                if (t < a.top_k && b >= 0 && b < kInvalidKey) {
                    sum += (uint32_t)b;
                    ++cnt;
                    const uint32_t hb = (uint32_t)b & 127u;
#pragma unroll
                    for (int w = 0; w < 4; ++w) hs[w] |= (hb >> 5) == (uint32_t)w ? 1u << (hb & 31) : 0u;
                }
            }
            const float mean = cnt ? (float)sum / (float)cnt : 0.f;
            ukey = ((uint32_t)fminf(mean * 64.f, 33554431.f) << 6) | (uint32_t)lane;
        }
        int common = 0, total = 0;   // vs. the neighbouring row (lane ^ 1), each <= 32
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t o = (uint32_t)__shfl_xor((int)hs[w], 1);
            common += __popc(hs[w] & o);
            total += __popc(hs[w]);
        }
        int csum = 0, tsum = 0;      // their sums over the wave, bit by bit
#pragma unroll
        for (int bit = 0; bit < 6; ++bit) {
            csum += (int)__popcll(__ballot((common >> bit) & 1)) << bit;
            tsum += (int)__popcll(__ballot((total >> bit) & 1)) << bit;
        }
        int rank = 0;
#pragma unroll 8
        for (int m = 0; m < kWave; ++m) rank += (uint32_t)__builtin_amdgcn_readlane((int)ukey, m) < ukey;
        if (100 * csum <= 35 * tsum) {
            const int pos = lane < wn ? paired_position(rank, wn) : kWave;
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                const uint64_t hit = __ballot(pos == r0 - w0 + i);
                if (hit) rows[i] = w0 + __builtin_ctzll(hit);
            }
        }
    }
}

// kTiled: K/V from a tiled cache (kv_tok / kv_head are the tiles' block and
// head strides); the chunk's V^T operands stay in registers.
template <int RW, bool KV8, bool kTiled>
__device__ __forceinline__ void prefill_group(const AttnArgs &a, int g, int r0, uint8_t *vt, uint8_t *qt,
                                              float *sct) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    const int hq = a.H * kGroup;
    const int top_k = a.top_k;

    int rows[RW];
    group_rows<RW>(a, g, r0, rows);
    // The rows' q: loaded now and, over bf16 caches, written to the LDS tiles
    // once the entries are sorted and the first block's loads are out, so all
    // these loads overlap.  The int8 walk writes them at once and loads its
    // first chunk inside the walk: q held across that load, and the chunk's
    // registers live outside the loop, took the int8 kernel from 100 to 144
    // AGPRs and its chunk attention from 727 to 875 us.
    u32x4 qv[RW][4];
#pragma unroll
    for (int i = 0; i < RW; ++i) load_q_tile(qv[i], a.q + ((int64_t)rows[i] * hq + g * kGroup) * kHeadDim);
    if constexpr (KV8) {
#pragma unroll
        for (int i = 0; i < RW; ++i) store_q_tile(qt + i * kQTileBytes, qv[i]);
    }
    Unit u[RW];
    Softmax st[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int r = rows[i];
        u[i] = row_unit(a, r, g);
        u[i].ok = u[i].ok && r0 + i < a.b.total_rows;   // rows past the end: not ok
        softmax_init(st[i]);
    }
    // Entry (row li, slot lt) on lane li*top_k + lt: its block if kept and
    // visible, with its row's position and K/V offset.
    const int li = lane / top_k, lt = lane - li * top_k;
    int rl = rows[0];
    Unit ul = u[0];   // the entry's row's unit, from the group's (wave-uniform) units
#pragma unroll
    for (int i = 1; i < RW; ++i) {
        rl = li == i ? rows[i] : rl;
        ul.s = li == i ? u[i].s : ul.s;
        ul.p = li == i ? u[i].p : ul.p;
        ul.ok = li == i ? u[i].ok : ul.ok;
    }
    int key = kInvalidKey;
    if (li < RW && r0 + li < a.b.total_rows && ul.ok) {
        const int b = a.idx[((int64_t)rl * a.H + g) * top_k + lt];
        if (b >= 0 && b * kBlock <= ul.p) key = b;
    }
    // token of the entry's block's first key in the key / value arrays
    const int64_t tok_l = block_token0(a.b, ul.s, seq_token0(a.b, ul.s), key == kInvalidKey ? 0 : key);
    // Sort the entries by (block, lane): lane k of the e_* values holds the
    // k-th entry (block * 4 + row, its row's position and block token).
    const uint32_t skey = ((uint32_t)key << 6) | (uint32_t)lane;
    force_ready((int)skey);
    int rank = 0;
#pragma unroll 8
    for (int m = 0; m < kWave; ++m) rank += (uint32_t)__builtin_amdgcn_readlane((int)skey, m) < skey;
    const int dst = rank << 2;
    const int e_key = __builtin_amdgcn_ds_permute(dst, (key << 2) | (li & 3));
    const int e_p = __builtin_amdgcn_ds_permute(dst, ul.p);
    const int e_lo = __builtin_amdgcn_ds_permute(dst, (int)(uint32_t)tok_l);
    const int e_hi = __builtin_amdgcn_ds_permute(dst, (int)(uint32_t)((uint64_t)tok_l >> 32));
    const int n_ent = (int)__popcll(__ballot(key != kInvalidKey));
    // Entries that read the same K/V (same first token: one block of one
    // sequence, or a page shared by sequences) are adjacent after the sort and
    // form a group; bit k of `starts` marks the entry that opens a group.
    const int prev_lo = __shfl_up(e_lo, 1), prev_hi = __shfl_up(e_hi, 1);
    const uint64_t starts = __ballot(lane < n_ent && (lane == 0 || prev_lo != e_lo || prev_hi != e_hi));
    auto group_end = [&](int k) -> int {       // one past the last entry of the group opened by k
        const uint64_t rest = k + 1 < kWave ? starts >> (k + 1) : 0ull;
        return rest ? k + 1 + __builtin_ctzll(rest) : n_ent;
    };

    force_ready(e_key);
    force_ready(e_p);
    force_ready(e_lo);
    force_ready(e_hi);

    if constexpr (!KV8) {
        // bf16 caches: one fold per (block, row) over the block's 64 keys.
        // The walk moves from run to run (a run: the entries that read one
        // block's K/V, usually one row).  K of the next run is requested as
        // soon as this run's last QK^T products are issued, V as soon as this
        // run's V is no longer needed in registers (tiled: after its last PV
        // products; strided: once staged in LDS), so each load has most of a
        // fold to arrive.  Past the last run the requests re-read it, so
        // every path has the same loads in flight.
        struct Run {
            int k, end, kb, p_max;    // entries [k, end); first key; largest position among its rows
            int64_t tok;              // token of the block's first key
        };
        auto run_at = [&](int k) -> Run {
            Run r;
            r.k = k;
            r.end = group_end(k);
            r.kb = (__builtin_amdgcn_readlane(e_key, k) >> 2) * kBlock;
            r.tok = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(e_hi, k) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane(e_lo, k));
            int pm = __builtin_amdgcn_readlane(e_p, k);
            for (int j = k + 1; j < r.end; ++j) pm = max(pm, __builtin_amdgcn_readlane(e_p, j));
            r.p_max = pm;
            return r;
        };
        u32x4 kreg[4][4];   // K operands of the block's 4 key tiles
        u32x4 vreg[2][8];   // V of each 32-key half: tiled, its 8 V^T operands; strided, its rows (load_block_v)
        auto load_k = [&](const Run &r) {
            if constexpr (kTiled) {
                load_block_k_tiled(kreg, a.k + (r.tok >> 6) * a.kv_tok + (int64_t)g * a.kv_head);
            } else {
                load_block_k(kreg, a.k + r.tok * a.kv_tok + (int64_t)g * a.kv_head, a.kv_tok, r.p_max - r.kb);
            }
        };
        auto load_v = [&](const Run &r) {
            if constexpr (kTiled) {
                load_block_v_tiled(vreg, a.v + (r.tok >> 6) * a.kv_tok + (int64_t)g * a.kv_head);
            } else {
                load_block_v(vreg, a.v + r.tok * a.kv_tok + (int64_t)g * a.kv_head, a.kv_tok, r.p_max - r.kb);
            }
        };
        Run r = run_at(0);
        if (n_ent > 0) {
            load_k(r);
            load_v(r);
        }
#pragma unroll
        for (int i = 0; i < RW; ++i) store_q_tile(qt + i * kQTileBytes, qv[i]);
        wave_lds_sync();   // q tiles written before the first fold reads them
        if (n_ent > 0) {
            for (;;) {
                const bool have = r.end < n_ent;
                const Run nx = have ? run_at(r.end) : r;
                if constexpr (kTiled) {
                    clear_tail_v_half(vreg[0], r.p_max - r.kb);
                    clear_tail_v_half(vreg[1], r.p_max - r.kb - 32);
                } else {
                    stage_v_rows(vreg[0], vt);
                    stage_v_rows(vreg[1], vt + 8192);
                    wave_lds_sync();
                    load_v(nx);
                }
                for (int j = r.k; j < r.end; ++j) {
                    const int row = __builtin_amdgcn_readlane(e_key, j) & 3;
                    const int p = __builtin_amdgcn_readlane(e_p, j);
                    u32x4 qb[4];
                    read_q<false>(qb, qt + row * kQTileBytes);
                    floatx4 sacc[4];
                    qk_block(sacc, qb, kreg);
                    if (j == r.end - 1) load_k(nx);
                    softmax_pv_block<RW, kTiled>(st, row, sacc, vreg, vt, r.kb, p, a.scale_log2);
                }
                if constexpr (kTiled) load_v(nx);
                else wave_lds_sync();   // PV reads finish before the next run's V overwrites the tile
                if (!have) break;
                r = nx;
            }
        }
    } else {
        // int8 cache: one fold per (32-key chunk, row), the chunk's codes
        // staged and converted in LDS.  A chunk: half hh of the block of the
        // run opened by entry k (wave-uniform values); p_max: the largest
        // position among its rows.
        struct Chunk {
            int kb, k, end, p_max;
            int64_t tok;      // token of the chunk's first key
        };
        auto chunk_at = [&](int k, int hh) -> Chunk {
            Chunk c;
            c.k = k;
            c.end = group_end(k);
            c.kb = (__builtin_amdgcn_readlane(e_key, k) >> 2) * kBlock + 32 * hh;
            c.tok = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(e_hi, k) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane(e_lo, k)) + 32 * hh;
            int pm = __builtin_amdgcn_readlane(e_p, k);
            for (int j = k + 1; j < c.end; ++j) pm = max(pm, __builtin_amdgcn_readlane(e_p, j));
            c.p_max = pm;
            return c;
        };
        int k = 0, half = 0;
        auto next_chunk = [&](Chunk &c) -> bool {   // advances (k, half) to the next chunk some row sees
            for (;;) {
                if (half == 0) {
                    half = 1;
                } else {
                    half = 0;
                    k = group_end(k);
                    if (k >= n_ent) return false;
                }
                c = chunk_at(k, half);
                if (c.kb <= c.p_max) return true;
            }
        };
        auto load = [&](ChunkRegs8 &r, const Chunk &c) {
            const int64_t off = c.tok * a.kv_tok + (int64_t)g * a.kv_head;
            const int64_t soff = c.tok * a.s_tok + (int64_t)g * a.s_head;
            load_chunk8(r, a.k8 + off, a.v8 + off, a.ks + soff, a.vs + soff, a.kv_tok, a.s_tok, c.p_max - c.kb);
        };
        // Fold one loaded chunk into every row of its run that sees it (keys
        // past a row's own position are masked in its fold).
        auto fold = [&](ChunkRegs8 &r, const Chunk &c) {
            u32x4 ka8[2][4];
            stage_v8(r, vt, sct);
            k_operands8(r, ka8);
            wave_lds_sync();
            for (int j = c.k; j < c.end; ++j) {
                const int row = __builtin_amdgcn_readlane(e_key, j) & 3;
                const int p = __builtin_amdgcn_readlane(e_p, j);
                if (c.kb > p) continue;
                u32x4 qb[4];
                read_q<true>(qb, qt + row * kQTileBytes);
                fold_rows<RW, true>(st, row, qb, ka8, c.kb, p, a.scale_log2, vt, sct);
            }
            wave_lds_sync();   // reads finish before the next chunk overwrites the tiles
        };
        // The prefetch is unconditional (past the last chunk it re-reads the
        // chunk being folded), so every path through the loop has the same
        // loads in flight and a fold waits only for its own chunk.
        wave_lds_sync();   // q tiles written before the first fold reads them
        if (n_ent > 0) {
            Chunk c0 = chunk_at(0, 0), c1;  // an entry's first half is always visible
            ChunkRegs8 ca, cb;
            load(ca, c0);
            for (;;) {
                const bool have1 = next_chunk(c1);
                if (!have1) c1 = c0;
                load(cb, c1);
                fold(ca, c0);
                if (!have1) break;
                const bool have0 = next_chunk(c0);
                if (!have0) c0 = c1;
                load(ca, c0);
                fold(cb, c1);
                if (!have0) break;
            }
        }
    }

#pragma unroll
    for (int i = 0; i < RW; ++i) {
        if (!u[i].ok) continue;
        const float l = sum_over_lane_groups(st[i].l);
        const int h = g * kGroup + lr;
        uint16_t *dst_o = a.out + ((int64_t)u[i].r * hq + h) * kHeadDim + 4 * lg;
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint2 w = make_uint2(pack_bf16x2(st[i].o[dt][0] * inv, st[i].o[dt][1] * inv),
                                       pack_bf16x2(st[i].o[dt][2] * inv, st[i].o[dt][3] * inv));
            *reinterpret_cast<uint2 *>(dst_o + 16 * dt) = w;
        }
        if (a.lse && lg == 0)
            a.lse[(int64_t)u[i].r * hq + h] = l > 0.f ? (st[i].m + log2f(l)) * kLn2 : -INFINITY;
    }
}

// Groups are enumerated head-major (consecutive groups: groups of one key head,
// in the order of their 64-row windows), one per wave.  kW waves per
// workgroup: 4 for the 4-row walk, whose four waves start together and keep
// their walks in step (L2 hits: one-wave workgroups took the chunk attention
// from ~375 to ~390-420 us); 1 for the shorter walks of small batches, where a
// SIMD then starts its next group as soon as its wave ends instead of waiting
// for the slowest of four (the 2,048-row prefill 50.4 -> 46.3 us a step).
// Workgroups go to the 8 XCDs in turn, so with one wave each, workgroup j
// takes group 32 (j / 32) + 4 (j % 8) + (j / 8) % 4: each XCD keeps the same
// 4 consecutive groups of every 32 as with four-wave workgroups (in a last
// partial 32, group j).
__device__ __forceinline__ int64_t prefill_group_of(int64_t j, int64_t n) {
    const int64_t base = j & ~int64_t(31);
    if (base + 32 > n) return j;
    return base + 4 * (j & 7) + ((j >> 3) & 3);
}

template <int RW, bool KV8, bool kTiled, int kW>
__global__ __launch_bounds__(64 * kW) void prefill_kernel(AttnArgs a, int groups_per_head) {
    // V tile per wave: a block's two 32-key halves (strided bf16), one chunk
    // (int8), none (tiled: V^T operands come straight from the cache)
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[kW][kTiled ? 16 : KV8 ? 8192 : 16384];
    __shared__ __attribute__((aligned(16))) uint8_t qt_all[kW][RW * kQTileBytes];
    __shared__ __attribute__((aligned(16))) float sc_all[kW][KV8 ? 64 : 4];
    const int wave = kW == 1 ? 0 : uniform(threadIdx.x >> 6);
    const int64_t n = (int64_t)groups_per_head * a.H;
    const int64_t j = (int64_t)blockIdx.x * kW + wave;
    if (j >= n) return;
    const int64_t grp = kW == 1 ? prefill_group_of(j, n) : j;
    const int g = (int)(grp / groups_per_head);
    const int r0 = (int)(grp % groups_per_head) * RW;
    prefill_group<RW, KV8, kTiled>(a, g, r0, vt_all[wave], qt_all[wave], sc_all[wave]);
}

// Decode.  The kept list of a (row, key head) is folded one block (two 32-key
// chunks, both in flight together) per state; the states of 4 consecutive
// slots combine into a partial (max, sum, weighted values), and the partials
// merge in slot order with log-sum-exp weights.  That tree depends only on
// top_k, and both decode kernels below compute it with the same helpers, in
// the same order: a row's bits never depend on the rest of the batch, on the
// kernel the launch picks, or on which workgroup finished last.

// One kept block (index b_raw) of unit u folded into st.
template <bool KV8, bool kTiled>
__device__ __forceinline__ void decode_fold_block(const AttnArgs &a, const Unit &u, int64_t kv0,
                                                  const u32x4 (&qb)[4], int b_raw, Softmax &st, uint8_t *vt,
                                                  float *sct) {
    const int b = u.ok ? b_raw : -1;
    const int kb0 = b * kBlock, kb1 = kb0 + 32;
    if (b < 0 || kb0 > u.p) return;
    const int64_t t0 = block_token0(a.b, u.s, kv0, b);     // the block's first key
    if constexpr (!KV8) {
        // bf16 caches: the block's 64 keys in one fold, as the prefill walk
        // folds a block (so decode and prefill share the fold's arithmetic)
        u32x4 kreg[4][4], vreg[2][8];
        const int last = min(u.p - kb0, 63);    // the block's largest visible key offset
        if constexpr (kTiled) {   // the tile of block t0 / 64 (whole: its keys past p are masked / cleared)
            const int64_t off = (t0 >> 6) * a.kv_tok + (int64_t)u.g * a.kv_head;
            load_block_k_tiled(kreg, a.k + off);
            load_block_v_tiled(vreg, a.v + off);
            clear_tail_v_half(vreg[0], last);
            clear_tail_v_half(vreg[1], last - 32);
        } else {
            const int64_t off = t0 * a.kv_tok + (int64_t)u.g * a.kv_head;
            load_block_k(kreg, a.k + off, a.kv_tok, last);
            load_block_v(vreg, a.v + off, a.kv_tok, last);
            stage_v_rows(vreg[0], vt);
            stage_v_rows(vreg[1], vt + 8192);
            wave_lds_sync();
        }
        floatx4 sacc[4];
        qk_block(sacc, qb, kreg);
        softmax_pv_block<1, kTiled>(*reinterpret_cast<Softmax(*)[1]>(&st), 0, sacc, vreg, vt, kb0, u.p,
                                    a.scale_log2);
        if constexpr (!kTiled) wave_lds_sync();   // reads finish before the tile is reused
        return;
    }
    const int64_t off = t0 * a.kv_tok + (int64_t)u.g * a.kv_head;
    if constexpr (KV8) {
        const int64_t soff = t0 * a.s_tok + (int64_t)u.g * a.s_head;
        const int64_t off1 = off + 32 * a.kv_tok, soff1 = soff + 32 * a.s_tok;
        ChunkRegs8 ca, cb;
        load_chunk8(ca, a.k8 + off, a.v8 + off, a.ks + soff, a.vs + soff, a.kv_tok, a.s_tok, u.p - kb0);
        if (kb1 <= u.p)
            load_chunk8(cb, a.k8 + off1, a.v8 + off1, a.ks + soff1, a.vs + soff1, a.kv_tok, a.s_tok, u.p - kb1);
        fold_chunk(st, qb, ca, kb0, u.p, a.scale_log2, vt, sct);
        if (kb1 <= u.p) fold_chunk(st, qb, cb, kb1, u.p, a.scale_log2, vt, sct);
    }
}

// A wave's state to LDS: max and sum per head to wm/wl, the 16 x 128
// unnormalised values to the wave's V tile (free once its folds are done).
__device__ __forceinline__ void decode_stash(const Softmax &st, float *wm, float *wl, uint8_t *vt) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    const float l = sum_over_lane_groups(st.l);
    if (lg == 0) {
        wm[lr] = st.m;
        wl[lr] = l;
    }
    float *wo = reinterpret_cast<float *>(vt);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<floatx4 *>(wo + lr * kHeadDim + 16 * dt + 4 * lg) = st.o[dt];
}

// The partial of the 4 stashed states w0..w0+3 (slot order) for head h, dims
// d0..d0+N-1.  Empty states (no visible key, or no slot) have max -inf and
// weight 0.
template <int N, int kTileBytes>
__device__ __forceinline__ void combine_group(const float (*wm)[16], const float (*wl)[16],
                                              const uint8_t (*vt)[kTileBytes], int w0, int h, int d0, float &M,
                                              float &Ls, float (&acc)[N]) {
    M = fmaxf(fmaxf(wm[w0][h], wm[w0 + 1][h]), fmaxf(wm[w0 + 2][h], wm[w0 + 3][h]));
    Ls = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    if (M == -INFINITY) return;
#pragma unroll
    for (int w = w0; w < w0 + 4; ++w) {
        const float mw = wm[w][h];
        if (mw == -INFINITY) continue;
        const float wgt = exp2f(mw - M);
        Ls += wgt * wl[w][h];
        const float *src = reinterpret_cast<const float *>(vt[w]) + h * kHeadDim + d0;
#pragma unroll
        for (int i0 = 0; i0 < N; i0 += 4) {
            const floatx4 x = *reinterpret_cast<const floatx4 *>(src + i0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i0 + i] += wgt * x[i];
        }
    }
}

// One partial (max mp > -inf, sum lp, values xp) merged into (Ls, acc) under
// the overall max M.
template <int N>
__device__ __forceinline__ void merge_partial(float M, float mp, float lp, const float (&xp)[N], float &Ls,
                                              float (&acc)[N]) {
    const float wgt = exp2f(mp - M);
    Ls += wgt * lp;
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] += wgt * xp[i];
}

// Normalise and store head h, dims d0..d0+N-1 of unit u, and its lse.
template <int N>
__device__ __forceinline__ void decode_write(const AttnArgs &a, const Unit &u, int h, int d0, float M, float Ls,
                                             const float (&acc)[N]) {
    const int hq = a.H * kGroup, hh = u.g * kGroup + h;
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    uint16_t *dst = a.out + ((int64_t)u.r * hq + hh) * kHeadDim + d0;
    if constexpr (N == 8) *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    else *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    if (a.lse && d0 == 0) a.lse[(int64_t)u.r * hq + hh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

// Split-K decode, for launches with few units: workgroup `split` of a unit
// folds slots 4*split .. +3 (one per wave) and combines them into partial
// `split`; with several partials each workgroup publishes its partial and the
// last to arrive (a per-unit counter) merges them.
template <bool KV8, bool kTiled>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a, int wg_per_unit) {
    // per wave: a block's V (strided bf16: both halves), a chunk's (int8), or
    // only the combine's stash (tiled)
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[4][kTiled || KV8 ? 8192 : 16384];
    __shared__ __attribute__((aligned(16))) float sc_all[4][KV8 ? 64 : 4];
    __shared__ float wm[4][16], wl[4][16];
    __shared__ int is_last;
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int64_t unit = blockIdx.x / wg_per_unit;
    const int split = blockIdx.x % wg_per_unit;
    if (unit >= (int64_t)a.b.total_rows * a.H) return;
    const Unit u = make_unit(a, unit);
    const int hq = a.H * kGroup;
    float *part_unit = a.ws_part + unit * wg_per_unit * (int64_t)kPartialFloats;
    const int slot = split * 4 + wave;
    if (slot < a.top_k) {
        Softmax st;
        softmax_init(st);
        // the block index, q and the sequence's first key do not depend on one
        // another: issue them together (in bounds for every unit of the grid)
        const int b_raw = a.idx[((int64_t)u.r * a.H + u.g) * a.top_k + slot];
        const int64_t kv0 = seq_token0(a.b, u.s);
        u32x4 qb[4];
        load_q<KV8>(qb, a.q + ((int64_t)u.r * hq + u.g * kGroup) * kHeadDim);
        decode_fold_block<KV8, kTiled>(a, u, kv0, qb, b_raw, st, vt_all[wave], sc_all[wave]);
        decode_stash(st, wm[wave], wl[wave], vt_all[wave]);
    } else if (lane < 16) {
        wm[wave][lane] = -INFINITY;
        wl[wave][lane] = 0.f;
    }
    __syncthreads();

    // thread = (head h, dims d0..d0+7)
    const int h = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
    float M, Ls, accv[8];
    combine_group<8>(wm, wl, vt_all, 0, h, d0, M, Ls, accv);

    if (wg_per_unit > 1) {
        // Publish the workgroup's partial with agent-scope stores, wait for
        // them, then count the workgroup in; the last one to arrive merges, in
        // split order, reading the others' partials with agent-scope loads.
        // Relaxed atomics order nothing in the language's model: this relies
        // on gfx950 compiling agent-scope stores and loads with the sc1 bit
        // (stores written through the XCD's L2 to the device-coherent level,
        // loads not served from a copy in it), on s_waitcnt returning only
        // once the stores are acknowledged, and on the counter's atomic add
        // being performed at that level.  A release fence would make it
        // formal but writes back the whole L2 in each of the many workgroups.
        // A partial: 16 maxima, 16 sums, then value i of thread t at 32 + 256 i + t
        // (each store and load instruction covers 1 KiB of consecutive words).
        float *pw = part_unit + split * (int64_t)kPartialFloats;
        if (d0 == 0) {
            __hip_atomic_store(pw + h, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pw + 16 + h, Ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __hip_atomic_store(pw + 32 + 256 * i + threadIdx.x, accv[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned prev = __hip_atomic_fetch_add(a.ws_count + unit, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            is_last = prev == (unsigned)(wg_per_unit - 1);
        }
        __syncthreads();
        if (!is_last) return;
        if (threadIdx.x == 0)   // leave the counter at zero for the next call
            __hip_atomic_store(a.ws_count + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!u.ok) return;
        // every split's max, sum and values in one batch of loads (one round
        // trip; splits past the last are not read), then the merge in split
        // order
        float ms[kMaxTopK / 4], lv[kMaxTopK / 4], xv[kMaxTopK / 4][8];
#pragma unroll
        for (int w = 0; w < kMaxTopK / 4; ++w) {
            if (w >= wg_per_unit) break;
            const float *ps = part_unit + w * kPartialFloats;
            ms[w] = __hip_atomic_load(ps + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            lv[w] = __hip_atomic_load(ps + 16 + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                xv[w][i] = __hip_atomic_load(ps + 32 + 256 * i + threadIdx.x, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        }
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kMaxTopK / 4; ++w)
            if (w < wg_per_unit) M = fmaxf(M, ms[w]);
        Ls = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) accv[i] = 0.f;
        if (M != -INFINITY) {
            // an empty partial (max -inf) has weight 0
#pragma unroll
            for (int w = 0; w < kMaxTopK / 4; ++w)
                if (w < wg_per_unit && ms[w] != -INFINITY) merge_partial<8>(M, ms[w], lv[w], xv[w], Ls, accv);
        }
    } else if (!u.ok) {
        return;
    }
    decode_write<8>(a, u, h, d0, M, Ls, accv);
}

// Decode with one workgroup per unit, for launches with many units: 8 waves
// fold 8 slots at a time (pass p: slots 8p + wave), each into a state of its
// own; after each pass the workgroup forms that pass's two partials, kept in
// registers, and merges all partials at the end.  Nothing leaves the CU until
// the output, and the arithmetic is decode_kernel's, step for step.
// Workgroups are dispatched to the chip's 8 XCDs in turn (workgroup i to XCD
// i mod 8), each XCD with its own L2.  Workgroup i takes unit base(i mod 8) +
// i / 8, so every XCD gets one contiguous run of units -- consecutive rows of
// one key head, which in a verify window keep mostly the same blocks, so their
// K/V is fetched into one L2 rather than into all eight.  A bijection of
// [0, n): the first n mod 8 XCDs take one unit more.  A unit's result does not
// depend on which workgroup computes it.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_unit(int64_t i, int64_t n) {
    const int64_t q = n / kXcds, r = n % kXcds, x = i % kXcds, k = i / kXcds;
    return x * q + min(x, r) + k;
}

template <bool KV8, bool kTiled>
__global__ __launch_bounds__(512) void decode_unit_kernel(AttnArgs a) {
    constexpr int kW = 8;
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[kW][kTiled || KV8 ? 8192 : 16384];
    __shared__ __attribute__((aligned(16))) float sc_all[kW][KV8 ? 64 : 4];
    __shared__ float wm[kW][16], wl[kW][16];
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int64_t n_units = (int64_t)a.b.total_rows * a.H;
    if ((int64_t)blockIdx.x >= n_units) return;
    const int64_t unit = xcd_unit(blockIdx.x, n_units);
    const Unit u = make_unit(a, unit);
    const int hq = a.H * kGroup;
    const int64_t kv0 = seq_token0(a.b, u.s);
    u32x4 qb[4];
    load_q<KV8>(qb, a.q + ((int64_t)u.r * hq + u.g * kGroup) * kHeadDim);
    const int n_part = (a.top_k + 3) / 4;   // partials of 4 slots
    // thread = (head h, dims d0..d0+3)
    const int h = threadIdx.x >> 5, d0 = (threadIdx.x & 31) * 4;
    float pm[kMaxTopK / 4], pl[kMaxTopK / 4], px[kMaxTopK / 4][4];
#pragma unroll
    for (int pass = 0; pass < kMaxTopK / kW; ++pass) {
        if (pass * kW >= a.top_k) break;
        if (pass > 0) __syncthreads();   // the previous pass's partials have read the tiles
        const int slot = pass * kW + wave;
        if (slot < a.top_k) {
            Softmax st;
            softmax_init(st);
            const int b_raw = a.idx[((int64_t)u.r * a.H + u.g) * a.top_k + slot];
            decode_fold_block<KV8, kTiled>(a, u, kv0, qb, b_raw, st, vt_all[wave], sc_all[wave]);
            decode_stash(st, wm[wave], wl[wave], vt_all[wave]);
        } else if (lane < 16) {
            wm[wave][lane] = -INFINITY;
            wl[wave][lane] = 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kW / 4; ++j)
            if (pass * (kW / 4) + j < n_part)
                combine_group<4>(wm, wl, vt_all, 4 * j, h, d0, pm[pass * (kW / 4) + j], pl[pass * (kW / 4) + j],
                                 px[pass * (kW / 4) + j]);
    }
    if (!u.ok) return;
    if (n_part == 1) {
        decode_write<4>(a, u, h, d0, pm[0], pl[0], px[0]);
        return;
    }
    float M = -INFINITY, Ls = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kMaxTopK / 4; ++w) M = fmaxf(M, w < n_part ? pm[w] : -INFINITY);
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kMaxTopK / 4; ++w)
            if (w < n_part && pm[w] != -INFINITY) merge_partial<4>(M, pm[w], pl[w], px[w], Ls, acc);
    }
    decode_write<4>(a, u, h, d0, M, Ls, acc);
}

// Waves a prefill launch should have before it trades rows per wave for more
// waves: two per SIMD of the 256 CUs.
constexpr int64_t kPrefillFillWaves = 2048;

template <int RW, bool KV8, bool kTiled>
static void launch_prefill_rw(const AttnArgs &a, hipStream_t st) {
    const int gph = (a.b.total_rows + RW - 1) / RW;
    const int64_t waves = (int64_t)gph * a.H;
    constexpr int kW = RW == 4 ? 4 : 1;   // waves per workgroup
    hipLaunchKernelGGL((prefill_kernel<RW, KV8, kTiled, kW>), dim3((unsigned)((waves + kW - 1) / kW)), dim3(64 * kW),
                       0, st, a, gph);
}

template <bool KV8, bool kTiled>
static void launch_prefill_t(const AttnArgs &a, hipStream_t st) {
    // 4 rows per wave while their 4 * top_k entries fit the 64 lanes, else 2;
    // fewer while the grid would leave SIMDs idle (a short batch walks longer
    // merged lists on fewer waves).  A row's result does not depend on it.
    int rw = a.top_k <= 16 ? 4 : 2;
    while (rw > 1 && (int64_t)((a.b.total_rows + rw - 1) / rw) * a.H < kPrefillFillWaves) rw /= 2;
    if (rw == 4) launch_prefill_rw<4, KV8, kTiled>(a, st);
    else if (rw == 2) launch_prefill_rw<2, KV8, kTiled>(a, st);
    else launch_prefill_rw<1, KV8, kTiled>(a, st);
}

hipError_t launch_prefill(const AttnArgs &a, hipStream_t st) {
    if (a.k8) launch_prefill_t<true, false>(a, st);
    else if (a.tiled) launch_prefill_t<false, true>(a, st);
    else launch_prefill_t<false, false>(a, st);
    return hipGetLastError();
}

// kDecodeUnitKernelMin: below it, the split over several workgroups per unit
// spreads a small batch over more CUs; from it, the one-workgroup kernel
// avoids publishing and re-reading partials (measured at top_k 16: split
// faster at 64 units, 18.3 against 20.2 us; one workgroup faster at 128, 20.9
// against 26.7 us, and at the 256 units of four 16-row windows, 23.7 against
// 42.7 us).

hipError_t launch_decode(const AttnArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.b.total_rows * a.H;
    if (units >= kDecodeUnitKernelMin) {
        const dim3 grid((unsigned)units), block(512);
        if (a.k8) hipLaunchKernelGGL((decode_unit_kernel<true, false>), grid, block, 0, st, a);
        else if (a.tiled) hipLaunchKernelGGL((decode_unit_kernel<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((decode_unit_kernel<false, false>), grid, block, 0, st, a);
        return hipGetLastError();
    }
    const int wg = decode_wg_per_unit(a.top_k);
    const dim3 grid((unsigned)(units * wg)), block(256);
    if (a.k8) hipLaunchKernelGGL((decode_kernel<true, false>), grid, block, 0, st, a, wg);
    else if (a.tiled) hipLaunchKernelGGL((decode_kernel<false, true>), grid, block, 0, st, a, wg);
    else hipLaunchKernelGGL((decode_kernel<false, false>), grid, block, 0, st, a, wg);
    return hipGetLastError();
}

}  // namespace msa
