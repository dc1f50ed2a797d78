// attention.hip -- exact softmax attention over the kept blocks.
//
// For query head h of key head g = h / 16 and a row at position p:
//   out[h] = sum_j softmax_j(scale * q[h].k[j]) v[j]  over the kept blocks'
//   keys j <= p;  lse[h] = log sum_j exp(scale * q[h].k[j]).
// The 16 query heads of a key head share the row's selection, so a wave holds
// all 16 heads of one (row, key head) and reads every kept key/value once for
// all of them (TensorFold pull request 1388, commit on 4,096-row prompt
// chunks).  Decode splits the kept keys into partials of 32-key pieces merged
// by a log-sum-exp combine (same pull request, commit adding the minimax_m3
// family).
//
// Per 32-key chunk, on v_mfma_f32_16x16x32_bf16:
//   S^T[key][head] = K Q^T      2 key tiles x 4 k-steps over the 128 dims
//   O^T[d][head]  += V^T P^T    8 d-tiles x one 32-key k-step
// With S^T, a lane holds one head's scores for 8 keys, which is exactly the
// P^T operand layout of the second product, so probabilities go from the
// softmax straight into the MFMA without leaving registers, and the running
// max / sum / rescale of a head stay inside its 4 lanes.  V is written to LDS
// transposed (d-major, keys permuted to the lanes' k-slot order, 16-byte
// groups XOR-swizzled) so each V^T operand is one conflict-free 16-byte read.
// Softmax runs in base 2 on scale*log2(e)-prescaled scores.
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

// Byte offset of 16-byte group `grp` (of 4) in row d of the transposed V tile.
__device__ __forceinline__ int vt_offset(int d, int grp) {
    return d * 64 + ((grp ^ (((d >> 2) ^ (d >> 4)) & 3)) << 4);
}

// Query B operand: head (lane % 16), dims 32*(lane/16) + 8*s + (0..7).
__device__ __forceinline__ void load_q(u32x4 (&qb)[4], const uint16_t *qrow_head0) {
    const int lane = threadIdx.x & 63;
    const uint16_t *src = qrow_head0 + (lane & 15) * kHeadDim + 32 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = load16(src + 8 * s);
}

// Registers of one 32-key chunk: K as MFMA A operands (key kbase + 16*mt +
// lane%16, dims 32*(lane/16) + 8*s) and V rows (keys kbase + 4*(lane/8) +
// 0..3, dims 16*(lane%8) + 0..15).  A key past p is read from key p instead
// (always in bounds): its score is masked to -inf, so its weight is 0.
struct ChunkRegs {
    u32x4 ka[2][4];
    u32x4 vr[4][2];
};

__device__ __forceinline__ void load_chunk(ChunkRegs &c, const uint16_t *kseq, const uint16_t *vseq,
                                           int64_t tok, int kbase, int p) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int key = min(kbase + 16 * mt + lr, p);
        const uint16_t *src = kseq + (int64_t)key * tok + 32 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) c.ka[mt][s] = load16(src + 8 * s);
    }
    const int kg = lane >> 3, dc = lane & 7;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int key = min(kbase + 4 * kg + kk, p);
        const uint16_t *src = vseq + (int64_t)key * tok + 16 * dc;
        c.vr[kk][0] = load16(src);
        c.vr[kk][1] = load16(src + 8);
    }
}

// Write one loaded chunk's V^T into this wave's 8 KiB LDS tile.  Key k of the
// chunk goes to slot 8*((k%16)/4) + 4*(k/16) + k%4, so lane group lg's
// k-slots (keys 4lg..4lg+3 and 16+4lg..16+4lg+3) are the 8 contiguous slots of
// group lg.  Keys 4kg..4kg+3 share one 8-byte word per dim.
__device__ __forceinline__ void stage_v(const ChunkRegs &c, uint8_t *vt) {
    const int lane = threadIdx.x & 63;
    const int kg = lane >> 3, dc = lane & 7;
    const int grp = kg & 3, half = kg >> 2;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int reg = t >> 3, dw = (t & 7) >> 1;
        uint32_t w0, w1;
        if (t & 1) {
            w0 = (c.vr[0][reg][dw] >> 16) | (c.vr[1][reg][dw] & 0xffff0000u);
            w1 = (c.vr[2][reg][dw] >> 16) | (c.vr[3][reg][dw] & 0xffff0000u);
        } else {
            w0 = (c.vr[0][reg][dw] & 0xffffu) | (c.vr[1][reg][dw] << 16);
            w1 = (c.vr[2][reg][dw] & 0xffffu) | (c.vr[3][reg][dw] << 16);
        }
        const int d = 16 * dc + t;
        *reinterpret_cast<uint2 *>(vt + vt_offset(d, grp) + 8 * half) = make_uint2(w0, w1);
    }
}

// Fold the chunk [kbase, kbase + 32) (keys <= p visible) into st: K operands
// from registers, V^T from the LDS tile (already staged and synced).
__device__ __forceinline__ void fold_staged(Softmax &st, const u32x4 (&qb)[4], const u32x4 (&ka)[2][4],
                                            int kbase, int p, float scale_log2, const uint8_t *vt) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    floatx4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_16x16x32(ka[mt][s], qb[s], acc);
        sacc[mt] = acc;
    }
    // Online softmax over this lane's 8 keys of head lr.
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = sacc[mt][i] * scale_log2;
            if (kbase + 16 * mt + 4 * lg + i > p) v = -INFINITY;
            z[mt][i] = v;
            mx = fmaxf(mx, v);
        }
    mx = max_over_lane_groups(mx);
    const float m_new = fmaxf(st.m, mx);        // finite: key kbase <= p is visible
    const float alpha = exp2f(st.m - m_new);    // 0 on the first chunk
    float pr[2][4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[mt][i] = exp2f(z[mt][i] - m_new);
            psum += pr[mt][i];
        }
    st.l = st.l * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
    const u32x4 pb = {pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                      pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const u32x4 va = *reinterpret_cast<const u32x4 *>(vt + vt_offset(16 * dt + lr, lg));
        st.o[dt] = mfma_16x16x32(va, pb, st.o[dt]);
    }
}

// Fold one loaded 32-key chunk into st (stage V^T, fold, release the tile).
__device__ __forceinline__ void fold_chunk(Softmax &st, const u32x4 (&qb)[4], const ChunkRegs &c,
                                           int kbase, int p, float scale_log2, uint8_t *vt) {
    stage_v(c, vt);
    wave_lds_sync();
    fold_staged(st, qb, c.ka, kbase, p, scale_log2, vt);
    wave_lds_sync();   // reads finish before the next chunk overwrites the tile
}

__device__ __forceinline__ void attend_chunk32(Softmax &st, const u32x4 (&qb)[4],
                                               const uint16_t *kseq, const uint16_t *vseq,
                                               int64_t tok, int kbase, int p, float scale_log2,
                                               uint8_t *vt) {
    ChunkRegs c;
    load_chunk(c, kseq, vseq, tok, kbase, p);
    fold_chunk(st, qb, c, kbase, p, scale_log2, vt);
}

// Unit (row r, key head g) of a head-major enumeration: consecutive units are
// consecutive rows of one key head, so neighbouring waves share local blocks.
struct Unit {
    int r, g, s, p;
    bool ok;
};

__device__ __forceinline__ Unit make_unit(const AttnArgs &a, int64_t unit) {
    Unit u;
    u.g = (int)(unit / a.b.total_rows);
    u.r = (int)(unit % a.b.total_rows);
    u.s = locate_seq(a.b.cu_rows, a.b.n_seqs, u.r);
    const int rows_s = a.b.cu_rows[u.s + 1] - a.b.cu_rows[u.s];
    const int L = a.b.seq_lens[u.s];
    u.ok = rows_s > 0 && rows_s <= L && L <= a.b.max_seq_len;
    u.p = L - rows_s + (u.r - a.b.cu_rows[u.s]);
    return u;
}

// Prefill.  One wave per (row, key head): it holds the group's 16 query heads
// (so every kept block is read once for all of them) and walks the row's kept
// blocks in ascending order, 32 keys at a time, with the next chunk's K/V
// loads in flight while the current one is folded.  A row's bits depend only
// on its own blocks and their order.  Consecutive units are consecutive rows
// of one key head, so a workgroup's waves share their local blocks.
__device__ __forceinline__ void prefill_unit(const AttnArgs &a, int64_t unit, uint8_t *vt) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
    const Unit u = make_unit(a, unit);
    if (!u.ok) return;
    const int hq = a.H * kGroup;
    const int64_t kv0 = a.b.kv_start[u.s];
    const uint16_t *kseq = a.k + kv0 * a.kv_tok + (int64_t)u.g * a.kv_head;
    const uint16_t *vseq = a.v + kv0 * a.kv_tok + (int64_t)u.g * a.kv_head;
    u32x4 qb[4];
    load_q(qb, a.q + ((int64_t)u.r * hq + u.g * kGroup) * kHeadDim);
    // Lane t holds kept block t; read with v_readlane (loaded before the
    // pipelined loop, so the loop never waits on it).
    const int32_t *sel = a.idx + ((int64_t)u.r * a.H + u.g) * a.top_k;
    const int my_b = lane < a.top_k ? sel[lane] : -1;

    Softmax st;
    softmax_init(st);
    int t = 0, half = 0;
    auto chunk_base = [&](int tt, int hh) -> int {
        const int b = __builtin_amdgcn_readlane(my_b, tt);
        const int kb = b * kBlock + 32 * hh;
        return (b < 0 || kb > u.p) ? -1 : kb;
    };
    auto next_chunk = [&]() -> int {     // advances (t, half) to the next visible chunk
        for (;;) {
            half ^= 1;
            if (half == 0 && ++t >= a.top_k) return -1;
            const int kb = chunk_base(t, half);
            if (kb >= 0) return kb;
        }
    };
    force_ready(my_b);
    int kb0 = chunk_base(0, 0);
    if (kb0 < 0) kb0 = next_chunk();
    ChunkRegs ca, cb;
    if (kb0 >= 0) load_chunk(ca, kseq, vseq, a.kv_tok, kb0, u.p);
#pragma unroll
    for (int s = 0; s < 4; ++s) force_ready(qb[s]);   // q complete before the loop
    while (kb0 >= 0) {
        const int kb1 = next_chunk();
        if (kb1 >= 0) load_chunk(cb, kseq, vseq, a.kv_tok, kb1, u.p);
        fold_chunk(st, qb, ca, kb0, u.p, a.scale_log2, vt);
        if (kb1 < 0) break;
        kb0 = next_chunk();
        if (kb0 >= 0) load_chunk(ca, kseq, vseq, a.kv_tok, kb0, u.p);
        fold_chunk(st, qb, cb, kb1, u.p, a.scale_log2, vt);
    }

    const float l = sum_over_lane_groups(st.l);
    const int h = u.g * kGroup + lr;
    uint16_t *dst = a.out + ((int64_t)u.r * hq + h) * kHeadDim + 4 * lg;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const uint2 w = make_uint2(pack_bf16x2(st.o[dt][0] * inv, st.o[dt][1] * inv),
                                   pack_bf16x2(st.o[dt][2] * inv, st.o[dt][3] * inv));
        *reinterpret_cast<uint2 *>(dst + 16 * dt) = w;
    }
    if (a.lse && lg == 0) a.lse[(int64_t)u.r * hq + h] = l > 0.f ? (st.m + log2f(l)) * kLn2 : -INFINITY;
}

__global__ __launch_bounds__(256) void prefill_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[4][8192];
    const int wave = uniform(threadIdx.x >> 6);
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave;
    if (unit < (int64_t)a.b.total_rows * a.H) prefill_unit(a, unit, vt_all[wave]);
}

// Decode: the kept list of a (row, key head) is split into top_k partials of
// one block (two 32-key chunks) each; wave `slot` folds partial `slot`, with
// both chunks' loads in flight together, and writes (max, sum, weighted
// values) to the workspace.  Workgroups of 4 waves take 4 consecutive slots;
// the last workgroup of a unit to finish (a per-unit counter) merges all its
// partials, in slot order, with log-sum-exp weights.  The partials and their
// merge order depend only on top_k, so a row's bits never depend on the rest
// of the batch or on which workgroup finished last.
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a, int wg_per_unit) {
    __shared__ __attribute__((aligned(16))) uint8_t vt_all[4][8192];
    __shared__ int is_last;
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int lg = lane >> 4, lr = lane & 15;
    const int64_t unit = blockIdx.x / wg_per_unit;
    const int split = blockIdx.x % wg_per_unit;
    if (unit >= (int64_t)a.b.total_rows * a.H) return;
    const Unit u = make_unit(a, unit);
    const int hq = a.H * kGroup;
    float *part_unit = a.ws_part + unit * a.top_k * (int64_t)kPartialFloats;
    const int slot = split * 4 + wave;

    if (slot < a.top_k) {
        Softmax st;
        softmax_init(st);
        // the block index, q and the sequence's first key do not depend on one
        // another: issue them together (in bounds for every unit of the grid)
        const int b_raw = a.idx[((int64_t)u.r * a.H + u.g) * a.top_k + slot];
        const int64_t kv0 = a.b.kv_start[u.s];
        u32x4 qb[4];
        load_q(qb, a.q + ((int64_t)u.r * hq + u.g * kGroup) * kHeadDim);
        const int b = u.ok ? b_raw : -1;
        const int kb0 = b * kBlock, kb1 = kb0 + 32;
        if (b >= 0 && kb0 <= u.p) {
            const uint16_t *kseq = a.k + kv0 * a.kv_tok + (int64_t)u.g * a.kv_head;
            const uint16_t *vseq = a.v + kv0 * a.kv_tok + (int64_t)u.g * a.kv_head;
            ChunkRegs ca, cb;
            load_chunk(ca, kseq, vseq, a.kv_tok, kb0, u.p);
            if (kb1 <= u.p) load_chunk(cb, kseq, vseq, a.kv_tok, kb1, u.p);
            fold_chunk(st, qb, ca, kb0, u.p, a.scale_log2, vt_all[wave]);
            if (kb1 <= u.p) fold_chunk(st, qb, cb, kb1, u.p, a.scale_log2, vt_all[wave]);
        }
        const float l = sum_over_lane_groups(st.l);
        float *part = part_unit + slot * (int64_t)kPartialFloats;
        if (lg == 0) {
            part[lr] = st.m;
            part[16 + lr] = l;
        }
        float *acc = part + 32 + lr * kHeadDim + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<floatx4 *>(acc + 16 * dt) = st.o[dt];
    }
    // Publish this workgroup's partials, count it in; the last one merges.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.ws_count + unit, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        is_last = prev == (unsigned)(wg_per_unit - 1);
    }
    __syncthreads();
    if (!is_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (threadIdx.x == 0)   // leave the counter at zero for the next call
        __hip_atomic_store(a.ws_count + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!u.ok) return;

    // Merge: thread = (head h, 8 dims), partials in slot order.  Loads go out
    // in batches of 8 partials (no loop-carried load chains).
    const int h = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
    float ms[kMaxTopK];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        ms[s] = s < a.top_k ? part_unit[s * kPartialFloats + h] : -INFINITY;
        M = fmaxf(M, ms[s]);
    }
    float accv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int s0 = 0; s0 < kMaxTopK; s0 += 8) {
            if (s0 >= a.top_k) break;
            float lv[8];
            floatx4 x0[8], x1[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                // an empty partial (no visible key) or a slot past top_k has weight 0;
                // read slot 0 instead so every load stays in bounds and finite
                const bool use = s0 + q < a.top_k && ms[s0 + q] != -INFINITY;
                const float *ps = part_unit + (use ? s0 + q : 0) * kPartialFloats;
                lv[q] = ps[16 + h];
                x0[q] = *reinterpret_cast<const floatx4 *>(ps + 32 + h * kHeadDim + d0);
                x1[q] = *reinterpret_cast<const floatx4 *>(ps + 32 + h * kHeadDim + d0 + 4);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bool use = s0 + q < a.top_k && ms[s0 + q] != -INFINITY;
                if (!use) continue;
                const float w = exp2f(ms[s0 + q] - M);
                Ls += w * lv[q];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accv[i] += w * x0[q][i];
                    accv[4 + i] += w * x1[q][i];
                }
            }
        }
    }
    const int hh = u.g * kGroup + h;
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    u32x4 wv;
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = pack_bf16x2(accv[2 * i] * inv, accv[2 * i + 1] * inv);
    *reinterpret_cast<u32x4 *>(a.out + ((int64_t)u.r * hq + hh) * kHeadDim + d0) = wv;
    if (a.lse && d0 == 0) a.lse[(int64_t)u.r * hq + hh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

hipError_t launch_prefill(const AttnArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.b.total_rows * a.H;
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_decode(const AttnArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.b.total_rows * a.H;
    const int wg = decode_wg_per_unit(a.top_k);
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)(units * wg)), dim3(256), 0, st, a, wg);
    return hipGetLastError();
}

}  // namespace msa
