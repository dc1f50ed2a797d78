/*
 * msa_oracle.c -- plain, slow, obviously-correct CPU reference for MiniMax-M3's
 * block-sparse attention (MSA).  TEST INFRASTRUCTURE ONLY: it is used by the
 * tests, by the smoke check and by the benchmark's CPU-baseline leg, never by the
 * product path.  It shares no code, header or table with the GPU library.
 *
 * What it follows (the pages give prose, not formulas):
 *   - "minimax-m3-sm120", section "What this fixes": the MSA model does a
 *     top-16 block selection per GQA group, scores blocks by max-pooling and
 *     always keeps the local block.
 *   - TensorFold pull request 1388 ("minimax_m3: a CUDA backend ..."), commit
 *     message that introduces the family: the lightning indexer gives index
 *     scores and a top-16 block selection per row and key head; decode attends
 *     over the kept blocks; prompt chunks attend over each tile's kept blocks.
 *   - same pull request, commit message on 4,096-row prompt chunks: the 16
 *     query heads of one key head share their row's block selection.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - index score = plain dot product iq . ik, no activation, no weight;
 *   - block size 64, max over the block's causally visible keys only;
 *   - the local block counts inside the top_k (local + best top_k-1 others);
 *   - ties between equal block scores go to the lower block index;
 *   - a key j is visible to a row at position p iff j <= p;
 *   - query head h belongs to key head floor(h / group).
 *
 * Precision: every sum is taken in double precision in ascending index order.
 * The block-score decision (the top-k) is taken on the scores rounded to
 * float, the precision the GPU kernels decide in; the Python wrapper does that
 * rounding explicitly before calling oracle_select_blocks().
 *
 * Parity status: every function here is pinned by CPU tests (closed forms,
 * brute force on tiny inputs, dense attention through a library routine);
 * parity with the trained model's real indexer form is unpinned (no weights).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* bf16 bit pattern -> value.  A bf16 is the top half of an IEEE binary32. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The sequence that owns global row r (cu_rows is a prefix sum of rows). */
static int seq_of_row(int n_seqs, const int32_t *cu_rows, int r)
{
    for (int s = 0; s < n_seqs; ++s)
        if (r >= cu_rows[s] && r < cu_rows[s + 1])
            return s;
    return -1;
}

/*
 * Position of global row r: the rows of a sequence are its last n positions,
 * so row i of n sits at seq_len - n + i.  Returns -1 on malformed metadata.
 */
static int64_t row_position(int n_seqs, const int32_t *cu_rows,
                            const int32_t *seq_lens, int r, int *seq_out)
{
    int s = seq_of_row(n_seqs, cu_rows, r);
    if (s < 0)
        return -1;
    int n = cu_rows[s + 1] - cu_rows[s];
    if (n > seq_lens[s])
        return -1;
    *seq_out = s;
    return (int64_t)seq_lens[s] - n + (r - cu_rows[s]);
}

/*
 * Steps 1 and 2: lightning-indexer scores and per-block max-pool.
 *   s[j]  = sum_d iq[r, g, d] * ik[j, g, d]         for every key j <= p
 *   S[b]  = max { s[j] : j in block b, j <= p }      for b <  floor(p/B)+1
 *   S[b]  = -inf                                     for b >= floor(p/B)+1
 * Output is double, [n_out, n_kv_heads, bs_stride]; row list `rows` selects
 * which global rows to compute (NULL: all rows, in order).
 * ik_head_stride == 0 means one index key shared by every key head.
 */
int oracle_block_scores(int n_seqs, const int32_t *cu_rows,
                        const int32_t *seq_lens, const int64_t *kv_start,
                        int n_kv_heads, int index_dim, int block,
                        const uint16_t *iq, const uint16_t *ik,
                        int64_t ik_tok_stride, int64_t ik_head_stride,
                        const int32_t *rows, int n_out, int bs_stride,
                        double *scores, int n_threads)
{
    int bad = 0;
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t u = 0; u < (int64_t)n_out * n_kv_heads; ++u) {
        int o = (int)(u / n_kv_heads), g = (int)(u % n_kv_heads);
        int r = rows ? rows[o] : o, s;
        int64_t p = row_position(n_seqs, cu_rows, seq_lens, r, &s);
        double *S = scores + ((int64_t)o * n_kv_heads + g) * bs_stride;
        if (p < 0 || p / block + 1 > bs_stride) {
            bad = 1;
            continue;
        }
        int64_t nb = p / block + 1;
        const uint16_t *qv = iq + ((int64_t)r * n_kv_heads + g) * index_dim;
        for (int64_t b = 0; b < bs_stride; ++b) {
            double best = -INFINITY;
            if (b < nb) {
                int64_t j_end = (b + 1) * block - 1;
                if (j_end > p)
                    j_end = p;
                for (int64_t j = b * block; j <= j_end; ++j) {
                    const uint16_t *kv = ik + (kv_start[s] + j) * ik_tok_stride +
                                         (int64_t)g * ik_head_stride;
                    double acc = 0.0;
                    for (int d = 0; d < index_dim; ++d)
                        acc += bf16_value(qv[d]) * bf16_value(kv[d]);
                    if (acc > best)
                        best = acc;
                }
            }
            S[b] = best;
        }
    }
    return bad ? -1 : 0;
}

/*
 * Step 3: top-k block selection for one (row, key head), on float scores.
 * nb = number of causal blocks of the row; the local block is nb-1.
 *   nb <= top_k : every block 0..nb-1 is kept;
 *   otherwise   : the local block, plus the top_k-1 highest-scoring blocks
 *                 among 0..nb-2, equal scores preferring the lower index.
 * The kept indices are written in ascending order, padded with -1.
 * Selection is done by repeated arg-max, the literal definition.
 */
static void select_one(const float *S, int64_t nb, int top_k, int32_t *out)
{
    char *taken = calloc((size_t)(nb > 0 ? nb : 1), 1);
    int n = 0;
    if (nb <= top_k) {
        for (int64_t b = 0; b < nb; ++b)
            taken[b] = 1;
    } else {
        taken[nb - 1] = 1;                      /* forced local block */
        for (int t = 0; t < top_k - 1; ++t) {
            int64_t arg = -1;
            for (int64_t b = 0; b < nb - 1; ++b) {
                if (taken[b])
                    continue;
                if (arg < 0 || S[b] > S[arg])   /* strict: ties keep lower b */
                    arg = b;
            }
            taken[arg] = 1;
        }
    }
    for (int64_t b = 0; b < nb; ++b)
        if (taken[b])
            out[n++] = (int32_t)b;
    while (n < top_k)
        out[n++] = -1;
    free(taken);
}

/* nb[u] is the causal block count of output row u; scores/out are row-major
 * [n_out, n_kv_heads, bs_stride] and [n_out, n_kv_heads, top_k]. */
int oracle_select_blocks(int n_out, int n_kv_heads, int bs_stride,
                         const int64_t *nb, const float *scores, int top_k,
                         int32_t *block_idx, int n_threads)
{
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t u = 0; u < (int64_t)n_out * n_kv_heads; ++u) {
        int o = (int)(u / n_kv_heads);
        select_one(scores + u * bs_stride, nb[o], top_k, block_idx + u * top_k);
    }
    return 0;
}

/*
 * Step 4: exact softmax attention over the kept keys, one key head's group of
 * query heads sharing the selection.  For query head h (key head g = h/group):
 *   J   = { j : floor(j/B) in block_idx[r, g, :], j <= p }
 *   z_j = scale * sum_d q[r, h, d] * k[j, g, d]
 *   m   = max_j z_j ;  w_j = exp(z_j - m) ;  l = sum_j w_j
 *   o   = sum_j w_j v[j, g, :] / l ;  lse = m + log(l)
 * An empty J gives o = 0 and lse = -inf.  block_idx rows follow `rows`.
 * out is double [n_out, n_kv_heads*group, head_dim]; lse may be NULL.
 */
/* Where attention reads its keys and values: bf16 values, or int8 codes with
 * one fp32 scale per (token, key head) (the value is code * scale). */
typedef struct {
    int int8;
    const uint16_t *k16, *v16;
    const int8_t *k8, *v8;
    const float *ks, *vs;
    int64_t tok, head;          /* elements of k / v */
    int64_t stok, shead;        /* elements of the scale arrays */
} kv_source;

static double kv_value(const kv_source *src, int is_v, int64_t t, int g, int d)
{
    int64_t e = t * src->tok + (int64_t)g * src->head + d;
    if (!src->int8)
        return bf16_value(is_v ? src->v16[e] : src->k16[e]);
    double scale = (double)(is_v ? src->vs : src->ks)[t * src->stok + (int64_t)g * src->shead];
    return (double)(is_v ? src->v8[e] : src->k8[e]) * scale;
}

static int attention_core(int n_seqs, const int32_t *cu_rows, const int32_t *seq_lens,
                          const int64_t *kv_start, int n_kv_heads, int group,
                          int head_dim, int block, int top_k, double scale,
                          const uint16_t *q, const kv_source *src,
                          const int32_t *block_idx, const int32_t *rows, int n_out,
                          double *out, double *lse, int n_threads)
{
    int bad = 0;
    int n_q = n_kv_heads * group;
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel reduction(| : bad)
    {
        int64_t cap = (int64_t)top_k * block;
        double *z = malloc(sizeof(double) * (size_t)cap);
        int64_t *key = malloc(sizeof(int64_t) * (size_t)cap);
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < (int64_t)n_out * n_kv_heads; ++u) {
            int o = (int)(u / n_kv_heads), g = (int)(u % n_kv_heads);
            int r = rows ? rows[o] : o, s;
            int64_t p = row_position(n_seqs, cu_rows, seq_lens, r, &s);
            if (p < 0) {
                bad = 1;
                continue;
            }
            /* gather the visible keys of the kept blocks, in list order */
            int64_t nk = 0;
            const int32_t *sel = block_idx + u * top_k;
            for (int t = 0; t < top_k; ++t) {
                if (sel[t] < 0)
                    continue;
                if ((int64_t)sel[t] * block > p) {
                    bad = 1;                    /* block beyond the row */
                    continue;
                }
                for (int64_t j = (int64_t)sel[t] * block;
                     j < (int64_t)(sel[t] + 1) * block && j <= p; ++j)
                    key[nk++] = j;
            }
            for (int hh = 0; hh < group; ++hh) {
                int h = g * group + hh;
                const uint16_t *qv = q + ((int64_t)r * n_q + h) * head_dim;
                double *ov = out + ((int64_t)o * n_q + h) * head_dim;
                for (int d = 0; d < head_dim; ++d)
                    ov[d] = 0.0;
                if (nk == 0) {
                    if (lse)
                        lse[(int64_t)o * n_q + h] = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (int64_t t = 0; t < nk; ++t) {
                    int64_t tok = kv_start[s] + key[t];
                    double acc = 0.0;
                    for (int d = 0; d < head_dim; ++d)
                        acc += bf16_value(qv[d]) * kv_value(src, 0, tok, g, d);
                    z[t] = scale * acc;
                    if (z[t] > m)
                        m = z[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < nk; ++t) {
                    int64_t tok = kv_start[s] + key[t];
                    double w = exp(z[t] - m);
                    l += w;
                    for (int d = 0; d < head_dim; ++d)
                        ov[d] += w * kv_value(src, 1, tok, g, d);
                }
                for (int d = 0; d < head_dim; ++d)
                    ov[d] /= l;
                if (lse)
                    lse[(int64_t)o * n_q + h] = m + log(l);
            }
        }
        free(z);
        free(key);
    }
    return bad ? -1 : 0;
}

int oracle_attention(int n_seqs, const int32_t *cu_rows, const int32_t *seq_lens,
                     const int64_t *kv_start, int n_kv_heads, int group,
                     int head_dim, int block, int top_k, double scale,
                     const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int64_t kv_tok_stride, int64_t kv_head_stride,
                     const int32_t *block_idx, const int32_t *rows, int n_out,
                     double *out, double *lse, int n_threads)
{
    kv_source src = {0};
    src.k16 = k;
    src.v16 = v;
    src.tok = kv_tok_stride;
    src.head = kv_head_stride;
    return attention_core(n_seqs, cu_rows, seq_lens, kv_start, n_kv_heads, group, head_dim, block,
                          top_k, scale, q, &src, block_idx, rows, n_out, out, lse, n_threads);
}

/*
 * Attention over an int8 key/value cache: every key and value element is
 * code * scale, with one fp32 scale per (token, key head) (TensorFold pull
 * request 1388, commit adding the minimax_m3 family: keys and values cached as
 * int8 with a scale per position and head; the scores take the keys' scales
 * and the weights the values' scales).  Otherwise exactly oracle_attention.
 */
int oracle_attention_kv8(int n_seqs, const int32_t *cu_rows, const int32_t *seq_lens,
                         const int64_t *kv_start, int n_kv_heads, int group,
                         int head_dim, int block, int top_k, double scale,
                         const uint16_t *q, const int8_t *k8, const int8_t *v8,
                         const float *k_scale, const float *v_scale,
                         int64_t tok_stride, int64_t head_stride,
                         int64_t scale_tok_stride, int64_t scale_head_stride,
                         const int32_t *block_idx, const int32_t *rows, int n_out,
                         double *out, double *lse, int n_threads)
{
    kv_source src = {0};
    src.int8 = 1;
    src.k8 = k8;
    src.v8 = v8;
    src.ks = k_scale;
    src.vs = v_scale;
    src.tok = tok_stride;
    src.head = head_stride;
    src.stok = scale_tok_stride;
    src.shead = scale_head_stride;
    return attention_core(n_seqs, cu_rows, seq_lens, kv_start, n_kv_heads, group, head_dim, block,
                          top_k, scale, q, &src, block_idx, rows, n_out, out, lse, n_threads);
}

/*
 * The int8 cache's quantisation of one bf16 (token, head) row of head_dim
 * values (this library's reading: the pages name a scale per position and head
 * but not its rule).  Taken in fp32, as the kernel that writes the cache does:
 *   scale = max_d |x_d| / 127             (fp32 division)
 *   code_d = round_half_even(x_d / scale), clamped to [-127, 127]
 * A row of zeros gets scale 0 and codes 0.  Inputs must be finite.
 */
void oracle_quantize_kv8(int64_t n_tokens, int n_heads, int head_dim, const uint16_t *x,
                         int64_t tok_stride, int64_t head_stride, int8_t *codes,
                         int64_t code_tok_stride, int64_t code_head_stride, float *scales,
                         int64_t scale_tok_stride, int64_t scale_head_stride)
{
    for (int64_t t = 0; t < n_tokens; ++t)
        for (int g = 0; g < n_heads; ++g) {
            const uint16_t *row = x + t * tok_stride + (int64_t)g * head_stride;
            int8_t *crow = codes + t * code_tok_stride + (int64_t)g * code_head_stride;
            float amax = 0.0f;
            for (int d = 0; d < head_dim; ++d) {
                float a = fabsf((float)bf16_value(row[d]));
                if (a > amax)
                    amax = a;
            }
            volatile float sc = amax / 127.0f;     /* a float, stored: no wider intermediate */
            scales[t * scale_tok_stride + (int64_t)g * scale_head_stride] = sc;
            for (int d = 0; d < head_dim; ++d) {
                if (sc == 0.0f) {
                    crow[d] = 0;
                    continue;
                }
                volatile float ratio = (float)bf16_value(row[d]) / sc;
                float c = rintf(ratio);
                if (c > 127.0f)
                    c = 127.0f;
                if (c < -127.0f)
                    c = -127.0f;
                crow[d] = (int8_t)c;
            }
        }
}
