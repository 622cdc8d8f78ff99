/*
 * CPU oracle for the DeepSeek Sparse Attention lightning indexer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code, header,
 * table or constant with the GPU library; both sides receive the same seeded
 * input bytes and nothing else.
 *
 * What it computes (plain definitions, written for reading rather than speed):
 *
 *  - Index score, DeepSeek-V3.2 architecture section, Eq. (1):
 *        I[t,s] = sum_{j=1..H} w[t,j] * ReLU( q[t,j] . k[s] )
 *    with one key k[s] per token shared by every head. Each q, w and decoded key
 *    element is widened to double, every product and sum is taken in double in
 *    the order the formula is written, and the final double is rounded once (RNE)
 *    to float32.
 *  - Fine-grained token selection, same section: keep the k highest scores of a
 *    row. Ties in value go to the lower index; -0.0 equals +0.0; -inf and NaN
 *    mark keys that do not exist and are never selected. The output lists the
 *    selection in value-descending order and pads with -1 when fewer than k keys
 *    exist (a full sort with std-style comparison, then its prefix).
 *  - Key decoding: fp8 e4m3fn (OCP 8-bit floating point spec), e2m1 with UE8M0
 *    group-32 scales (OCP Microscaling v1.0), bf16; an fp8 key is its code times
 *    the token's fp32 scale, which the llama.cpp thread describes as a
 *    quantisation scale (a multiplier at dequantisation).
 *  - The ways a row names its keys: a contiguous range [ks, ke) (vLLM
 *    sparse_indexer page: row_ks / row_ke), a block table of fixed-size pages
 *    (same page: block_table, row_indices), candidate blocks with a valid
 *    sparse-column count (same page: sparse_indices, end), and candidate blocks of
 *    a paged row (sparse_indices with a per-row block_table).
 *
 * Parallelism: rows are independent (every query is one row in the varlen
 * decode layout), so rows are spread over OpenMP threads. Nothing is blocked,
 * fused or reordered inside a row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { REF_BF16 = 1, REF_FP8_E4M3 = 2, REF_MXFP4 = 3 };

/* ---------------------------------------------------------------- decoding */

/* OCP OFP8 E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent field 0 is subnormal m/8 * 2^(1-7). */
double ref_decode_fp8_e4m3fn(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* OCP MX v1.0 FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; no
 * infinities or NaN; exponent field 0 is subnormal m/2 * 2^(1-1). */
double ref_decode_e2m1(uint8_t nibble)
{
    int sign = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int m = nibble & 1;
    double mag;
    if (e == 0)
        mag = ldexp((double)m / 2.0, 1 - 1);
    else
        mag = ldexp(1.0 + (double)m / 2.0, e - 1);
    return sign ? -mag : mag;
}

/* OCP MX v1.0 E8M0 scale: 2^(E-127); E = 255 is NaN. */
double ref_decode_ue8m0(uint8_t e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* bfloat16: the upper half of an IEEE-754 binary32. */
double ref_decode_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Decode one query row q[t] of heads x dim elements into doubles. */
static void decode_query(const void* q, int q_dtype, int64_t row, int heads, int dim, double* out)
{
    int64_t n = (int64_t)heads * dim;
    for (int64_t i = 0; i < n; i++) {
        if (q_dtype == REF_BF16)
            out[i] = ref_decode_bf16(((const uint16_t*)q)[row * n + i]);
        else
            out[i] = ref_decode_fp8_e4m3fn(((const uint8_t*)q)[row * n + i]);
    }
}

/* Decode the key of one token. ``k`` points at the token's code bytes and
 * ``sc`` at its scale (fp32 for fp8, dim/32 UE8M0 bytes for MXFP4, unused for
 * bf16). */
static void decode_key(const uint8_t* k, const void* sc, int k_dtype, int dim, double* out)
{
    for (int i = 0; i < dim; i++) {
        if (k_dtype == REF_BF16) {
            uint16_t b;
            memcpy(&b, k + 2 * i, 2);
            out[i] = ref_decode_bf16(b);
        } else if (k_dtype == REF_FP8_E4M3) {
            out[i] = ref_decode_fp8_e4m3fn(k[i]) * (double)*(const float*)sc;
        } else {
            uint8_t byte = k[i / 2];
            uint8_t nib = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            out[i] = ref_decode_e2m1(nib) * ref_decode_ue8m0(((const uint8_t*)sc)[i / 32]);
        }
    }
}

static int key_bytes(int k_dtype, int dim)
{
    return k_dtype == REF_BF16 ? 2 * dim : k_dtype == REF_FP8_E4M3 ? dim : dim / 2;
}

static int64_t scale_bytes(int k_dtype, int dim)
{
    return k_dtype == REF_FP8_E4M3 ? 4 : k_dtype == REF_MXFP4 ? dim / 32 : 0;
}

/* Eq. (1) for one query row (decoded) against one decoded key. */
static float index_score(const double* qd, const float* w, int heads, int dim, const double* kd)
{
    double acc = 0.0;
    for (int j = 0; j < heads; j++) {
        double dot = 0.0;
        for (int i = 0; i < dim; i++)
            dot += qd[(int64_t)j * dim + i] * kd[i];
        double relu = dot > 0.0 ? dot : 0.0;
        if (isnan(dot))
            relu = dot;
        acc += (double)w[j] * relu;
    }
    return (float)acc;
}

/* ---------------------------------------------------------------- logits */

/* Contiguous rows: logits[r][c] = I(r, ks[r] + c) for c < ke[r] - ks[r],
 * -inf for the rest of [0, ld). */
void ref_logits_dense(const void* q, int q_dtype, const float* w, const uint8_t* k,
                      const void* k_scale, int k_dtype, const int32_t* row_ks,
                      const int32_t* row_ke, int rows, int heads, int dim, float* logits,
                      int64_t ld)
{
    int kb = key_bytes(k_dtype, dim);
    int64_t sb = scale_bytes(k_dtype, dim);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; r++) {
        double* qd = malloc(sizeof(double) * (size_t)heads * dim);
        double* kd = malloc(sizeof(double) * (size_t)dim);
        decode_query(q, q_dtype, r, heads, dim, qd);
        int64_t len = (int64_t)row_ke[r] - row_ks[r];
        for (int64_t c = 0; c < ld; c++) {
            if (c >= len) {
                logits[r * ld + c] = -INFINITY;
                continue;
            }
            int64_t s = row_ks[r] + c;
            decode_key(k + s * kb, (const uint8_t*)k_scale + s * sb, k_dtype, dim, kd);
            logits[r * ld + c] = index_score(qd, w + (int64_t)r * heads, heads, dim, kd);
        }
        free(qd);
        free(kd);
    }
}

/* Paged rows: token s of row r lives in page block_table[req][s / page_size],
 * slot s % page_size, with req = row_req[r] (or r when row_req is NULL).
 * logits[r][s] for s < seq_lens[r], -inf for the rest of [0, ld). */
void ref_logits_paged(const void* q, int q_dtype, const float* w, const uint8_t* k_pages,
                      const void* k_scale_pages, int k_dtype, int page_size,
                      const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                      const int32_t* row_req, int rows, int heads, int dim, float* logits,
                      int64_t ld)
{
    int kb = key_bytes(k_dtype, dim);
    int64_t sb = scale_bytes(k_dtype, dim);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; r++) {
        double* qd = malloc(sizeof(double) * (size_t)heads * dim);
        double* kd = malloc(sizeof(double) * (size_t)dim);
        decode_query(q, q_dtype, r, heads, dim, qd);
        int64_t req = row_req ? row_req[r] : r;
        for (int64_t s = 0; s < ld; s++) {
            if (s >= seq_lens[r]) {
                logits[r * ld + s] = -INFINITY;
                continue;
            }
            int64_t page = block_table[req * bt_ld + s / page_size];
            int64_t slot = page * page_size + s % page_size;
            decode_key(k_pages + slot * kb, (const uint8_t*)k_scale_pages + slot * sb, k_dtype,
                       dim, kd);
            logits[r * ld + s] = index_score(qd, w + (int64_t)r * heads, heads, dim, kd);
        }
        free(qd);
        free(kd);
    }
}

/* Candidate-block rows: column c names token cand[r][c / block] * block +
 * c % block of the row's range [ks, ke) (relative to ks). A column is scored when
 * c < n_cols[r] (the valid sparse-column count) and its token is < ke - ks;
 * every other column of [0, ld) is -inf. */
void ref_logits_sparse(const void* q, int q_dtype, const float* w, const uint8_t* k,
                       const void* k_scale, int k_dtype, const int32_t* row_ks,
                       const int32_t* row_ke, const int32_t* cand, int64_t cand_ld,
                       const int32_t* n_cols, int block, int rows, int heads, int dim,
                       float* logits, int64_t ld)
{
    int kb = key_bytes(k_dtype, dim);
    int64_t sb = scale_bytes(k_dtype, dim);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; r++) {
        double* qd = malloc(sizeof(double) * (size_t)heads * dim);
        double* kd = malloc(sizeof(double) * (size_t)dim);
        decode_query(q, q_dtype, r, heads, dim, qd);
        int64_t len = (int64_t)row_ke[r] - row_ks[r];
        for (int64_t c = 0; c < ld; c++) {
            int64_t b = c / block;
            int64_t tok = b < cand_ld ? (int64_t)cand[r * cand_ld + b] * block + c % block : -1;
            if (c >= n_cols[r] || b >= cand_ld || tok < 0 || tok >= len) {
                logits[r * ld + c] = -INFINITY;
                continue;
            }
            int64_t s = row_ks[r] + tok;
            decode_key(k + s * kb, (const uint8_t*)k_scale + s * sb, k_dtype, dim, kd);
            logits[r * ld + c] = index_score(qd, w + (int64_t)r * heads, heads, dim, kd);
        }
        free(qd);
        free(kd);
    }
}

/* Candidate blocks over a paged cache (the two-level decode layout of the vLLM
 * sparse_indexer page: a decode row carries a per-row page table next to its
 * sparse_indices, and the indexer cache's page is a multiple of the sparse block).
 * Column c names the row's logical token cand[r][c / block] * block + c % block; it
 * is scored when c < n_cols[r] and the token is < seq_lens[r], reading the key at
 * page block_table[req][token / page_size], slot token % page_size, with req =
 * row_req[r] (or r). Every other column of [0, ld) is -inf. */
void ref_logits_paged_sparse(const void* q, int q_dtype, const float* w, const uint8_t* k_pages,
                             const void* k_scale_pages, int k_dtype, int page_size,
                             const int32_t* block_table, int64_t bt_ld, const int32_t* seq_lens,
                             const int32_t* row_req, const int32_t* cand, int64_t cand_ld,
                             const int32_t* n_cols, int block, int rows, int heads, int dim,
                             float* logits, int64_t ld)
{
    int kb = key_bytes(k_dtype, dim);
    int64_t sb = scale_bytes(k_dtype, dim);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; r++) {
        double* qd = malloc(sizeof(double) * (size_t)heads * dim);
        double* kd = malloc(sizeof(double) * (size_t)dim);
        decode_query(q, q_dtype, r, heads, dim, qd);
        int64_t req = row_req ? row_req[r] : r;
        for (int64_t c = 0; c < ld; c++) {
            int64_t b = c / block;
            int64_t tok = b < cand_ld ? (int64_t)cand[r * cand_ld + b] * block + c % block : -1;
            if (c >= n_cols[r] || b >= cand_ld || tok < 0 || tok >= seq_lens[r]) {
                logits[r * ld + c] = -INFINITY;
                continue;
            }
            int64_t page = block_table[req * bt_ld + tok / page_size];
            int64_t slot = page * page_size + tok % page_size;
            decode_key(k_pages + slot * kb, (const uint8_t*)k_scale_pages + slot * sb, k_dtype,
                       dim, kd);
            logits[r * ld + c] = index_score(qd, w + (int64_t)r * heads, heads, dim, kd);
        }
        free(qd);
        free(kd);
    }
}

/* ---------------------------------------------------------------- top-k */

typedef struct {
    float v;
    int32_t idx;
} scored;

/* Selection order: higher value first; equal values (numeric equality, so
 * -0.0 == +0.0) by lower index. */
static int by_score(const void* pa, const void* pb)
{
    const scored* a = pa;
    const scored* b = pb;
    if (a->v > b->v)
        return -1;
    if (a->v < b->v)
        return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

/* For each row, the k best of logits[r][0 : lens[r]] (lens NULL: all ncols)
 * among entries that are neither -inf nor NaN, in selection order, padded with
 * index -1 / value -inf. out_val may be NULL. */
void ref_topk(const float* logits, int64_t ld, const int32_t* lens, int64_t ncols, int rows,
              int k, int32_t* out_idx, float* out_val, int64_t out_ld)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; r++) {
        int64_t n = lens ? lens[r] : ncols;
        scored* buf = malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
        int64_t m = 0;
        for (int64_t c = 0; c < n; c++) {
            float v = logits[r * ld + c];
            if (isnan(v) || v == -INFINITY)
                continue;
            buf[m].v = v;
            buf[m].idx = (int32_t)c;
            m++;
        }
        qsort(buf, (size_t)m, sizeof(scored), by_score);
        for (int i = 0; i < k; i++) {
            out_idx[r * out_ld + i] = i < m ? buf[i].idx : -1;
            if (out_val)
                out_val[r * out_ld + i] = i < m ? buf[i].v : -INFINITY;
        }
        free(buf);
    }
}

/* ---------------------------------------------------------------- candidate blocks
 *
 * The two-level indexer (vLLM sparse_indexer page: a candidate-source layer publishes
 * candidate_topk_blocks blocks of candidate_block_size tokens that the consuming
 * layers score; DeepGEMM release note: consumers score only the blocks handed to
 * them). The pages do not say how the source layer ranks blocks; the reading taken
 * here: a block's score is the largest score of its tokens (-inf and NaN entries do
 * not count, and a block with no other entry has no score and is never published);
 * the n_top blocks first in the selection order above (higher score first, equal
 * scores by lower block id) are published, in ascending block id as the consumers
 * require, then -1 up to n_top. Returns nothing; n_cand[r] gets the published count.
 * Row r covers tokens 0 .. lens[r]-1 (lens clamped to [0, ncols]); block b covers
 * tokens b*block .. b*block+block-1 of those. */
void ref_candidate_blocks(const float* logits, int64_t ld, const int32_t* lens, int64_t ncols, int rows,
                          int block, int n_top, int32_t* cand, int64_t cand_ld, int32_t* n_cand)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; r++) {
        int64_t n = lens ? lens[r] : ncols;
        if (n < 0)
            n = 0;
        if (n > ncols)
            n = ncols;
        const int64_t nblk = (n + block - 1) / block;
        scored* buf = malloc(sizeof(scored) * (size_t)(nblk > 0 ? nblk : 1));
        int64_t m = 0;
        for (int64_t b = 0; b < nblk; b++) {
            int have = 0;
            float best = 0.0f;
            for (int64_t c = b * block; c < n && c < (b + 1) * block; c++) {
                float v = logits[r * ld + c];
                if (!(v > -INFINITY)) /* -inf or NaN */
                    continue;
                if (!have || v > best)
                    best = v;
                have = 1;
            }
            if (have) {
                buf[m].v = best;
                buf[m].idx = (int32_t)b;
                m++;
            }
        }
        qsort(buf, (size_t)m, sizeof(scored), by_score);
        const int64_t take = m < n_top ? m : n_top;
        /* publish in ascending block id: mark the chosen blocks, then walk the ids */
        unsigned char* chosen = calloc((size_t)(nblk > 0 ? nblk : 1), 1);
        for (int64_t i = 0; i < take; i++)
            chosen[buf[i].idx] = 1;
        int64_t o = 0;
        for (int64_t b = 0; b < nblk; b++)
            if (chosen[b])
                cand[r * cand_ld + o++] = (int32_t)b;
        for (; o < n_top; o++)
            cand[r * cand_ld + o] = -1;
        n_cand[r] = (int32_t)take;
        free(chosen);
        free(buf);
    }
}

/* ---------------------------------------------------------------- key-cache writer
 *
 * Each new key (128 bf16 values) is quantised into the cache format and stored at
 * its slot. The vLLM sparse_indexer page names the formats (an fp8 key with a
 * per-token fp32 scale, and MXFP4 with UE8M0 granularity-32 scales) but not the
 * quantisation recipe, so the plainest readings are taken:
 *  - fp8: scale = amax / 448 (amax the largest |value| of the token, 448 the largest
 *    e4m3fn value), code = the e4m3fn value nearest to value * (448 / amax), ties to
 *    the even code; both quotients and the product in float32; amax = 0 gives scale 0
 *    and zero codes. A key decodes as code * scale, as the scan reads it.
 *  - MXFP4 (OCP MX v1.0 conversion): per group of 32 the shared exponent X =
 *    floor(log2(amax)) - 2 (2 = the largest e2m1 exponent), stored as UE8M0 X + 127
 *    clamped to [0, 254]; each element value / 2^X goes to the nearest e2m1 value,
 *    ties to the even code, magnitudes above 6 to 6.
 * "Nearest" is found by trying every code of the format, so the encoders follow the
 * definition of round-to-nearest-even directly. Signs carry over (-0 keeps its sign).
 */

/* e4m3fn code of a finite float (nearest of the 127 non-negative finite codes by
 * magnitude, ties to the even code; magnitudes above 448 give 448). */
uint8_t ref_encode_fp8_e4m3fn(float y)
{
    double a = fabs((double)y);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 127; c++) { /* 0x7F is NaN */
        double d = fabs(ref_decode_fp8_e4m3fn((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* e2m1 nibble of a finite double (nearest of the 8 magnitudes, ties to the even
 * code, saturating at 6). */
uint8_t ref_encode_e2m1(double v)
{
    double a = fabs(v);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(ref_decode_e2m1((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 8 : 0));
}

/* One key row of 128 bf16 values into the cache format: fp8 -> 128 codes and one
 * float scale; MXFP4 -> 64 bytes (element 2j in the low nibble of byte j) and 4
 * UE8M0 bytes. */
static void quantize_key(const uint16_t* x16, int k_dtype, uint8_t* codes, void* scale)
{
    float x[128];
    for (int i = 0; i < 128; i++)
        x[i] = (float)ref_decode_bf16(x16[i]);
    if (k_dtype == REF_FP8_E4M3) {
        float amax = 0.0f;
        for (int i = 0; i < 128; i++)
            if (fabsf(x[i]) > amax)
                amax = fabsf(x[i]);
        if (amax == 0.0f) {
            for (int i = 0; i < 128; i++)
                codes[i] = ref_encode_fp8_e4m3fn(x[i]); /* +-0 */
            *(float*)scale = 0.0f;
            return;
        }
        float inv = 448.0f / amax;
        for (int i = 0; i < 128; i++)
            codes[i] = ref_encode_fp8_e4m3fn(x[i] * inv);
        *(float*)scale = amax / 448.0f;
        return;
    }
    /* MXFP4 */
    for (int g = 0; g < 4; g++) {
        const float* xg = x + 32 * g;
        float amax = 0.0f;
        for (int i = 0; i < 32; i++)
            if (fabsf(xg[i]) > amax)
                amax = fabsf(xg[i]);
        int X = -127;
        if (amax > 0.0f) {
            int e;
            frexp((double)amax, &e); /* amax = m 2^e, m in [0.5, 1) */
            X = (e - 1) - 2;
        }
        int biased = X + 127;
        if (biased < 0)
            biased = 0;
        if (biased > 254)
            biased = 254;
        ((uint8_t*)scale)[g] = (uint8_t)biased;
        for (int i = 0; i < 32; i += 2) {
            uint8_t lo = ref_encode_e2m1(ldexp((double)xg[i], 127 - biased));
            uint8_t hi = ref_encode_e2m1(ldexp((double)xg[i + 1], 127 - biased));
            codes[16 * g + i / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* Writes n new keys (bf16 [n, 128]) into a cache of n_slots key rows: key i goes to
 * slot slot_mapping[i]; a negative slot (a padding token) writes nothing. fp8: codes
 * [n_slots, 128] + float scales [n_slots]; MXFP4: codes [n_slots, 64] + UE8M0
 * [n_slots, 4]. Slots outside the cache are skipped and counted; returns that count. */
int64_t ref_kcache_write(const uint16_t* k_new, int64_t n, const int64_t* slot_mapping, int k_dtype,
                         uint8_t* cache, void* cache_scale, int64_t n_slots)
{
    const int kb = k_dtype == REF_FP8_E4M3 ? 128 : 64;
    const int sb = k_dtype == REF_FP8_E4M3 ? 4 : 4;
    int64_t bad = 0;
    for (int64_t i = 0; i < n; i++) {
        int64_t s = slot_mapping[i];
        if (s < 0)
            continue;
        if (s >= n_slots) {
            bad++;
            continue;
        }
        quantize_key(k_new + i * 128, k_dtype, cache + s * kb, (uint8_t*)cache_scale + s * sb);
    }
    return bad;
}

int ref_version(void)
{
    return 1;
}
