/*
 * pa_oracle.c -- plain, slow CPU reference for paged decode attention and for
 * the KV-append scatter.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests/, the smoke check and the CPU
 * baseline leg of bench.py can check the GPU library against an independent
 * definition.  It shares no source, header, table or constant with the GPU
 * library.
 *
 * What it computes, and where that is defined:
 *
 *   oracle_decode -- the PagedAttention pseudocode of the vLLM concept page
 *     ("Technical principles" section): for one sequence, walk its page table,
 *     concatenate the key and value blocks it names into one contiguous K and
 *     V, then run standard scaled-dot-product attention of the query over
 *     them: scores = Q.K^T / sqrt(head_dim) (the scale is an argument here),
 *     softmax, then weights.V.  Logical KV is contiguous while its physical
 *     blocks may sit anywhere in the pool (vLLM-internals blog, section 1.1);
 *     only the unfilled tail of the last block is not part of the sequence
 *     (same blog, section 1.2), so the concatenation is cut to seq_len rows.
 *     Query head h reads KV head h / (H / Hkv) (grouped-query attention, as
 *     named on the concept page).  Everything is done in double precision,
 *     with the softmax taken as exp(z - max z) / sum exp(z - max z).
 *
 *   oracle_decode_multi -- several new query tokens per sequence (the verify
 *     step of speculative decoding): query token i of a sequence with q_len
 *     new tokens attends causally to the first L - q_len + i + 1 tokens; each
 *     row is oracle_decode over that prefix.
 *
 *   oracle_kv_append -- write each new token's K and V row into the slot that
 *     slot_mapping names (block = slot / block_size, offset = slot %
 *     block_size): a bit copy for f32 and bf16 caches; for an 8-bit cache the
 *     value x is multiplied in binary32 by inv = 1.0f / scale and stored as the
 *     nearest OCP E4M3FN value (ties to even mantissa), NaN kept as NaN and
 *     magnitudes beyond 448 saturated to +-448.
 *
 *   oracle_e4m3_to_f64 -- the E4M3FN value of a code from the format
 *     definition: sign s, exponent e (4 bits, bias 7), mantissa m (3 bits);
 *     e = 0 gives (-1)^s 2^-6 m/8, S.1111.111 is NaN, otherwise
 *     (-1)^s 2^(e-7) (1 + m/8).  The largest finite value is 448.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -fPIC -shared -ffp-contract=off
 * (no fast-math: the fp32 multiply in the append must round like IEEE binary32).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };
enum { OR_OK = 0, OR_EARG = 1, OR_EBLOCK = 2, OR_ESLOT = 3, OR_ENOMEM = 4, OR_ELEN = 5 };

/* Threads an OpenMP loop of this library runs on (for reporting only). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- codecs */

double oracle_bf16_to_f64(uint16_t h)
{
    /* bf16 is the upper half of an IEEE binary32 */
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3_to_f64(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Non-negative finite E4M3FN values, code 0..126, increasing with the code. */
static double g_e4m3_val[127];

__attribute__((constructor)) static void init_e4m3_table(void)
{
    for (int c = 0; c < 127; ++c)
        g_e4m3_val[c] = oracle_e4m3_to_f64((uint8_t)c);
}

/* Nearest E4M3FN code to binary32 y, ties to the even code (even mantissa). */
uint8_t oracle_e4m3_from_f32(float y)
{
    uint32_t bits;
    memcpy(&bits, &y, sizeof bits);
    uint8_t sign = (bits >> 31) ? 0x80 : 0x00;
    if (isnan(y))
        return sign | 0x7F;
    double a = fabs((double)y);
    if (a >= 448.0)
        return sign | 0x7E;
    /* largest code c with value(c) <= a */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_e4m3_val[mid] <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    double below = a - g_e4m3_val[c];
    double above = g_e4m3_val[c + 1] - a;  /* c < 126 here since a < 448 */
    int pick;
    if (below < above)
        pick = c;
    else if (above < below)
        pick = c + 1;
    else
        pick = (c & 1) ? c + 1 : c;
    return sign | (uint8_t)pick;
}

void oracle_e4m3_encode_array(const float *x, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_from_f32(x[i]);
}

void oracle_e4m3_decode_array(const uint8_t *c, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_to_f64(c[i]);
}

void oracle_bf16_decode_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f64(h[i]);
}

static double load_as_f64(const void *base, int dtype, int64_t idx)
{
    switch (dtype) {
    case OR_F32:
        return (double)((const float *)base)[idx];
    case OR_BF16:
        return oracle_bf16_to_f64(((const uint16_t *)base)[idx]);
    default:
        return oracle_e4m3_to_f64(((const uint8_t *)base)[idx]);
    }
}

/* ---------------------------------------------------------------- decode */

/*
 * q            [S, H, D]            dtype q_dtype (f32 or bf16)
 * key_cache    [NB, bs, Hkv, D]     dtype kv_dtype (f32, bf16 or e4m3 codes)
 * value_cache  [NB, bs, Hkv, D]
 * k_scale, v_scale                  multiply decoded e4m3 K / V (ignored otherwise)
 * block_tables [S, max_nb] int32;  seq_lens [S] int32
 * rows         flat query-row ids s*H + h to compute, or NULL for all S*H in order
 * out          [n_rows, D] double
 * weights      optional [n_rows, weights_stride] double: the softmax weight of
 *              each of the first seq_len tokens (entries beyond are left alone)
 *
 * Returns OR_OK, or an error for a block id outside [0, NB), a length outside
 * [0, max_nb*bs], bad sizes or no memory.  seq_len 0 gives an all-zero row.
 */
int oracle_decode(const void *q, int q_dtype, const void *key_cache, const void *value_cache,
                  int kv_dtype, double k_scale, double v_scale, const int32_t *block_tables,
                  int64_t max_nb, const int32_t *seq_lens, int64_t S, int64_t H, int64_t Hkv,
                  int64_t D, int64_t bs, int64_t NB, double scale, const int64_t *rows,
                  int64_t n_rows, double *out, double *weights, int64_t weights_stride)
{
    if (S < 0 || H <= 0 || Hkv <= 0 || H % Hkv || D <= 0 || bs <= 0 || NB < 0 || max_nb < 0)
        return OR_EARG;
    if (q_dtype != OR_F32 && q_dtype != OR_BF16)
        return OR_EARG;
    if (kv_dtype != OR_F32 && kv_dtype != OR_BF16 && kv_dtype != OR_E4M3)
        return OR_EARG;
    if (rows == NULL)
        n_rows = S * H;
    const int64_t G = H / Hkv;
    const double ks = (kv_dtype == OR_E4M3) ? k_scale : 1.0;
    const double vs = (kv_dtype == OR_E4M3) ? v_scale : 1.0;
    int status = OR_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t row = rows ? rows[r] : r;
        double *o = out + r * D;
        if (row < 0 || row >= S * H) {
#pragma omp atomic write
            status = OR_EARG;
            continue;
        }
        const int64_t s = row / H, h = row % H, kv = h / G;
        const int64_t L = seq_lens[s];
        if (L < 0 || L > max_nb * bs) {
#pragma omp atomic write
            status = OR_ELEN;
            continue;
        }
        for (int64_t d = 0; d < D; ++d)
            o[d] = 0.0;
        if (L == 0)
            continue;

        /* 1. concatenate the blocks named by the page table: K_s, V_s [nb*bs, D] */
        const int64_t nb = (L + bs - 1) / bs;
        double *K = malloc(sizeof(double) * (size_t)(nb * bs * D));
        double *V = malloc(sizeof(double) * (size_t)(nb * bs * D));
        double *z = malloc(sizeof(double) * (size_t)L);
        if (!K || !V || !z) {
            free(K);
            free(V);
            free(z);
#pragma omp atomic write
            status = OR_ENOMEM;
            continue;
        }
        int bad = 0;
        for (int64_t j = 0; j < nb && !bad; ++j) {
            const int64_t phys = block_tables[s * max_nb + j];
            if (phys < 0 || phys >= NB) {
                bad = 1;
                break;
            }
            for (int64_t t = 0; t < bs; ++t)
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t src = ((phys * bs + t) * Hkv + kv) * D + d;
                    K[(j * bs + t) * D + d] = load_as_f64(key_cache, kv_dtype, src) * ks;
                    V[(j * bs + t) * D + d] = load_as_f64(value_cache, kv_dtype, src) * vs;
                }
        }
        if (bad) {
            free(K);
            free(V);
            free(z);
#pragma omp atomic write
            status = OR_EBLOCK;
            continue;
        }

        /* 2. scores over the first L rows only (the concatenation cut to L) */
        const int64_t qbase = (s * H + h) * D;
        double zmax = -INFINITY;
        for (int64_t t = 0; t < L; ++t) {
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d)
                acc += load_as_f64(q, q_dtype, qbase + d) * K[t * D + d];
            z[t] = scale * acc;
            if (z[t] > zmax)
                zmax = z[t];
        }
        /* 3. softmax */
        double denom = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            z[t] = exp(z[t] - zmax);
            denom += z[t];
        }
        for (int64_t t = 0; t < L; ++t)
            z[t] /= denom;
        /* 4. weighted sum of the value rows */
        for (int64_t t = 0; t < L; ++t)
            for (int64_t d = 0; d < D; ++d)
                o[d] += z[t] * V[t * D + d];
        if (weights)
            for (int64_t t = 0; t < L; ++t)
                weights[r * weights_stride + t] = z[t];
        free(K);
        free(V);
        free(z);
    }
    return status;
}

/* ---------------------------------------------------------------- multi-token decode */

/*
 * Several new query tokens per sequence (speculative decoding's verify step,
 * P-EAGLE page: the target model checks K drafted tokens in one pass).
 * query_start_loc [S+1]: sequence s owns query tokens qsl[s] .. qsl[s+1]-1 of
 * q [T, H, D]; they are the sequence's last q_len = qsl[s+1] - qsl[s]
 * positions, so query token i (0-based within the sequence) sits at position
 * L - q_len + i and attends to positions 0 .. L - q_len + i (causal language
 * modelling: a token sees itself and everything before it).  Each output row
 * is exactly oracle_decode of that one query row over the sequence cut to
 * L - q_len + i + 1 tokens.  rows: flat ids token * H + h (NULL = all T * H).
 */
int oracle_decode_multi(const void *q, int q_dtype, const void *key_cache, const void *value_cache,
                        int kv_dtype, double k_scale, double v_scale, const int32_t *block_tables,
                        int64_t max_nb, const int32_t *seq_lens, const int32_t *query_start_loc,
                        int64_t S, int64_t T, int64_t H, int64_t Hkv, int64_t D, int64_t bs,
                        int64_t NB, double scale, const int64_t *rows, int64_t n_rows, double *out)
{
    if (S < 0 || T < 0 || H <= 0 || D <= 0)
        return OR_EARG;
    if (query_start_loc[0] != 0 || query_start_loc[S] != T)
        return OR_EARG;
    for (int64_t s = 0; s < S; ++s)
        if (query_start_loc[s + 1] < query_start_loc[s])
            return OR_EARG;
    if (rows == NULL)
        n_rows = T * H;
    const size_t qelt = q_dtype == OR_F32 ? 4 : 2;
    int status = OR_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t row = rows ? rows[r] : r;
        if (row < 0 || row >= T * H) {
#pragma omp atomic write
            status = OR_EARG;
            continue;
        }
        const int64_t tok = row / H, h = row % H;
        int64_t s = 0;
        while (query_start_loc[s + 1] <= tok)      /* the sequence owning this token */
            ++s;
        const int64_t i = tok - query_start_loc[s];
        const int64_t q_len = query_start_loc[s + 1] - query_start_loc[s];
        const int64_t L = seq_lens[s];
        if (q_len > L) {
#pragma omp atomic write
            status = OR_ELEN;
            continue;
        }
        const int32_t visible = (int32_t)(L - q_len + i + 1);
        const int64_t one_row = h;   /* row h of a one-sequence batch */
        const int rc = oracle_decode((const char *)q + (size_t)(tok * H * D) * qelt, q_dtype,
                                     key_cache, value_cache, kv_dtype, k_scale, v_scale,
                                     block_tables + s * max_nb, max_nb, &visible, 1, H, Hkv, D,
                                     bs, NB, scale, &one_row, 1, out + r * D, NULL, 0);
        if (rc) {
#pragma omp atomic write
            status = rc;
        }
    }
    return status;
}

/* ---------------------------------------------------------------- append */

/*
 * k, v         [T, Hkv, D]  dtype in_dtype
 * slots        [T] int64: block * bs + offset; negative = skip this token
 * key_cache    [NB, bs, Hkv, D] dtype cache_dtype, written in place
 *
 * f32 and bf16 caches need in_dtype == cache_dtype (bit copy).  An e4m3 cache
 * takes f32 or bf16 rows, each value x stored as e4m3(x *f32 (1.0f / scale)).
 * All slots are checked before anything is written.
 */
int oracle_kv_append(const void *k, const void *v, int in_dtype, int64_t T, int64_t Hkv,
                     int64_t D, const int64_t *slots, void *key_cache, void *value_cache,
                     int cache_dtype, int64_t NB, int64_t bs, float k_scale, float v_scale)
{
    if (T < 0 || Hkv <= 0 || D <= 0 || NB < 0 || bs <= 0)
        return OR_EARG;
    if (cache_dtype == OR_E4M3) {
        if (in_dtype != OR_F32 && in_dtype != OR_BF16)
            return OR_EARG;
    } else if (cache_dtype != in_dtype || (cache_dtype != OR_F32 && cache_dtype != OR_BF16)) {
        return OR_EARG;
    }
    for (int64_t t = 0; t < T; ++t)
        if (slots[t] >= NB * bs)
            return OR_ESLOT;

    const float k_inv = 1.0f / k_scale;
    const float v_inv = 1.0f / v_scale;
    const int64_t row = Hkv * D;
    /* slots are unique by contract, so tokens can be written in any order */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const int64_t slot = slots[t];
        if (slot < 0)
            continue;
        const int64_t blk = slot / bs, off = slot % bs;
        const int64_t dst = (blk * bs + off) * row;
        const int64_t src = t * row;
        if (cache_dtype == OR_F32) {
            memcpy((float *)key_cache + dst, (const float *)k + src, sizeof(float) * (size_t)row);
            memcpy((float *)value_cache + dst, (const float *)v + src, sizeof(float) * (size_t)row);
        } else if (cache_dtype == OR_BF16) {
            memcpy((uint16_t *)key_cache + dst, (const uint16_t *)k + src,
                   sizeof(uint16_t) * (size_t)row);
            memcpy((uint16_t *)value_cache + dst, (const uint16_t *)v + src,
                   sizeof(uint16_t) * (size_t)row);
        } else {
            for (int64_t i = 0; i < row; ++i) {
                float xk = (float)load_as_f64(k, in_dtype, src + i);  /* exact: f32/bf16 */
                float xv = (float)load_as_f64(v, in_dtype, src + i);
                float yk = xk * k_inv;
                float yv = xv * v_inv;
                ((uint8_t *)key_cache)[dst + i] = oracle_e4m3_from_f32(yk);
                ((uint8_t *)value_cache)[dst + i] = oracle_e4m3_from_f32(yv);
            }
        }
    }
    return OR_OK;
}
