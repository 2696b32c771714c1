/*
 * Drives every function of oracle/pa_oracle.c on small inputs, success and
 * error paths alike, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check the oracle's host memory accesses.
 * Exit status 0 when every return code is the expected one.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

int oracle_decode(const void *q, int q_dtype, const void *key_cache, const void *value_cache,
                  int kv_dtype, double k_scale, double v_scale, const int32_t *block_tables,
                  int64_t max_nb, const int32_t *seq_lens, int64_t S, int64_t H, int64_t Hkv,
                  int64_t D, int64_t bs, int64_t NB, double scale, const int64_t *rows,
                  int64_t n_rows, double *out, double *weights, int64_t weights_stride);
int oracle_decode_multi(const void *q, int q_dtype, const void *key_cache, const void *value_cache,
                        int kv_dtype, double k_scale, double v_scale, const int32_t *block_tables,
                        int64_t max_nb, const int32_t *seq_lens, const int32_t *query_start_loc,
                        int64_t S, int64_t T, int64_t H, int64_t Hkv, int64_t D, int64_t bs,
                        int64_t NB, double scale, const int64_t *rows, int64_t n_rows, double *out);
int oracle_kv_append(const void *k, const void *v, int in_dtype, int64_t T, int64_t Hkv,
                     int64_t D, const int64_t *slots, void *key_cache, void *value_cache,
                     int cache_dtype, int64_t NB, int64_t bs, float k_scale, float v_scale);
void oracle_e4m3_encode_array(const float *x, uint8_t *out, int64_t n);
void oracle_e4m3_decode_array(const uint8_t *c, double *out, int64_t n);
void oracle_bf16_decode_array(const uint16_t *h, double *out, int64_t n);
int oracle_num_threads(void);

enum { F32 = 0, BF16 = 1, E4M3 = 2 };
enum { S = 3, H = 4, HKV = 2, D = 8, BS = 4, NB = 8, MAXNB = 3 };

static int failures = 0;
#define EXPECT(call, want)                                                                     \
    do {                                                                                       \
        int rc_ = (call);                                                                      \
        if (rc_ != (want)) {                                                                   \
            printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_, (want));   \
            ++failures;                                                                        \
        }                                                                                      \
    } while (0)

static uint32_t rng = 12345u;
static float frand(void)
{
    rng = rng * 1664525u + 1013904223u;
    return (float)((rng >> 8) & 0xffff) / 32768.0f - 1.0f;
}
static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void)
{
    float qf[S * H * D], kf[NB * BS * HKV * D], vf[NB * BS * HKV * D];
    uint16_t qb[S * H * D], kb[NB * BS * HKV * D], vb[NB * BS * HKV * D];
    uint8_t k8[NB * BS * HKV * D], v8[NB * BS * HKV * D];
    for (int i = 0; i < S * H * D; ++i) {
        qf[i] = frand();
        qb[i] = to_bf16(qf[i]);
    }
    for (int i = 0; i < NB * BS * HKV * D; ++i) {
        kf[i] = frand();
        vf[i] = frand();
        kb[i] = to_bf16(kf[i]);
        vb[i] = to_bf16(vf[i]);
    }
    oracle_e4m3_encode_array(kf, k8, NB * BS * HKV * D);
    oracle_e4m3_encode_array(vf, v8, NB * BS * HKV * D);
    /* tables: seq 0 empty, seq 1 two blocks (5 tokens), seq 2 three blocks (11 tokens); -1 unused */
    int32_t bt[S * MAXNB] = {-1, -1, -1, 4, 1, -1, 7, 0, 2};
    int32_t lens[S] = {0, 5, 11};
    double out[S * H * D], w[S * H * MAXNB * BS];
    const double sc = 1.0 / sqrt((double)D);

    EXPECT(oracle_decode(qf, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, S, H, HKV, D, BS, NB, sc,
                         NULL, 0, out, w, MAXNB * BS), 0);
    EXPECT(oracle_decode(qb, BF16, kb, vb, BF16, 1, 1, bt, MAXNB, lens, S, H, HKV, D, BS, NB, sc,
                         NULL, 0, out, NULL, 0), 0);
    EXPECT(oracle_decode(qb, BF16, k8, v8, E4M3, 0.5, 0.25, bt, MAXNB, lens, S, H, HKV, D, BS, NB,
                         sc, NULL, 0, out, NULL, 0), 0);
    int64_t rows[3] = {11, 4, 0};
    EXPECT(oracle_decode(qf, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, S, H, HKV, D, BS, NB, sc,
                         rows, 3, out, w, MAXNB * BS), 0);
    int64_t bad_row[1] = {S * H};
    EXPECT(oracle_decode(qf, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, S, H, HKV, D, BS, NB, sc,
                         bad_row, 1, out, NULL, 0), 1);
    int32_t bt_bad[S * MAXNB] = {-1, -1, -1, 4, NB, -1, 7, 0, 2};         /* id == NB */
    EXPECT(oracle_decode(qf, F32, kf, vf, F32, 1, 1, bt_bad, MAXNB, lens, S, H, HKV, D, BS, NB, sc,
                         NULL, 0, out, NULL, 0), 2);
    int32_t lens_bad[S] = {0, 5, MAXNB * BS + 1};
    EXPECT(oracle_decode(qf, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens_bad, S, H, HKV, D, BS, NB, sc,
                         NULL, 0, out, NULL, 0), 5);
    EXPECT(oracle_decode(qf, 7, kf, vf, F32, 1, 1, bt, MAXNB, lens, S, H, HKV, D, BS, NB, sc, NULL,
                         0, out, NULL, 0), 1);

    /* several query tokens: seq 1 has 2, seq 2 has 3 (T = 5), seq 0 none */
    float qm[5 * H * D];
    for (int i = 0; i < 5 * H * D; ++i)
        qm[i] = frand();
    int32_t qsl[S + 1] = {0, 0, 2, 5};
    double outm[5 * H * D];
    EXPECT(oracle_decode_multi(qm, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, qsl, S, 5, H, HKV, D,
                               BS, NB, sc, NULL, 0, outm), 0);
    int64_t mrows[2] = {19, 0};
    EXPECT(oracle_decode_multi(qm, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, qsl, S, 5, H, HKV, D,
                               BS, NB, sc, mrows, 2, outm), 0);
    int32_t qsl_long[S + 1] = {0, 0, 5, 5};        /* 5 query tokens on a 5-token sequence: ok */
    EXPECT(oracle_decode_multi(qm, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, qsl_long, S, 5, H, HKV,
                               D, BS, NB, sc, NULL, 0, outm), 0);
    int32_t qsl_over[S + 1] = {0, 5, 5, 5};        /* 5 query tokens on an empty sequence */
    EXPECT(oracle_decode_multi(qm, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, qsl_over, S, 5, H, HKV,
                               D, BS, NB, sc, NULL, 0, outm), 5);
    int32_t qsl_bad[S + 1] = {0, 3, 2, 5};         /* decreasing */
    EXPECT(oracle_decode_multi(qm, F32, kf, vf, F32, 1, 1, bt, MAXNB, lens, qsl_bad, S, 5, H, HKV,
                               D, BS, NB, sc, NULL, 0, outm), 1);

    /* append: one padding token, the rest into distinct slots */
    enum { T = 4 };
    int64_t slots[T] = {-1, 5, NB * BS - 1, 17};
    float kn[T * HKV * D], vn[T * HKV * D];
    uint16_t knb[T * HKV * D], vnb[T * HKV * D];
    for (int i = 0; i < T * HKV * D; ++i) {
        kn[i] = frand() * 300.0f;
        vn[i] = frand();
        knb[i] = to_bf16(kn[i]);
        vnb[i] = to_bf16(vn[i]);
    }
    EXPECT(oracle_kv_append(kn, vn, F32, T, HKV, D, slots, kf, vf, F32, NB, BS, 1, 1), 0);
    EXPECT(oracle_kv_append(knb, vnb, BF16, T, HKV, D, slots, kb, vb, BF16, NB, BS, 1, 1), 0);
    EXPECT(oracle_kv_append(knb, vnb, BF16, T, HKV, D, slots, k8, v8, E4M3, NB, BS, 0.37f, 3.0f), 0);
    EXPECT(oracle_kv_append(kn, vn, F32, T, HKV, D, slots, k8, v8, E4M3, NB, BS, 0.37f, 3.0f), 0);
    EXPECT(oracle_kv_append(kn, vn, F32, T, HKV, D, slots, kb, vb, BF16, NB, BS, 1, 1), 1);
    int64_t slots_bad[T] = {0, 1, NB * BS, 2};
    EXPECT(oracle_kv_append(kn, vn, F32, T, HKV, D, slots_bad, kf, vf, F32, NB, BS, 1, 1), 3);

    /* codecs over every code */
    uint8_t codes[256];
    uint16_t bcodes[256];
    double dec[256];
    for (int i = 0; i < 256; ++i) {
        codes[i] = (uint8_t)i;
        bcodes[i] = (uint16_t)(i * 257);
    }
    oracle_e4m3_decode_array(codes, dec, 256);
    oracle_bf16_decode_array(bcodes, dec, 256);
    float special[6] = {NAN, INFINITY, -INFINITY, 0.0f, -0.0f, 1e30f};
    uint8_t sp8[6];
    oracle_e4m3_encode_array(special, sp8, 6);
    if (oracle_num_threads() < 1)
        ++failures;

    printf("oracle sanitizer run: %d failure(s)\n", failures);
    return failures != 0;
}
