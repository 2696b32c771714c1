/*
 * Exhaustive check of the oracle's E4M3FN encoder over every binary32 bit
 * pattern, against a second encoder written here by a different method.
 *
 * The oracle picks the nearest of the 127 non-negative finite E4M3FN values by
 * searching a table.  This file instead rounds the binary32 fields directly:
 * keep the top 3 mantissa bits and round the 20 dropped bits to nearest, ties
 * to even (a carry moves into the exponent); below 2^-6 the value is rounded
 * to an integer multiple of 2^-9 the same way.  NaN stays NaN (S.1111.111) and
 * magnitudes >= 448 (infinity included) saturate to S.1111.110 -- the OCP
 * 8-bit floating point specification's E4M3 with saturation.
 *
 * Prints the number of mismatches (and the first few); exit status 0 iff none.
 */
#include <inttypes.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t oracle_e4m3_from_f32(float y);

static uint8_t encode_fields(uint32_t bits)
{
    const uint8_t sign = (uint8_t)((bits >> 24) & 0x80u);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    if (mag > 0x7F800000u)                 /* NaN */
        return sign | 0x7Fu;
    if (mag >= 0x43E00000u)                /* >= 448.0f, infinity included */
        return sign | 0x7Eu;
    const uint32_t exp = mag >> 23;        /* biased binary32 exponent */
    const uint32_t man = mag & 0x7FFFFFu;
    if (exp >= 121u) {                     /* >= 2^-6: a normal E4M3 value */
        uint32_t code = ((exp - 120u) << 3) | (man >> 20);
        const uint32_t rest = man & 0xFFFFFu, half = 0x80000u;
        if (rest > half || (rest == half && (code & 1u)))
            code += 1u;
        return sign | (uint8_t)code;
    }
    /* below 2^-6: count units of 2^-9.  value = M * 2^(exp - 150) with M the
       full significand (exp >= 1), or man * 2^-149 for a binary32 subnormal. */
    const uint32_t M = exp ? (man | 0x800000u) : man;
    const uint32_t shift = exp ? (141u - exp) : 140u;  /* value / 2^-9 = M >> shift */
    if (shift >= 32u)
        return sign;                       /* far below half a unit */
    uint32_t q = M >> shift;
    const uint32_t rest = M & ((1u << shift) - 1u), half = 1u << (shift - 1u);
    if (rest > half || (rest == half && (q & 1u)))
        q += 1u;
    return sign | (uint8_t)q;
}

int main(void)
{
    uint64_t mismatches = 0;
#pragma omp parallel for reduction(+ : mismatches) schedule(static, 1 << 20)
    for (int64_t i = 0; i < (int64_t)1 << 32; ++i) {
        const uint32_t bits = (uint32_t)i;
        float f;
        memcpy(&f, &bits, sizeof f);
        const uint8_t a = oracle_e4m3_from_f32(f), b = encode_fields(bits);
        if (a != b) {
            if (mismatches < 5) {
#pragma omp critical
                printf("mismatch bits=0x%08" PRIx32 " oracle=0x%02x fields=0x%02x\n", bits, a, b);
            }
            ++mismatches;
        }
    }
    printf("%" PRIu64 "\n", mismatches);
    return mismatches != 0;
}
