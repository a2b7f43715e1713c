/*
 * Host backend of the workloads' counter-based input generator (inputs only:
 * no part of the decode method is computed here).
 *
 * For counter c of the stream with key k:
 *     x = (c + k) mod 2^32,  h = lowbias32(x)
 *     value = table[h >> 16]                 (a BF16 bit pattern)
 *     if outlier_per_65536 > 0 and (h & 0xFFFF) < outlier_per_65536:
 *         value = outlier_bits, with the sign bit set when bit 15 of h is 1
 * lowbias32(x): x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b;
 *               x ^= x >> 16   (all mod 2^32).
 * The table (65,536 BF16 quantiles of N(0,1)) is passed in by the caller, so
 * this file holds no data of its own.  The numpy backend in __init__.py is
 * the definition; tests check this file against it bit for bit.
 */
#include <stdint.h>

static uint32_t lowbias32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

/* out[i] = value of counter start + i, i < count */
void gen_draw_bits(uint32_t key, uint64_t start, int64_t count, const uint16_t *table,
                   uint32_t outlier_per_65536, uint16_t outlier_bits, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const uint32_t x = (uint32_t)(start + (uint64_t)i) + key;
        const uint32_t h = lowbias32(x);
        uint16_t v = table[h >> 16];
        if (outlier_per_65536 && (h & 0xFFFFu) < outlier_per_65536)
            v = (uint16_t)(outlier_bits | (((h >> 15) & 1u) ? 0x8000u : 0u));
        out[i] = v;
    }
}
