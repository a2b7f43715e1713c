/*
 * fp8kv CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct implementation of one paged decode step
 * over an FP8 (e4m3) KV cache with page-tag integrity, in binary64.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * this file's library.  It shares no code, header, table or helper with the
 * HIP library: every function below is written from the definitions.
 *
 * Sources (the write-ups on running Kimi and GLM at scale):
 *  - "Smaller, faster, safer: running Kimi and GLM at scale" (Cloudflare
 *    post body, KV-cache section): the cache is stored as FP8 e4m3 instead
 *    of BF16 and the attention kernel converts values as it reads them.
 *  - same post, integrity section; and the commentary page's section
 *    "Giving Every Physical Cache Page a 'Generation Number'" (pseudocode):
 *    every physical page carries a tag that changes on reallocation, each
 *    request records the (page, tag) pairs it expects, the mapping is checked
 *    before decode reads the cache, a mismatch aborts only that request
 *    (fail closed: no output).
 *  - FP8 e4m3 format: OCP 8-bit floating point, E4M3 variant (bias 7,
 *    no infinities, S.1111.111 is NaN, largest finite 448).
 *
 * Readings where the pages are silent (scale granularity, rounding, the
 * attention formula, the GQA mapping, the output of an aborted request) are
 * the plain ones: per-kv-head fp32 scales for K and V; x/scale rounded to
 * binary32 and then to e4m3 by round-to-nearest-even with saturation at 448;
 * textbook single-query scaled dot-product attention with q-head h reading
 * kv-head h / (Hq/Hkv); aborted rows are written as +0.
 *
 * Logical cache layout used here: [num_pages][Hkv][page_size][head_dim],
 * one byte (e4m3) or one uint16 (bf16) per element.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* e4m3 decode: straight from the format definition.                          */
/*   code = s eeee mmm, bias 7                                                */
/*   e == 0            : (-1)^s * m * 2^-9          (subnormal, incl. +-0)    */
/*   e == 15 && m == 7 : NaN                                                  */
/*   otherwise         : (-1)^s * (1 + m/8) * 2^(e-7)                         */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_decode(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return copysign(NAN, s ? -1.0 : 1.0); /* NaN keeps the sign bit */
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

void oracle_e4m3_table(double *out256) {
    for (int c = 0; c < 256; ++c) out256[c] = oracle_e4m3_decode((uint8_t)c);
}

/* ------------------------------------------------------------------------ */
/* e4m3 encode: the code whose magnitude is nearest to |v| among the 127      */
/* finite non-negative magnitudes (codes 0x00..0x7E, strictly increasing).    */
/* An exact tie picks the even code (= round half to even on the mantissa).   */
/* |v| beyond the largest magnitude saturates to 0x7E (448); +-inf too.       */
/* The sign bit is copied from v (so -0 and negative underflow give 0x80).    */
/* NaN gives 0x7F with the sign of v.                                         */
/* The 127 magnitudes and the 126 midpoints between neighbours are taken     */
/* once from the decode above (each midpoint is exact in binary64: a few     */
/* significant bits); encoding is a binary search over the magnitudes and    */
/* one exact comparison with the midpoint.                                   */
/* ------------------------------------------------------------------------ */
static double g_mag[127];  /* magnitude of code c, c = 0..126 */
static double g_mid[126];  /* midpoint of codes c and c+1     */

__attribute__((constructor)) static void build_encode_tables(void) {
    for (int c = 0; c < 127; ++c) g_mag[c] = oracle_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 126; ++c) g_mid[c] = (g_mag[c] + g_mag[c + 1]) / 2.0;
}

uint8_t oracle_e4m3_encode(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs(v);
    if (a >= g_mag[126]) return (uint8_t)(sign | 0x7E);
    /* largest c in [0,126) with mag(c) <= a, by binary search */
    int lo = 0, hi = 126; /* invariant: mag(lo) <= a < mag(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_mag[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double midpoint = g_mid[lo]; /* between lo and hi = lo + 1 */
    int c;
    if (a < midpoint)
        c = lo;
    else if (a > midpoint)
        c = hi;
    else
        c = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | c);
}

/* Encode an array of binary32 values (same rule as oracle_e4m3_encode). */
void oracle_e4m3_encode_f32_array(const float *in, uint8_t *out, long n) {
    for (long i = 0; i < n; ++i) out[i] = oracle_e4m3_encode((double)in[i]);
}

/* BF16 bits -> value (exact). */
static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a binary64 value to the nearest BF16 (ties to even).  BF16 carries
 * 8 significant bits and binary32's exponent range. */
uint16_t oracle_bf16_rne(double x) {
    if (isnan(x)) return 0x7FC0;
    double a = fabs(x);
    double r;
    if (a == 0.0 || isinf(a)) {
        r = a;
    } else if (a < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(a, 133)), -133); /* subnormal quantum 2^-133 */
    } else {
        int e;
        double f = frexp(a, &e);                    /* a = f * 2^e, f in [0.5,1) */
        r = ldexp(nearbyint(ldexp(f, 8)), e - 8);   /* 8 significant bits */
        if (r > 3.3895313892515355e38) r = INFINITY; /* above max finite bf16 */
    }
    float fr = (float)r; /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &fr, 4);
    uint16_t bits = (uint16_t)(u >> 16);
    if (signbit(x)) bits |= 0x8000;
    return bits;
}

/* ------------------------------------------------------------------------ */
/* Tag check (the generation-number pseudocode, applied to the pages the     */
/* step's attention reads).  n_b = ceil(ctx_lens[b] / page_size).  A request */
/* aborts iff one of its first n_b entries names a page outside [0, N) or a  */
/* page whose current tag differs from the expected one.  A length that does */
/* not fit the table aborts too (fail closed).                               */
/* ------------------------------------------------------------------------ */
void oracle_verify(const int32_t *page_table, const uint32_t *expected_tags,
                   int32_t max_pages, const int32_t *ctx_lens, int32_t batch,
                   const uint32_t *pool_tags, int32_t num_pages, int32_t page_size,
                   uint8_t *abort_out) {
    for (int b = 0; b < batch; ++b) {
        int ctx = ctx_lens[b];
        int bad = 0;
        if (ctx < 0) {
            bad = 1;
        } else {
            long n = ((long)ctx + page_size - 1) / page_size;
            if (n > max_pages) {
                bad = 1;
            } else {
                for (long i = 0; i < n; ++i) {
                    int32_t id = page_table[(long)b * max_pages + i];
                    if (id < 0 || id >= num_pages) {
                        bad = 1;
                        continue;
                    }
                    if (pool_tags[id] != expected_tags[(long)b * max_pages + i]) bad = 1;
                }
            }
        }
        abort_out[b] = (uint8_t)bad;
    }
}

/* ------------------------------------------------------------------------ */
/* Quantize-on-append.  Token t (request seq[t], position pos[t]) goes to    */
/* page page_table[seq][pos / page_size], slot pos % page_size.  For every  */
/* kv-head h and dim d: code = E( fl32( bf16(x) / scale[h] ) ).              */
/* fl32(x/s) is the binary32 quotient rounded to nearest even; computing    */
/* x/s in binary64 and rounding to binary32 gives exactly that quotient     */
/* (binary64 carries more than 2*24+2 significand bits).                     */
/* A BF16 cache stores the BF16 bits unchanged.                              */
/* Tokens of aborted requests are skipped; so are tokens whose request is   */
/* not a row of the table (num_seqs rows), whose position falls outside the  */
/* table, or whose page entry is out of range (nothing is written: a token  */
/* with no valid destination must not land in a page someone else holds).  */
/* Returns the number skipped for an invalid request, position or entry.    */
/* ------------------------------------------------------------------------ */
int oracle_append(int32_t cache_dtype, int32_t num_pages, int32_t page_size,
                  int32_t num_kv_heads, int32_t head_dim, void *k_cache, void *v_cache,
                  const float *k_scale, const float *v_scale, const uint16_t *k_new,
                  const uint16_t *v_new, int32_t num_tokens, const int32_t *token_seq,
                  const int32_t *token_pos, const int32_t *page_table, int32_t num_seqs,
                  int32_t max_pages, const uint8_t *abort_flags) {
    /* 1. where each token goes: page and slot (page -1: nowhere) */
    size_t nt = (size_t)(num_tokens > 0 ? num_tokens : 1);
    int32_t *dst_page = (int32_t *)malloc(sizeof(int32_t) * nt);
    int32_t *dst_slot = (int32_t *)malloc(sizeof(int32_t) * nt);
    int skipped = 0;
    for (long t = 0; t < num_tokens; ++t) {
        int b = token_seq[t];
        int pos = token_pos[t];
        dst_page[t] = -1;
        dst_slot[t] = 0;
        if (b < 0 || b >= num_seqs) {
            ++skipped;
            continue;
        }
        if (abort_flags && abort_flags[b]) continue;
        if (pos < 0 || pos / page_size >= max_pages) {
            ++skipped;
            continue;
        }
        int32_t page = page_table[(long)b * max_pages + pos / page_size];
        if (page < 0 || page >= num_pages) {
            ++skipped;
            continue;
        }
        dst_page[t] = page;
        dst_slot[t] = pos % page_size;
    }
    /* 2. the elements: every (kv-head, dim) column is independent of the
     *    others; inside a column the tokens go in order, so a slot named by
     *    several tokens keeps the last one, as a plain loop over tokens would.
     *    Columns are taken 32 dims at a time (one task per block). */
    const int blk = 32;
    long blocks = (long)num_kv_heads * ((head_dim + blk - 1) / blk);
#pragma omp parallel for schedule(static)
    for (long k = 0; k < blocks; ++k) {
        int h = (int)(k / ((head_dim + blk - 1) / blk));
        int d0 = (int)(k % ((head_dim + blk - 1) / blk)) * blk;
        int d1 = d0 + blk < head_dim ? d0 + blk : head_dim;
        for (long t = 0; t < num_tokens; ++t) {
            if (dst_page[t] < 0) continue;
            long dst = (((long)dst_page[t] * num_kv_heads + h) * page_size + dst_slot[t]) * head_dim;
            long src = ((long)t * num_kv_heads + h) * head_dim;
            for (int d = d0; d < d1; ++d) {
                if (cache_dtype == 0) {
                    float kq = (float)(bf16_value(k_new[src + d]) / (double)k_scale[h]);
                    float vq = (float)(bf16_value(v_new[src + d]) / (double)v_scale[h]);
                    ((uint8_t *)k_cache)[dst + d] = oracle_e4m3_encode((double)kq);
                    ((uint8_t *)v_cache)[dst + d] = oracle_e4m3_encode((double)vq);
                } else {
                    ((uint16_t *)k_cache)[dst + d] = k_new[src + d];
                    ((uint16_t *)v_cache)[dst + d] = v_new[src + d];
                }
            }
        }
    }
    free(dst_slot);
    free(dst_page);
    return skipped;
}

/* value of one cached element, times its per-head scale, in binary64 (exact:
 * a 4-bit significand times a 24-bit one fits in 53 bits). */
static double cache_value(int32_t cache_dtype, const void *cache, long idx, float scale) {
    if (cache_dtype == 0)
        return oracle_e4m3_decode(((const uint8_t *)cache)[idx]) * (double)scale;
    return bf16_value(((const uint16_t *)cache)[idx]);
}

/* ------------------------------------------------------------------------ */
/* Single-query scaled dot-product attention over the paged cache, binary64. */
/* For request b (not aborted), q-head h, kv-head g = h / (Hq/Hkv), tokens    */
/* j in [0, ctx_lens[b]) at page page_table[b][j/page_size], slot j%page_size:*/
/*   s_j = sm_scale * sum_d q[b][h][d] * khat_j[d]                           */
/*   w_j = exp(s_j - max_j s_j)                                              */
/*   o[d] = sum_j w_j vhat_j[d] / sum_j w_j                                  */
/* khat = DEC(code) * k_scale[g] for e4m3 (BF16 value for a BF16 cache).     */
/* Aborted requests and empty contexts give o = +0.                          */
/* Outputs: out64 [B][Hq][D] binary64; out_bf16 (nullable) RNE of out64.     */
/* Requests are assumed to name valid pages (the tag check guarantees it for */
/* every request it lets through); an invalid entry returns -1.              */
/* rows (nullable): only compute these (b*Hq+h) rows; others are untouched. */
/* ------------------------------------------------------------------------ */
int oracle_attention(int32_t cache_dtype, int32_t num_pages, int32_t page_size,
                     int32_t num_kv_heads, int32_t head_dim, const void *k_cache,
                     const void *v_cache, const float *k_scale, const float *v_scale,
                     const uint16_t *q, int32_t num_q_heads, const int32_t *page_table,
                     int32_t max_pages, const int32_t *ctx_lens, int32_t batch,
                     float sm_scale, const uint8_t *abort_flags, double *out64,
                     uint16_t *out_bf16, const int32_t *rows, int32_t num_rows) {
    int G = num_q_heads / num_kv_heads;
    long total = rows ? (long)num_rows : (long)batch * num_q_heads;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < total; ++r) {
        long row = rows ? (long)rows[r] : r;
        int b = (int)(row / num_q_heads);
        int h = (int)(row % num_q_heads);
        int g = h / G;
        double *o = out64 + row * head_dim;
        for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
        int n = ctx_lens[b];
        int ok = !(abort_flags && abort_flags[b]) && n > 0;
        for (int j = 0; ok && j < n; ++j) {
            if (j / page_size >= max_pages) { ok = 0; break; }
            int32_t page = page_table[(long)b * max_pages + j / page_size];
            if (page < 0 || page >= num_pages) { ok = 0; break; }
        }
        if (!(abort_flags && abort_flags[b]) && n > 0 && !ok) {
#pragma omp atomic write
            status = -1;
        }
        if (ok) {
            double *s = (double *)malloc(sizeof(double) * (size_t)n);
            const uint16_t *qr = q + row * head_dim;
            double smax = -INFINITY;
            for (int j = 0; j < n; ++j) {
                int32_t page = page_table[(long)b * max_pages + j / page_size];
                long base = (((long)page * num_kv_heads + g) * page_size + j % page_size) * head_dim;
                double dot = 0.0;
                for (int d = 0; d < head_dim; ++d)
                    dot += bf16_value(qr[d]) * cache_value(cache_dtype, k_cache, base + d, k_scale[g]);
                s[j] = (double)sm_scale * dot;
                if (s[j] > smax) smax = s[j];
            }
            double wsum = 0.0;
            for (int j = 0; j < n; ++j) {
                double w = exp(s[j] - smax);
                int32_t page = page_table[(long)b * max_pages + j / page_size];
                long base = (((long)page * num_kv_heads + g) * page_size + j % page_size) * head_dim;
                for (int d = 0; d < head_dim; ++d)
                    o[d] += w * cache_value(cache_dtype, v_cache, base + d, v_scale[g]);
                wsum += w;
            }
            for (int d = 0; d < head_dim; ++d) o[d] /= wsum;
            free(s);
        }
        if (out_bf16)
            for (int d = 0; d < head_dim; ++d) out_bf16[row * head_dim + d] = oracle_bf16_rne(o[d]);
    }
    return status;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the attention rows are spread over (timing only; results do not
 * depend on it: every row is computed by one thread in a fixed order). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
