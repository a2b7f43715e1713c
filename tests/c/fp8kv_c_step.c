/*
 * One decode step driven through the C ABI alone (no Python, no torch),
 * checked against the CPU oracle.  Test code: it links the library and the
 * oracle's library and compares them.
 *
 * Three requests hold prompts of 37, 100 and 260 tokens in an e4m3 cache
 * (16 q-heads over 2 kv-heads); their pages come from the library's pool,
 * whose tags go to the device with fp8kv_pool_sync.  Request 1 remembers a
 * wrong tag for one of its pages.  The step is the fused check + append of
 * each request's new token and the attention for one query per request.
 *
 * Checked: the abort flags equal the oracle's ({0, 1, 0}); every byte of both
 * pools equals the oracle's cache through fp8kv_cache_offset (so the aborted
 * request's new token was not written); every output row is within 2e-3 of
 * the oracle's binary64 attention, and the aborted request's rows are +0.
 * Prints one line and exits 0 on success, 1 on a mismatch, 2 on an error.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8kv.h"

/* the oracle's entry points (oracle/fp8kv_oracle.c) */
void oracle_verify(const int32_t *page_table, const uint32_t *expected_tags, int32_t max_pages,
                   const int32_t *ctx_lens, int32_t batch, const uint32_t *pool_tags,
                   int32_t num_pages, int32_t page_size, uint8_t *abort_out);
int oracle_append(int32_t cache_dtype, int32_t num_pages, int32_t page_size,
                  int32_t num_kv_heads, int32_t head_dim, void *k_cache, void *v_cache,
                  const float *k_scale, const float *v_scale, const uint16_t *k_new,
                  const uint16_t *v_new, int32_t num_tokens, const int32_t *token_seq,
                  const int32_t *token_pos, const int32_t *page_table, int32_t num_seqs,
                  int32_t max_pages, const uint8_t *abort_flags);
int oracle_attention(int32_t cache_dtype, int32_t num_pages, int32_t page_size,
                     int32_t num_kv_heads, int32_t head_dim, const void *k_cache,
                     const void *v_cache, const float *k_scale, const float *v_scale,
                     const uint16_t *q, int32_t num_q_heads, const int32_t *page_table,
                     int32_t max_pages, const int32_t *ctx_lens, int32_t batch, float sm_scale,
                     const uint8_t *abort_flags, double *out64, uint16_t *out_bf16,
                     const int32_t *rows, int32_t num_rows);

enum { B = 3, HQ = 16, HKV = 2, D = 128, PAGE = 16, NPAGES = 64, MAXP = 17 };
static const int kPrompt[B] = {37, 100, 260};

#define HIP(x)                                                                      \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));  \
      exit(2);                                                                      \
    }                                                                               \
  } while (0)
#define LIB(x)                                                                      \
  do {                                                                              \
    fp8kv_status s_ = (x);                                                          \
    if (s_ != FP8KV_OK) {                                                           \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, fp8kv_status_string(s_)); \
      exit(2);                                                                      \
    }                                                                               \
  } while (0)

/* a seeded 64-bit LCG; values roughly N(0, 1) (sum of four uniforms) */
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_state >> 11) * (1.0 / 9007199254740992.0);
}
static uint16_t bf16_bits(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float bf16_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint16_t normal_bf16(void) {
  double s = uniform01() + uniform01() + uniform01() + uniform01() - 2.0;
  return bf16_bits((float)(s * 1.7320508));
}

static void *dev_copy(const void *host, size_t bytes) {
  void *d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 1));
  if (bytes) HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(void) {
  const fp8kv_cache_desc desc = {NPAGES, PAGE, HKV, D, FP8KV_E4M3};
  const size_t pool_bytes = fp8kv_cache_bytes(&desc);

  /* pages from the pool: each request gets the pages of its prompt and new token */
  fp8kv_pool *pool = NULL;
  LIB(fp8kv_pool_create(NPAGES, 7, &pool));
  static int32_t pt[B][MAXP];
  static uint32_t et[B][MAXP];
  int32_t ctx[B], new_pos[B];
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < MAXP; ++i) pt[b][i] = -1, et[b][i] = 0;
    new_pos[b] = kPrompt[b];
    ctx[b] = kPrompt[b] + 1;
    LIB(fp8kv_pool_alloc(pool, (ctx[b] + PAGE - 1) / PAGE, pt[b], et[b]));
  }
  et[1][2] ^= 1u; /* request 1 remembers a stale tag */
  uint32_t *d_tags = NULL;
  HIP(hipMalloc((void **)&d_tags, sizeof(uint32_t) * NPAGES));
  LIB(fp8kv_pool_sync(pool, d_tags, 0));
  static uint32_t pool_tags[NPAGES];
  LIB(fp8kv_pool_read_tags(pool, pool_tags));

  /* tokens: every request's prompt and new token, K and V [t][Hkv][D]; Q [B][Hq][D] */
  int total = 0, off[B];
  for (int b = 0; b < B; ++b) off[b] = total, total += ctx[b];
  uint16_t *kb = malloc(sizeof(uint16_t) * (size_t)total * HKV * D);
  uint16_t *vb = malloc(sizeof(uint16_t) * (size_t)total * HKV * D);
  uint16_t *qb = malloc(sizeof(uint16_t) * B * HQ * D);
  for (long i = 0; i < (long)total * HKV * D; ++i) kb[i] = normal_bf16(), vb[i] = normal_bf16();
  for (int i = 0; i < B * HQ * D; ++i) qb[i] = normal_bf16();
  /* per-kv-head scales: amax / 448 over everything stored */
  float ks[HKV] = {0}, vs[HKV] = {0};
  for (long t = 0; t < total; ++t)
    for (int h = 0; h < HKV; ++h)
      for (int d = 0; d < D; ++d) {
        long i = (t * HKV + h) * D + d;
        ks[h] = fmaxf(ks[h], fabsf(bf16_float(kb[i])));
        vs[h] = fmaxf(vs[h], fabsf(bf16_float(vb[i])));
      }
  for (int h = 0; h < HKV; ++h) ks[h] /= 448.0f, vs[h] /= 448.0f;

  /* prompt tokens (bulk append) and each request's new token, in separate arrays */
  int nprompt = 0;
  for (int b = 0; b < B; ++b) nprompt += kPrompt[b];
  uint16_t *kp = malloc(sizeof(uint16_t) * (size_t)nprompt * HKV * D);
  uint16_t *vp = malloc(sizeof(uint16_t) * (size_t)nprompt * HKV * D);
  int32_t *seq = malloc(sizeof(int32_t) * nprompt), *pos = malloc(sizeof(int32_t) * nprompt);
  uint16_t kn[B * HKV * D], vn[B * HKV * D];
  for (int b = 0, j = 0; b < B; ++b) {
    for (int t = 0; t < kPrompt[b]; ++t, ++j) {
      memcpy(kp + (long)j * HKV * D, kb + (long)(off[b] + t) * HKV * D, sizeof(uint16_t) * HKV * D);
      memcpy(vp + (long)j * HKV * D, vb + (long)(off[b] + t) * HKV * D, sizeof(uint16_t) * HKV * D);
      seq[j] = b;
      pos[j] = t;
    }
    memcpy(kn + b * HKV * D, kb + (long)(off[b] + kPrompt[b]) * HKV * D, sizeof(uint16_t) * HKV * D);
    memcpy(vn + b * HKV * D, vb + (long)(off[b] + kPrompt[b]) * HKV * D, sizeof(uint16_t) * HKV * D);
  }

  /* device state */
  void *d_k = NULL, *d_v = NULL;
  HIP(hipMalloc(&d_k, pool_bytes));
  HIP(hipMalloc(&d_v, pool_bytes));
  HIP(hipMemset(d_k, 0, pool_bytes));
  HIP(hipMemset(d_v, 0, pool_bytes));
  float *d_ks = dev_copy(ks, sizeof ks), *d_vs = dev_copy(vs, sizeof vs);
  int32_t *d_pt = dev_copy(pt, sizeof pt);
  uint32_t *d_et = dev_copy(et, sizeof et);
  int32_t *d_ctx = dev_copy(ctx, sizeof ctx), *d_newpos = dev_copy(new_pos, sizeof new_pos);
  uint16_t *d_kp = dev_copy(kp, sizeof(uint16_t) * (size_t)nprompt * HKV * D);
  uint16_t *d_vp = dev_copy(vp, sizeof(uint16_t) * (size_t)nprompt * HKV * D);
  int32_t *d_seq = dev_copy(seq, sizeof(int32_t) * nprompt);
  int32_t *d_pos = dev_copy(pos, sizeof(int32_t) * nprompt);
  uint16_t *d_kn = dev_copy(kn, sizeof kn), *d_vn = dev_copy(vn, sizeof vn);
  uint16_t *d_q = dev_copy(qb, sizeof(uint16_t) * B * HQ * D);
  uint8_t *d_abort = NULL;
  float *d_out = NULL;
  HIP(hipMalloc((void **)&d_abort, B));
  HIP(hipMalloc((void **)&d_out, sizeof(float) * B * HQ * D));
  const size_t ws_bytes = fp8kv_decode_workspace_size(&desc, B, HQ, 0);
  void *d_ws = NULL;
  HIP(hipMalloc(&d_ws, ws_bytes ? ws_bytes : 1));

  /* the step */
  const float sm_scale = 1.0f / sqrtf((float)D);
  LIB(fp8kv_append(&desc, d_k, d_v, d_ks, d_vs, d_kp, d_vp, nprompt, d_seq, d_pos, B, d_pt, MAXP,
                   NULL, 0));
  LIB(fp8kv_verify_append(&desc, d_k, d_v, d_ks, d_vs, d_kn, d_vn, d_newpos, d_pt, d_et, MAXP,
                          d_ctx, B, d_tags, d_abort, 0));
  LIB(fp8kv_decode_attention(&desc, d_k, d_v, d_ks, d_vs, d_q, HQ, d_pt, MAXP, d_ctx, B, sm_scale,
                             d_abort, d_out, FP8KV_OUT_F32, 0, d_ws, ws_bytes, 0));
  HIP(hipDeviceSynchronize());
  uint8_t ab[B];
  float *out = malloc(sizeof(float) * B * HQ * D);
  uint8_t *kc = malloc(pool_bytes), *vc = malloc(pool_bytes);
  HIP(hipMemcpy(ab, d_abort, B, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(out, d_out, sizeof(float) * B * HQ * D, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(kc, d_k, pool_bytes, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(vc, d_v, pool_bytes, hipMemcpyDeviceToHost));

  /* the oracle on the same inputs: check, then prompt and new tokens, then attention */
  uint8_t ab_o[B];
  oracle_verify(&pt[0][0], &et[0][0], MAXP, ctx, B, pool_tags, NPAGES, PAGE, ab_o);
  const size_t elems = (size_t)NPAGES * HKV * PAGE * D;
  uint8_t *ko = calloc(elems, 1), *vo = calloc(elems, 1);
  int32_t nseq[B];
  for (int b = 0; b < B; ++b) nseq[b] = b;
  oracle_append(0, NPAGES, PAGE, HKV, D, ko, vo, ks, vs, kp, vp, nprompt, seq, pos, &pt[0][0], B,
                MAXP, NULL);
  oracle_append(0, NPAGES, PAGE, HKV, D, ko, vo, ks, vs, kn, vn, B, nseq, new_pos, &pt[0][0], B,
                MAXP, ab_o);
  double *ref = malloc(sizeof(double) * B * HQ * D);
  if (oracle_attention(0, NPAGES, PAGE, HKV, D, ko, vo, ks, vs, qb, HQ, &pt[0][0], MAXP, ctx, B,
                       sm_scale, ab_o, ref, NULL, NULL, 0) != 0) {
    fprintf(stderr, "oracle attention failed\n");
    return 2;
  }

  int bad = 0;
  for (int b = 0; b < B; ++b)
    if (ab[b] != ab_o[b] || ab[b] != (b == 1)) {
      fprintf(stderr, "abort flag of request %d: %d (oracle %d)\n", b, ab[b], ab_o[b]);
      bad = 1;
    }
  long compared = 0;
  for (int p = 0; p < NPAGES; ++p)
    for (int h = 0; h < HKV; ++h)
      for (int s = 0; s < PAGE; ++s)
        for (int d = 0; d < D; ++d) {
          const size_t io = (((size_t)p * HKV + h) * PAGE + s) * D + d;
          const int64_t ok_ = fp8kv_cache_offset(&desc, 0, p, h, s, d);
          const int64_t ov_ = fp8kv_cache_offset(&desc, 1, p, h, s, d);
          if (ok_ < 0 || ov_ < 0 || kc[ok_] != ko[io] || vc[ov_] != vo[io]) {
            if (bad < 8) fprintf(stderr, "cache byte (page %d, head %d, slot %d, dim %d)\n", p, h, s, d);
            bad += 1;
          }
          compared += 2;
        }
  double max_err = 0.0;
  for (int i = 0; i < B * HQ * D; ++i) {
    const double e = fabs((double)out[i] - ref[i]);
    if (e > max_err) max_err = e;
    const int b = i / (HQ * D);
    if (ab_o[b] && (out[i] != 0.0f || signbit(out[i]))) bad += 1;
  }
  if (max_err > 2e-3) bad += 1;
  printf("fp8kv C step: %s (abort %d%d%d, %ld cache bytes compared, max abs err %.3e)\n",
         bad ? "MISMATCH" : "ok", ab[0], ab[1], ab[2], compared, max_err);

  fp8kv_pool_destroy(pool);
  hipFree(d_k), hipFree(d_v), hipFree(d_ks), hipFree(d_vs), hipFree(d_pt), hipFree(d_et);
  hipFree(d_ctx), hipFree(d_newpos), hipFree(d_kp), hipFree(d_vp), hipFree(d_seq), hipFree(d_pos);
  hipFree(d_kn), hipFree(d_vn), hipFree(d_q), hipFree(d_abort), hipFree(d_out), hipFree(d_ws);
  hipFree(d_tags);
  free(kb), free(vb), free(qb), free(kp), free(vp), free(seq), free(pos), free(out), free(kc);
  free(vc), free(ko), free(vo), free(ref);
  return bad ? 1 : 0;
}
