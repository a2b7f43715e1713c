/*
 * fp8kv -- one decode step of paged attention over an FP8 (e4m3) KV cache
 * with page-tag integrity, for AMD Instinct MI355X (gfx950).
 *
 * The method (Cloudflare, "Smaller, faster, safer: running Kimi and GLM at
 * scale", KV-cache and integrity sections; restated on the commentary page in
 * "Giving Every Physical Cache Page a 'Generation Number'"):
 *   - keys and values are stored in 8-bit floating point, e4m3, instead of
 *     BF16, halving the cache; the attention kernel converts on read;
 *   - every physical cache page carries a tag that changes whenever the page
 *     is reallocated; each request records the (page, tag) pairs it expects;
 *   - before decode reads the cache, a separate batched check compares the
 *     two; a mismatch aborts that request only (fail closed), and a
 *     deployment that does not enable the check runs a no-op path.
 *
 * Conventions for every entry point below:
 *   - "d_" pointers are device pointers owned by the caller; "h_" pointers are
 *     host pointers owned by the caller.  The library keeps no pointer past a
 *     call's return, allocates no device memory in the hot-path calls and
 *     never synchronizes the stream.  Work is enqueued on `stream` in call
 *     order; errors detected on the host are returned before anything is
 *     enqueued.
 *   - Device pointers to 16-byte vectors (Q, new K/V rows, cache pools,
 *     outputs) must be 16-byte aligned.
 *   - No call throws; each returns an fp8kv_status.  A tag mismatch is data,
 *     not an error: it sets the request's abort flag.
 *   - Nothing here is thread-safe for concurrent calls on one pool object.
 *
 * Fixed shapes: page_size 16 tokens, head_dim 128.  Hq % Hkv == 0 and the
 * group size G = Hq / Hkv is at most 32.  Q-head h reads kv-head h / G.
 *
 * Cache layout.  One K pool and one V pool per layer, each
 *     [num_pages][num_kv_heads][tile]
 * where a tile holds the 16 tokens x 128 dims of one (page, kv-head):
 * 2048 bytes for e4m3, 4096 bytes for bf16.  Inside a tile the elements are
 * stored in the order the attention kernel's matrix-core fragments consume
 * them, so that each of 64 lanes reads its fragment with 16-byte loads and no
 * reshuffle.  With E = bytes per element (1 or 2), C = 16 / E elements per
 * 16-byte chunk, and the tile viewed as [2*E chunks-rows][64 lanes][16 bytes]:
 *   K element (slot s, dim d):  f = d % 32,  lane = 16*(d/32) + s
 *   V element (slot s, dim d):  f = 4*(d%8) + s%4,  lane = 16*(s/4) + d/8
 *   byte offset in tile = (f / C) * 1024 + 16 * lane + E * (f % C)
 * fp8kv_cache_offset() evaluates this formula.
 */
#ifndef FP8KV_H
#define FP8KV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fp8kv_status;
enum {
  FP8KV_OK = 0,
  FP8KV_INVALID_ARG = -1,          /* null pointer, negative size, bad id    */
  FP8KV_UNSUPPORTED = -2,          /* page_size != 16, head_dim != 128, G>32 */
  FP8KV_OUT_OF_PAGES = -3,         /* pool has fewer free pages than asked   */
  FP8KV_WORKSPACE_TOO_SMALL = -4,  /* decode workspace below the query size  */
  FP8KV_HIP_ERROR = -5             /* a HIP call failed: fp8kv_last_hip_error */
};

enum { FP8KV_E4M3 = 0, FP8KV_BF16 = 1 };          /* cache element type       */
enum { FP8KV_OUT_BF16 = 0, FP8KV_OUT_F32 = 1 };   /* attention output type    */

typedef struct {
  int32_t num_pages;     /* physical pages in each pool                        */
  int32_t page_size;     /* tokens per page; must be 16                        */
  int32_t num_kv_heads;  /* Hkv                                                */
  int32_t head_dim;      /* must be 128                                        */
  int32_t cache_dtype;   /* FP8KV_E4M3 or FP8KV_BF16                           */
} fp8kv_cache_desc;

/* Human-readable name of a status code (static string). */
const char *fp8kv_status_string(fp8kv_status status);

/* The hipError_t of the last failing HIP call made by this library on the
 * calling thread (0 if none). */
int32_t fp8kv_last_hip_error(void);

/* Bytes of ONE pool (K or V) for this descriptor; 0 if the descriptor is
 * invalid. */
size_t fp8kv_cache_bytes(const fp8kv_cache_desc *desc);

/* Byte offset of element (page, kv_head, slot, dim) inside a pool, following
 * the layout above; `is_v` selects the V order.  -1 if out of range. */
int64_t fp8kv_cache_offset(const fp8kv_cache_desc *desc, int32_t is_v, int32_t page,
                           int32_t kv_head, int32_t slot, int32_t dim);

/* ------------------------------------------------------------------------ */
/* Page pool: free list and one generation tag per physical page.            */
/* The pages' integrity scheme: a page's tag changes every time the page is  */
/* handed out again (integrity section; "Generation Number" section).  Here  */
/* the tag is a uint32 counter, seeded-random at creation and incremented    */
/* (mod 2^32) on every allocation of the page.  Pages are reused first-in    */
/* first-out.  The library owns the host object; the caller owns the device  */
/* tag array (uint32[num_pages]) that fp8kv_pool_sync keeps current.         */
/* ------------------------------------------------------------------------ */
typedef struct fp8kv_pool fp8kv_pool;

/* Create a pool of num_pages free pages (ids 0..num_pages-1).  Host only: no
 * HIP call is made.  *out receives the pool. */
fp8kv_status fp8kv_pool_create(int32_t num_pages, uint64_t seed, fp8kv_pool **out);

/* Release the pool (waits for its last pending tag upload, if any). */
void fp8kv_pool_destroy(fp8kv_pool *pool);

/* Take n pages.  On success h_page_ids[0..n) receive the ids and h_tags[0..n)
 * their new tags (the values a request must record as expected).  If fewer
 * than n pages are free nothing is taken and FP8KV_OUT_OF_PAGES is returned. */
fp8kv_status fp8kv_pool_alloc(fp8kv_pool *pool, int32_t n, int32_t *h_page_ids,
                              uint32_t *h_tags);

/* Release n pages: each listed page loses one holder, and a page without
 * holders returns to the free list.  Every id must be in range, currently
 * held and listed once; otherwise nothing changes and FP8KV_INVALID_ARG is
 * returned.  Tags are not changed on free; they change at the next allocation. */
fp8kv_status fp8kv_pool_free(fp8kv_pool *pool, int32_t n, const int32_t *h_page_ids);

/* Add one holder to each of n pages that are currently held: a request that
 * maps pages another request already holds (a shared prefix) records their
 * current tags (fp8kv_pool_tag) as its expected tags.  The tags do not change;
 * a shared page returns to the free list only when every holder has freed it.
 * Shared pages are read-only for their holders: a request writes its new
 * tokens into pages it holds alone (the library does not enforce this; an
 * append into a shared page is visible to every holder).  Every id must be in
 * range, currently held and listed once; otherwise nothing changes and
 * FP8KV_INVALID_ARG is returned.  Cache reuse across requests is what the
 * integrity section of the Cloudflare post names as the reason a bad mapping
 * reaches further. */
fp8kv_status fp8kv_pool_share(fp8kv_pool *pool, int32_t n, const int32_t *h_page_ids);

/* Number of holders of a page (0: free; -1 for an id out of range). */
int32_t fp8kv_pool_refcount(const fp8kv_pool *pool, int32_t page_id);

/* Current tag of a page (0 for an id out of range). */
uint32_t fp8kv_pool_tag(const fp8kv_pool *pool, int32_t page_id);

/* Number of free pages. */
int32_t fp8kv_pool_num_free(const fp8kv_pool *pool);

/* Copy the host tags of all num_pages pages into h_tags. */
fp8kv_status fp8kv_pool_read_tags(const fp8kv_pool *pool, uint32_t *h_tags);

/* Upload the tags changed since the last sync (all tags on the first call)
 * into d_tags with an asynchronous host-to-device copy on `stream`, so that
 * it is ordered before a later fp8kv_verify_tags on the same stream.  Uses a
 * pinned staging buffer owned by the pool; a new sync waits for the previous
 * upload to leave that buffer. */
fp8kv_status fp8kv_pool_sync(fp8kv_pool *pool, uint32_t *d_tags, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Batched page-tag check (integrity section of the Cloudflare post; the    */
/* "Generation Number" pseudocode).  A separate kernel, run before append   */
/* and attention on the same stream; never fused into attention.            */
/*   n_b = ceil(d_ctx_lens[b] / page_size)  (the pages attention will read)  */
/*   d_abort[b] = 1 iff d_ctx_lens[b] < 0, or n_b > max_pages_per_seq, or     */
/*                some i < n_b has d_page_table[b][i] outside [0, num_pages)  */
/*                or d_pool_tags[id] != d_expected_tags[b][i]; else 0.        */
/* d_page_table int32 [batch][max_pages_per_seq]; d_expected_tags uint32,    */
/* same shape; d_ctx_lens int32 [batch] (tokens the step attends over,       */
/* i.e. cached tokens + the appended one); d_pool_tags uint32 [num_pages];   */
/* d_abort uint8 [batch], written for every b.  Entries past n_b are ignored.*/
/* ------------------------------------------------------------------------ */
fp8kv_status fp8kv_verify_tags(const int32_t *d_page_table, const uint32_t *d_expected_tags,
                               int32_t max_pages_per_seq, const int32_t *d_ctx_lens,
                               int32_t batch, const uint32_t *d_pool_tags, int32_t num_pages,
                               int32_t page_size, uint8_t *d_abort, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Quantize-on-append: write new tokens' K and V into their cache pages.     */
/* (Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale",     */
/* KV-cache section: the cache holds keys and values as FP8 e4m3 instead of  */
/* BF16; integrity section: a request whose mapping failed the check must not */
/* touch the cache, so its writes are skipped too.)                          */
/* Token t of num_tokens belongs to request d_token_seq[t] (a row of the     */
/* page table, < num_seqs) at position p = d_token_pos[t]; it goes to page   */
/* d_page_table[seq][p / 16], slot p % 16.  For e4m3 every element is        */
/*     code = E( fl32( bf16(x) / scale[h] ) )                               */
/* with fl32 the correctly rounded binary32 quotient and E round-to-nearest- */
/* even onto OCP e4m3 with saturation at +-448 (sign kept, NaN -> 0x7F|sign). */
/* A BF16 cache stores the input bits unchanged (scales unused).             */
/* d_k_new / d_v_new: BF16 bits [num_tokens][Hkv][128].  d_k_scale /         */
/* d_v_scale: fp32 [Hkv] for this layer.  d_abort (nullable, uint8 [num_seqs])*/
/* skips tokens of aborted requests -- a stale mapping must not write into a */
/* page now owned by someone else.  Tokens whose request, position or page   */
/* id is out of range are skipped; nothing outside the pools is written.     */
/* Tokens are written in parallel: if several tokens of one call name the    */
/* same slot, the slot holds one of them (which one is not specified).       */
/* ------------------------------------------------------------------------ */
fp8kv_status fp8kv_append(const fp8kv_cache_desc *desc, void *d_k_cache, void *d_v_cache,
                          const float *d_k_scale, const float *d_v_scale,
                          const uint16_t *d_k_new, const uint16_t *d_v_new, int32_t num_tokens,
                          const int32_t *d_token_seq, const int32_t *d_token_pos,
                          int32_t num_seqs, const int32_t *d_page_table,
                          int32_t max_pages_per_seq, const uint8_t *d_abort,
                          hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Tag check fused with the step's append (same two operations as            */
/* fp8kv_verify_tags followed by fp8kv_append gated on d_abort, in one        */
/* launch).  One workgroup per request b: it checks the request's pages as    */
/* fp8kv_verify_tags does, writes d_abort[b], and only if the check passed    */
/* quantizes the request's new token (d_k_new/d_v_new row b, BF16             */
/* [batch][Hkv][128]) into position d_new_pos[b].  The check is still its    */
/* own batched pass ahead of attention, as the integrity section describes.  */
/* Fail closed: the new token must lie inside the context that was checked   */
/* (0 <= d_new_pos[b] < d_ctx_lens[b]), so that every page written is one    */
/* whose tag was compared; otherwise the request is aborted (d_abort[b] = 1) */
/* and nothing is written.  Page counts are computed in 64 bits: a length    */
/* near INT32_MAX aborts (its pages do not fit the table) instead of         */
/* wrapping.  Hkv <= 16 (one workgroup encodes the whole token).             */
/* ------------------------------------------------------------------------ */
fp8kv_status fp8kv_verify_append(const fp8kv_cache_desc *desc, void *d_k_cache, void *d_v_cache,
                                 const float *d_k_scale, const float *d_v_scale,
                                 const uint16_t *d_k_new, const uint16_t *d_v_new,
                                 const int32_t *d_new_pos, const int32_t *d_page_table,
                                 const uint32_t *d_expected_tags, int32_t max_pages_per_seq,
                                 const int32_t *d_ctx_lens, int32_t batch,
                                 const uint32_t *d_pool_tags, uint8_t *d_abort,
                                 hipStream_t stream);

/* The same with q_len new tokens per request (several tokens checked in one  */
/* step, speculative decoding): d_k_new/d_v_new BF16 [batch][q_len][Hkv][128], */
/* token i of request b goes to position d_new_pos[b] + i, all only if the    */
/* request's check passed and all q_len positions lie inside the checked     */
/* context (d_new_pos[b] >= 0 and d_new_pos[b] + q_len <= d_ctx_lens[b]; else  */
/* the request aborts and writes nothing).  q_len = 1 is fp8kv_verify_append. */
/* Errors as above, and FP8KV_INVALID_ARG for q_len < 1.                      */
fp8kv_status fp8kv_verify_append_q(const fp8kv_cache_desc *desc, void *d_k_cache,
                                   void *d_v_cache, const float *d_k_scale,
                                   const float *d_v_scale, const uint16_t *d_k_new,
                                   const uint16_t *d_v_new, const int32_t *d_new_pos,
                                   int32_t q_len, const int32_t *d_page_table,
                                   const uint32_t *d_expected_tags, int32_t max_pages_per_seq,
                                   const int32_t *d_ctx_lens, int32_t batch,
                                   const uint32_t *d_pool_tags, uint8_t *d_abort,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Paged decode attention (one query token per request) over the cache,      */
/* converting e4m3 on read (Cloudflare, "Smaller, faster, safer: running Kimi */
/* and GLM at scale", KV-cache section: the attention kernel turns the stored */
/* FP8 values back into wider numbers as it loads them; integrity section: a  */
/* request flagged by the check reads nothing and produces no output; the    */
/* check is a separate pass and a deployment without it runs a no-op tracker, */
/* here a NULL d_abort).  The formula itself is not on the pages: it is      */
/* textbook single-query scaled dot-product attention with grouped kv-heads. */
/* For request b and q-head h (kv-head g = h/G):                             */
/*   s_j = sm_scale * k_scale[g] * sum_d q[b][h][d] * DEC(K[j][g][d]),        */
/*   o   = v_scale[g] * sum_j e^{s_j - max s} DEC(V[j][g]) / sum_j e^{s_j-max s}*/
/* over the d_ctx_lens[b] tokens j of the request (token j at page           */
/* d_page_table[b][j/16], slot j%16).  The (request, kv-head, page) work is   */
/* shared equally by num_workers/4 workgroups of 4 waves; a (request,         */
/* kv-head) whose pages fall to several workgroups is finished by a          */
/* log-sum-exp merge of their partial (max, sum, weighted V) in workgroup    */
/* order (flash-decoding split-K) in a second short kernel, so the result    */
/* is deterministic for a given batch and num_workers.                       */
/*   d_q: BF16 bits [batch][Hq][128];  d_out: [batch][Hq][128] of BF16 bits   */
/*   (out_dtype FP8KV_OUT_BF16, round-to-nearest-even) or fp32 (FP8KV_OUT_F32).*/
/*   d_abort (nullable): requests flagged 1 produce +0 rows and read nothing  */
/*   from the cache; NULL is the no-op tracker (no check at all).  Requests   */
/*   with d_ctx_lens[b] <= 0 or more pages than max_pages_per_seq also give   */
/*   +0 rows.  Without the check, page ids outside [0, num_pages) are still   */
/*   never dereferenced; their tokens are left out (results for such a        */
/*   request are unspecified).                                                */
/*   batch <= 4096 and batch * (max_pages_per_seq + 16) < 2^31 (the work      */
/*   split counts pages in 32 bits), else FP8KV_UNSUPPORTED (every decode      */
/*   entry point).  num_workers: 0 picks the device's resident wave count     */
/*   (compute units x 12); otherwise rounded up to a multiple of 4.           */
/*   d_workspace: at least fp8kv_decode_workspace_size() bytes for the same   */
/*   batch, num_q_heads and num_workers on the current device.  Calls that    */
/*   share a workspace must not overlap.                                      */
/* ------------------------------------------------------------------------ */
int32_t fp8kv_decode_num_workers(int32_t requested);

size_t fp8kv_decode_workspace_size(const fp8kv_cache_desc *desc, int32_t batch,
                                   int32_t num_q_heads, int32_t num_workers);

fp8kv_status fp8kv_decode_attention(const fp8kv_cache_desc *desc, const void *d_k_cache,
                                    const void *d_v_cache, const float *d_k_scale,
                                    const float *d_v_scale, const uint16_t *d_q,
                                    int32_t num_q_heads, const int32_t *d_page_table,
                                    int32_t max_pages_per_seq, const int32_t *d_ctx_lens,
                                    int32_t batch, float sm_scale, const uint8_t *d_abort,
                                    void *d_out, int32_t out_dtype, int32_t num_workers,
                                    void *d_workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* fp8kv_decode_attention without a workspace argument, for callers that      */
/* cannot allocate device memory (code under HIP graph capture, tight serving */
/* loops, harnesses that forbid hipMalloc).  Same arguments, results and      */
/* errors as fp8kv_decode_attention with the same num_workers (bit for bit),  */
/* except that the partial states live in a fixed device array of the        */
/* library: FP8KV_NOALLOC_SCRATCH_BYTES bytes on every device the library    */
/* runs on, held until the process ends.  A call whose workspace              */
/* (fp8kv_decode_workspace_size for the same batch, num_q_heads and          */
/* num_workers) exceeds it returns FP8KV_WORKSPACE_TOO_SMALL before anything  */
/* is enqueued: 32 MiB covers, at 64 q-heads over 8 kv-heads and the default */
/* worker count of a 256-CU device, batches up to about 900 requests.  The   */
/* call allocates nothing (no hipMalloc, hipFree or allocating library call); */
/* the first call on a device looks up the array's address for that device. */
/* The array's contents before a call do not matter (nothing needs to start  */
/* at zero).  Every call on one device shares that device's array: calls     */
/* that may overlap on one GPU (several streams, several host threads) race  */
/* and must be ordered by the caller.                                         */
/* ------------------------------------------------------------------------ */
#define FP8KV_NOALLOC_SCRATCH_BYTES (32u << 20)

fp8kv_status fp8kv_decode_attention_noalloc(const fp8kv_cache_desc *desc, const void *d_k_cache,
                                            const void *d_v_cache, const float *d_k_scale,
                                            const float *d_v_scale, const uint16_t *d_q,
                                            int32_t num_q_heads, const int32_t *d_page_table,
                                            int32_t max_pages_per_seq, const int32_t *d_ctx_lens,
                                            int32_t batch, float sm_scale, const uint8_t *d_abort,
                                            void *d_out, int32_t out_dtype, int32_t num_workers,
                                            hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Several new tokens per request checked in one step: speculative decoding, */
/* where a draft proposes tokens and the main model verifies them together   */
/* (page "Kimi and GLM Reasoning Slimming: Hands-On Test", section "It       */
/* Follows the Same Path as Cloudflare's Earlier Infire Optimizations").     */
/* Same as fp8kv_decode_attention with q_len queries per request:            */
/*   d_q: BF16 bits [batch][q_len][Hq][128]; d_out: [batch][q_len][Hq][128]. */
/*   d_ctx_lens[b] counts the request's tokens after all q_len new ones were */
/*   appended (fp8kv_append with q_len tokens per request); query i stands   */
/*   for the new token at position ctx-q_len+i and attends tokens            */
/*   0..ctx-q_len+i (causal among the new tokens; a query with no token to   */
/*   see gives +0).  (Hq / Hkv) * q_len <= 32: the (query, head) pairs of a  */
/*   kv-head share one or two 16-wide MFMA tiles, so checking q_len tokens   */
/*   reads the cache once.  Above 16 pairs the kernel runs 2 waves per SIMD  */
/*   instead of 3.  q_len = 1 is fp8kv_decode_attention.  Larger products    */
/*   return FP8KV_UNSUPPORTED and fp8kv_decode_workspace_size_q() 0.         */
/*   d_workspace: at least fp8kv_decode_workspace_size_q() bytes.             */
/* ------------------------------------------------------------------------ */
size_t fp8kv_decode_workspace_size_q(const fp8kv_cache_desc *desc, int32_t batch,
                                     int32_t num_q_heads, int32_t q_len, int32_t num_workers);

fp8kv_status fp8kv_decode_attention_q(const fp8kv_cache_desc *desc, const void *d_k_cache,
                                      const void *d_v_cache, const float *d_k_scale,
                                      const float *d_v_scale, const uint16_t *d_q,
                                      int32_t num_q_heads, int32_t q_len,
                                      const int32_t *d_page_table, int32_t max_pages_per_seq,
                                      const int32_t *d_ctx_lens, int32_t batch, float sm_scale,
                                      const uint8_t *d_abort, void *d_out, int32_t out_dtype,
                                      int32_t num_workers, void *d_workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Prompts shared by groups of requests: prefix caching, where requests      */
/* continuing the same prompt map the same cache pages (page "Kimi and GLM   */
/* Reasoning Slimming: Hands-On Test", section "It Follows the Same Path as  */
/* Cloudflare's Earlier Infire Optimizations").  Same result as              */
/* fp8kv_decode_attention (one new token per request), computed so that     */
/* each of a prompt's pages is read once per kv-head for its whole group:    */
/* the group's (request, q-head) pairs form the MFMA columns over those      */
/* pages, each request's own tokens are attended as usual, and the two parts */
/* are joined by their log-sum-exp.                                          */
/*   num_groups <= 32; h_group_start: host int32 [num_groups+1], group k =   */
/*   requests [h_group_start[k], h_group_start[k+1]) (non-decreasing, within  */
/*   the batch; requests outside every group have no shared prompt);         */
/*   h_prefix_len: host int32 [num_groups], tokens of group k's prompt, a     */
/*   multiple of 16, at most 16*max_pages_per_seq (0: no shared prompt).      */
/*   Every request of group k lists the prompt's prefix_len/16 pages first in */
/*   its table; they are read from the table of the group's first request.   */
/*   The tag check reads each request's own table, so the call fails closed: */
/*   a member whose first prefix_len/16 entries differ from the first        */
/*   request's gets +0 rows (whatever its abort flag), and each member's rows */
/*   depend only on its own flag (an aborted first request does not affect   */
/*   the others).  Rows of requests whose context does not extend past their  */
/*   prompt (ctx <= prefix_len), of aborted requests and of contexts the table */
/*   cannot hold are +0 too.  The host arrays are read during the call only.  */
/*   d_workspace: at least fp8kv_decode_workspace_size_shared() bytes (same  */
/*   groups; 0 for invalid arguments).  Errors as fp8kv_decode_attention,     */
/*   and FP8KV_INVALID_ARG for a bad group description.                      */
/* ------------------------------------------------------------------------ */
size_t fp8kv_decode_workspace_size_shared(const fp8kv_cache_desc *desc, int32_t batch,
                                          int32_t num_q_heads, int32_t max_pages_per_seq,
                                          int32_t num_groups, const int32_t *h_group_start,
                                          const int32_t *h_prefix_len, int32_t num_workers);

fp8kv_status fp8kv_decode_attention_shared(
    const fp8kv_cache_desc *desc, const void *d_k_cache, const void *d_v_cache,
    const float *d_k_scale, const float *d_v_scale, const uint16_t *d_q, int32_t num_q_heads,
    int32_t num_groups, const int32_t *h_group_start, const int32_t *h_prefix_len,
    const int32_t *d_page_table, int32_t max_pages_per_seq, const int32_t *d_ctx_lens,
    int32_t batch, float sm_scale, const uint8_t *d_abort, void *d_out, int32_t out_dtype,
    int32_t num_workers, void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Measurement reference: reads every byte of d_buf (bytes a multiple of 16, */
/* 16-byte aligned) once, with the attention kernel's tile loads (16-byte    */
/* buffer loads, same cache policy, 4 KiB per wave at a time) but in order   */
/* and with no page indirection, and writes an XOR of what it read to d_sink */
/* (uint32, fp8kv_debug_read_sink_words() of them).                           */
/* Timing it gives the streaming-read rate the attention kernel is compared  */
/* with.  FP8KV_INVALID_ARG for null pointers or a size not a multiple of 16. */
/* ------------------------------------------------------------------------ */
int32_t fp8kv_debug_read_sink_words(void);

fp8kv_status fp8kv_debug_read_bandwidth(const void *d_buf, size_t bytes, uint32_t *d_sink,
                                        hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Self-test of the on-read conversion: d_out[i] = the value the attention   */
/* kernel's e4m3 -> bf16 (which = 0) or e4m3 -> f16 (which = 1) conversion   */
/* gives for code d_codes[i], widened to fp32.  n a multiple of 4.           */
/* ------------------------------------------------------------------------ */
fp8kv_status fp8kv_debug_convert_e4m3(const uint8_t *d_codes, float *d_out, int32_t n,
                                      int32_t which, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8KV_H */
