// fp8kv: HIP kernels for gfx950 (MI355X) and their C-ABI launchers.
//
// One decode step over an FP8 e4m3 paged KV cache with page-tag integrity
// (Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale":
// KV-cache section -- e4m3 storage converted on read; integrity section --
// per-page generation tags checked by a separate batch pass before decode,
// mismatching requests aborted).
//
// Kernels:
//   verify_tags_kernel      one workgroup per request: any stale/out-of-range
//                           page among the pages the step reads -> abort[b]=1
//   verify_append_kernel<C> the same check and the request's new token
//                           appended in one launch (append skipped on abort)
//   append_kernel<C>        quantize-on-append of any number of tokens
//   decode_kernel<C, D, NT> persistent workgroups, each an equal slice of the
//                           (request, kv-head, page) list: paged K/V tiles are
//                           loaded straight into matrix-core fragment registers
//                           (16-byte buffer loads, tile layout = fragment
//                           order), converted e4m3 -> bf16/f16 in hardware,
//                           QK^T and PV on MFMA, online softmax in registers,
//                           4 waves merged through LDS; writes the output, or a
//                           (max, sum, weighted V) partial for a split segment
//   merge_flat_kernel,      log-sum-exp merge of the partials in workgroup
//   merge_grouped_kernel    order (few pieces per segment / many)
//   prefix_kernel<C, NT>    prompts shared by groups of requests: each one's
//                           pages read once per kv-head with the group's
//                           (request, q-head) pairs as MFMA columns
//   shared_fused_kernel<NT> that prompt pass and the decode of the requests'
//                           own tokens in one grid (e4m3, up to 16 columns)
//   view_kernel             each request's table and context past its prompt
//                           (the separate-launch form)
//   combine_kernel          the prompt's partials and the own-token rows joined
//                           by log-sum-exp (after the fused grid it also merges
//                           the own-token decode's split segments)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cfloat>
#include <type_traits>

#include "fp8kv.h"
#include "fp8kv_internal.h"

// Device memory of fp8kv_decode_attention_noalloc: the decode's partial
// states and prefix sums for callers that cannot allocate (graph capture,
// serving loops).  One copy per device, held until the process ends; host
// code never passes this name to a kernel (on the host it is only a stand-in
// for the symbol): it uses the address hipGetSymbolAddress gives per device.
static __device__ __align__(256) unsigned char scratch[FP8KV_NOALLOC_SCRATCH_BYTES];

namespace fp8kv_detail {
thread_local int32_t g_last_hip_error = 0;
void record_hip_error(int32_t e) { g_last_hip_error = e; }
}  // namespace fp8kv_detail

namespace {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// (query, head) columns of one kv-head: one or two 16-column MFMA tiles
constexpr int kTileCols = 16;
constexpr int kMaxGroup = 2 * kTileCols;
// word 3 of a raw buffer resource on gfx9-family parts (32-bit data, no
// swizzle, no index stride)
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the K/V tile loads: nt (streaming).  Each tile is read
// once per step, so keeping it out of the normal replacement order costs no
// reuse; measured on gfx950, random 2 KB reads with nt run ~13% faster than
// with the default policy.  (Pages shared by many requests are re-read; the
// shared-prompt call reads those with the default policy, once per batch.)
constexpr int kKvLoadPolicy = 2;
constexpr float kLog2e = 1.4426950408889634f;
// log2 of the largest softmax weight the attention loops let build up before
// they move their reference max (weights and sums stay far from f16/f32
// overflow; most steps then leave the accumulators alone)
constexpr float kLazyRescale = 8.0f;

// pages in flight per wave (register ring depth), per cache type
#ifndef FP8KV_DEPTH_E4M3
#define FP8KV_DEPTH_E4M3 2
#endif
#ifndef FP8KV_DEPTH_BF16
#define FP8KV_DEPTH_BF16 1
#endif
// the same with two column tiles (2 waves per SIMD, more registers per wave)
#ifndef FP8KV_DEPTH_E4M3_2T
#define FP8KV_DEPTH_E4M3_2T 2
#endif
#ifndef FP8KV_DEPTH_BF16_2T
#define FP8KV_DEPTH_BF16_2T 2
#endif
// waves per compute unit the automatic worker count aims for
#ifndef FP8KV_WAVES_PER_CU
#define FP8KV_WAVES_PER_CU 12
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <int CACHE>
struct Tile;
template <>
struct Tile<FP8KV_E4M3> {
  static constexpr int kBytes = 2048;  // 16 tokens x 128 dims x 1 byte
  static constexpr int kChunks = 2;    // 16-byte loads per lane per tile
};
template <>
struct Tile<FP8KV_BF16> {
  static constexpr int kBytes = 4096;
  static constexpr int kChunks = 4;
};

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------

// 8 e4m3 codes (two dwords, byte i -> element i) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(unsigned w0, unsigned w1) {
  u32x4_t r;
  r.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, r);
}

// 4 e4m3 codes (one dword) -> 4 f16, exact.
__device__ __forceinline__ f16x4_t e4m3x4_to_f16(unsigned w) {
  u32x2_t r;
  r.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  return __builtin_bit_cast(f16x4_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<unsigned>(b) << 16);
}

// binary32 -> OCP e4m3, round to nearest even, saturating at +-448, sign
// kept, NaN -> 0x7F|sign.  Bit-level: the normal range keeps 3 mantissa bits
// and rounds the 20 dropped bits half-to-even; below 2^-6 the codes are the
// multiples of 2^-9, so |x|*512 rounded half-to-even is the code.
__device__ __forceinline__ unsigned e4m3_encode(float x) {
  const unsigned u = __float_as_uint(x);
  const unsigned sign = (u >> 24) & 0x80u;
  const unsigned a = u & 0x7FFFFFFFu;
  unsigned code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;
  } else if (a >= 0x43E00000u) {  // |x| >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {   // |x| < 2^-6
    code = static_cast<unsigned>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  } else {
    const unsigned r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return code | sign;
}

// The max over the four lanes l, l^16, l^32, l^48 (they hold the same MFMA
// column), through the row-swap instructions (no LDS round trip).  The IEEE
// maximum builtin (v_maximum3_f32) would skip the canonicalising v_max of each
// operand, but gave results that varied from call to call on identical inputs
// here: fmaxf it is.
__device__ __forceinline__ float wave_max_rows_swap(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 1. page-tag check
// ---------------------------------------------------------------------------
struct VerifyArgs {
  const int32_t* page_table;
  const uint32_t* expected;
  const int32_t* ctx_lens;
  const uint32_t* tags;
  uint8_t* abort;
  int32_t max_pages, num_pages, page_size;
};

// One workgroup per request; each thread takes kVerifyUnroll entries per round
// and issues all of their loads (page ids and expected tags, then the current
// tags) before comparing any, so a round costs two dependent load latencies.
constexpr int kVerifyThreads = 512;
constexpr int kVerifyUnroll = 4;

// Entries i0 + u*kVerifyThreads (u < kVerifyUnroll) of a request's list of n:
// nonzero if one of them names a page outside the pool or a stale tag.
__device__ __forceinline__ int check_round(const VerifyArgs& a, const int32_t* pt,
                                           const uint32_t* et, int n, int i0) {
  int32_t id[kVerifyUnroll];
  uint32_t ex[kVerifyUnroll], cur[kVerifyUnroll];
#pragma unroll
  for (int u = 0; u < kVerifyUnroll; ++u) {
    const int i = i0 + u * kVerifyThreads;
    id[u] = i < n ? pt[i] : 0;
    ex[u] = i < n ? et[i] : 0;
  }
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kVerifyUnroll; ++u) {
    const int i = i0 + u * kVerifyThreads;
    const bool valid = static_cast<unsigned>(id[u]) < static_cast<unsigned>(a.num_pages);
    cur[u] = (i < n && valid) ? a.tags[id[u]] : 0u;
    if (i < n && !valid) bad = 1;
  }
#pragma unroll
  for (int u = 0; u < kVerifyUnroll; ++u) {
    const int i = i0 + u * kVerifyThreads;
    if (i < n && cur[u] != ex[u]) bad = 1;
  }
  return bad;
}

// pages of a context of ctx tokens (64-bit: a length near INT32_MAX must not
// wrap to a small count and pass)
__device__ __forceinline__ int64_t pages_of(int ctx, int page_size) {
  return ctx < 0 ? 0 : (static_cast<int64_t>(ctx) + page_size - 1) / page_size;
}

__global__ __launch_bounds__(kVerifyThreads) void verify_tags_kernel(VerifyArgs a) {
  const int b = blockIdx.x;
  const int ctx = a.ctx_lens[b];
  const int64_t n = pages_of(ctx, a.page_size);
  int bad = (ctx < 0 || n > a.max_pages) ? 1 : 0;
  const int nchk = bad ? 0 : static_cast<int>(n);
  const int32_t* pt = a.page_table + static_cast<int64_t>(b) * a.max_pages;
  const uint32_t* et = a.expected + static_cast<int64_t>(b) * a.max_pages;
  for (int i0 = threadIdx.x; i0 < nchk; i0 += kVerifyUnroll * kVerifyThreads)
    bad |= check_round(a, pt, et, nchk, i0);
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) a.abort[b] = static_cast<uint8_t>(bad ? 1 : 0);
}

// ---------------------------------------------------------------------------
// 2. quantize-on-append
// ---------------------------------------------------------------------------
struct AppendArgs {
  uint8_t* k_cache;
  uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* token_seq;
  const int32_t* token_pos;
  const int32_t* page_table;
  const uint8_t* abort;
  int64_t page_stride;  // bytes per physical page in one pool
  int64_t total_items;  // num_tokens * Hkv * 32
  int32_t num_seqs, max_pages, num_pages, Hkv;
};

// Quantized (or copied) bytes of dims [4c, 4c+4) of one token and kv-head:
// one 32-bit K store (e4m3) or 64-bit (bf16), V scattered per element (its
// layout puts consecutive dims in different lanes).  Four dims per thread
// spreads a token's 2*Hkv*128 correctly rounded divisions over 32*Hkv lanes.
struct Chunk4 {
  u32x2_t k, v;  // e4m3: k.x / v.x hold 4 codes; bf16: the raw 8 bytes
};

// ks, vs: the kv-head's scales (unused for a bf16 cache)
template <int CACHE>
__device__ __forceinline__ Chunk4 append_encode4(u32x2_t k, u32x2_t v, float ks, float vs) {
  Chunk4 r;
  r.k = k;
  r.v = v;
  if constexpr (CACHE == FP8KV_E4M3) {
    unsigned kq = 0u, vq = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t kb = (i & 1) ? (k[i >> 1] >> 16) : (k[i >> 1] & 0xFFFF);
      const uint16_t vb = (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFF);
      kq |= e4m3_encode(bf16_to_f32(kb) / ks) << (8 * i);
      vq |= e4m3_encode(bf16_to_f32(vb) / vs) << (8 * i);
    }
    r.k.x = kq;
    r.v.x = vq;
  }
  return r;
}

template <int CACHE>
__device__ __forceinline__ void append_store4(const AppendArgs& a, const Chunk4& r, int h, int c,
                                              int32_t pid, int slot) {
  const int64_t tile = static_cast<int64_t>(pid) * a.page_stride +
                       static_cast<int64_t>(h) * Tile<CACHE>::kBytes;
  uint8_t* kt = a.k_cache + tile;
  uint8_t* vt = a.v_cache + tile;
  const int d0 = 4 * c;
  const int f0 = d0 & 31;
  const int klane = 16 * (d0 >> 5) + slot;
  if constexpr (CACHE == FP8KV_E4M3) {
    *reinterpret_cast<unsigned*>(kt + (f0 >> 4) * 1024 + 16 * klane + (f0 & 15)) = r.k.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = d0 + i;
      const int f = 4 * (d & 7) + (slot & 3);
      const int vlane = 16 * (slot >> 2) + (d >> 3);
      vt[(f >> 4) * 1024 + 16 * vlane + (f & 15)] = static_cast<uint8_t>(r.v.x >> (8 * i));
    }
  } else {
    *reinterpret_cast<u32x2_t*>(kt + (f0 >> 3) * 1024 + 16 * klane + 2 * (f0 & 7)) = r.k;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = d0 + i;
      const int f = 4 * (d & 7) + (slot & 3);
      const int vlane = 16 * (slot >> 2) + (d >> 3);
      *reinterpret_cast<uint16_t*>(vt + (f >> 3) * 1024 + 16 * vlane + 2 * (f & 7)) =
          static_cast<uint16_t>((i & 1) ? (r.v[i >> 1] >> 16) : (r.v[i >> 1] & 0xFFFF));
    }
  }
}

// One (token, kv-head, 4-dim chunk) item.  The new values and the token's
// request and position are loaded together, then the request's abort flag and
// page id together; the encode runs while those are in flight, so an item
// waits for two load latencies before its store.
template <int CACHE>
__device__ __forceinline__ void append_item(const AppendArgs& a, int64_t item) {
  const int c = static_cast<int>(item & 31);
  const int64_t th = item >> 5;
  const int h = static_cast<int>(th % a.Hkv);
  const int64_t tok = th / a.Hkv;
  const int64_t src = (tok * a.Hkv + h) * kHeadDim + 4 * c;
  // level 1: everything indexed by the item alone
  const u32x2_t kin = *reinterpret_cast<const u32x2_t*>(a.k_new + src);
  const u32x2_t vin = *reinterpret_cast<const u32x2_t*>(a.v_new + src);
  const int seq = a.token_seq[tok];
  const int pos = a.token_pos[tok];
  float ks = 1.0f, vs = 1.0f;
  if constexpr (CACHE == FP8KV_E4M3) {
    ks = a.k_scale[h];
    vs = a.v_scale[h];
  }
  // level 2: indexed by the request (clamped, so the loads need no branch)
  const bool ok = seq >= 0 && seq < a.num_seqs && pos >= 0 && pos / kPage < a.max_pages;
  const int sq = ok ? seq : 0;
  const int pg = ok ? pos / kPage : 0;
  const int32_t pid = a.page_table[static_cast<int64_t>(sq) * a.max_pages + pg];
  // without an abort array the load reads a byte of the token's request id
  // (valid memory) and the value is ignored: no branch around the load
  const uint8_t flag =
      *(a.abort ? a.abort + sq : reinterpret_cast<const uint8_t*>(a.token_seq + tok));
  const bool aborted = a.abort != nullptr && flag != 0;
  const Chunk4 r = append_encode4<CACHE>(kin, vin, ks, vs);
  if (!ok || aborted || static_cast<unsigned>(pid) >= static_cast<unsigned>(a.num_pages)) return;
  append_store4<CACHE>(a, r, h, c, pid, pos % kPage);
}

// A grid-stride loop: a bulk fill of any size fits the 32-bit grid (up to
// 2^30 items, 4M tokens at 8 kv-heads, every thread takes one item; a loop
// over fewer threads measured 15% slower on a 1M-token fill).
constexpr int64_t kAppendMaxBlocks = 1 << 22;
template <int CACHE>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t item = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
       item < a.total_items; item += stride)
    append_item<CACHE>(a, item);
}

// ---------------------------------------------------------------------------
// 3. tag check fused with the step's append (one workgroup per request)
// ---------------------------------------------------------------------------
struct VerifyAppendArgs {
  VerifyArgs v;
  AppendArgs w;
  const int32_t* new_pos;  // position of each request's first new token
  int32_t qlen;            // new tokens per request (k_new: [B][qlen][Hkv][128])
};

// The check still runs as its own batched pass ahead of attention; fusing it
// with the append only removes a launch: a request's token is written after
// (and only if) all of that request's pages passed.  The token is loaded and
// encoded while the check's loads are in flight; only the stores wait.

template <int CACHE>
__global__ __launch_bounds__(kVerifyThreads) void verify_append_kernel(VerifyAppendArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int ctx = a.v.ctx_lens[b];
  const int pos0 = a.new_pos[b];
  // items: (new token, kv-head, 4 dims); a thread takes items tid, tid + 512, ..
  const int per_tok = a.w.Hkv * (kHeadDim / 4);
  const int items = a.qlen * per_tok;
  const int tok = tid / per_tok;  // of the first item
  const int pos = pos0 + tok;
  const int64_t n = pages_of(ctx, a.v.page_size);
  // Fail closed: the new tokens (positions pos0 .. pos0+qlen-1) must lie inside
  // the context the check covers, so every page written is a page checked;
  // otherwise the request aborts and nothing is written.
  const bool inside = pos0 >= 0 && static_cast<int64_t>(pos0) + a.qlen <= ctx;
  int bad = (ctx < 0 || n > a.v.max_pages || !inside) ? 1 : 0;
  const bool pos_ok = !bad;  // then pos / 16 < n <= max_pages
  const int nchk = bad ? 0 : static_cast<int>(n);
  const int32_t* pt = a.v.page_table + static_cast<int64_t>(b) * a.v.max_pages;
  const uint32_t* et = a.v.expected + static_cast<int64_t>(b) * a.v.max_pages;
  // 1. the first round of the check's loads: page ids and expected tags
  int32_t id[kVerifyUnroll];
  uint32_t ex[kVerifyUnroll];
#pragma unroll
  for (int u = 0; u < kVerifyUnroll; ++u) {
    const int i = tid + u * kVerifyThreads;
    id[u] = i < nchk ? pt[i] : 0;
    ex[u] = i < nchk ? et[i] : 0;
  }
  // 2. this thread's share of the append (4 dims of one kv-head): the token's
  //    inputs and its page id
  const bool mine = tid < items;
  const int h = (tid - tok * per_tok) >> 5, c = tid & 31;
  const int64_t src =
      ((static_cast<int64_t>(b) * a.qlen + tok) * a.w.Hkv + h) * kHeadDim + 4 * c;
  u32x2_t kin = {0u, 0u}, vin = {0u, 0u};
  int32_t pid = -1;
  if (mine && pos_ok) {
    pid = a.w.page_table[static_cast<int64_t>(b) * a.w.max_pages + pos / kPage];
    kin = *reinterpret_cast<const u32x2_t*>(a.w.k_new + src);
    vin = *reinterpret_cast<const u32x2_t*>(a.w.v_new + src);
  }
  // 3. current tags of the listed pages
  uint32_t cur[kVerifyUnroll];
#pragma unroll
  for (int u = 0; u < kVerifyUnroll; ++u) {
    const int i = tid + u * kVerifyThreads;
    const bool valid = static_cast<unsigned>(id[u]) < static_cast<unsigned>(a.v.num_pages);
    cur[u] = (i < nchk && valid) ? a.v.tags[id[u]] : 0u;
    if (i < nchk && (!valid)) bad = 1;
  }
  // 4. encode while the tag loads are in flight
  Chunk4 prep;
  if (mine && pos_ok)
    prep = append_encode4<CACHE>(kin, vin, CACHE == FP8KV_E4M3 ? a.w.k_scale[h] : 1.0f,
                                 CACHE == FP8KV_E4M3 ? a.w.v_scale[h] : 1.0f);
  // 5. compare; requests longer than one round continue in a loop
#pragma unroll
  for (int u = 0; u < kVerifyUnroll; ++u) {
    const int i = tid + u * kVerifyThreads;
    if (i < nchk && cur[u] != ex[u]) bad = 1;
  }
  for (int i0 = tid + kVerifyUnroll * kVerifyThreads; i0 < nchk;
       i0 += kVerifyUnroll * kVerifyThreads)
    bad |= check_round(a.v, pt, et, nchk, i0);
  bad = __syncthreads_or(bad);
  if (tid == 0) a.v.abort[b] = static_cast<uint8_t>(bad ? 1 : 0);
  if (bad) return;
  if (mine && pos_ok && static_cast<unsigned>(pid) < static_cast<unsigned>(a.w.num_pages))
    append_store4<CACHE>(a.w, prep, h, c, pid, pos % kPage);
  // more new tokens than one pass of the workgroup: the rest after the check
  for (int it = tid + kVerifyThreads; it < items; it += kVerifyThreads) {
    const int t = it / per_tok;
    const int hh = (it - t * per_tok) >> 5, cc = it & 31;
    const int p = pos0 + t;
    if (pos0 < 0 || p / kPage >= a.w.max_pages) continue;
    const int32_t pg = a.w.page_table[static_cast<int64_t>(b) * a.w.max_pages + p / kPage];
    if (static_cast<unsigned>(pg) >= static_cast<unsigned>(a.w.num_pages)) continue;
    const int64_t sx = ((static_cast<int64_t>(b) * a.qlen + t) * a.w.Hkv + hh) * kHeadDim + 4 * cc;
    const Chunk4 q = append_encode4<CACHE>(*reinterpret_cast<const u32x2_t*>(a.w.k_new + sx),
                                           *reinterpret_cast<const u32x2_t*>(a.w.v_new + sx),
                                           CACHE == FP8KV_E4M3 ? a.w.k_scale[hh] : 1.0f,
                                           CACHE == FP8KV_E4M3 ? a.w.v_scale[hh] : 1.0f);
    append_store4<CACHE>(a.w, q, hh, cc, pg, p % kPage);
  }
}

// ---------------------------------------------------------------------------
// 4. decode: persistent workgroups, equal work per workgroup
// ---------------------------------------------------------------------------
// Work list: for every live request b (in order) and kv-head g, a segment of
// kPieceItems items that read nothing (a piece's fixed cost) and then the n_b
// pages the step reads: W = Hkv * sum_b (kPieceItems + n_b) items (one page
// item = 16 tokens of one kv-head: 2 KiB of K + 2 KiB of V for e4m3).
// Workgroup w of NWG takes items [w*W/NWG, (w+1)*W/NWG), so every workgroup
// gets the same cost however ragged the lengths.  Its slice is cut at (request, kv-head)
// boundaries into pieces; inside a piece the 4 waves take pages round robin,
// each with its own online softmax, and are merged through LDS at the end of
// the piece.  A piece that is a whole segment writes the output; any other
// piece leaves (max, sum, weighted V) in slot  w + segment  (unique per
// (workgroup, segment) pair) for the merge pass.
//
// Each wave walks its own padded sequence of pages (per piece, its pages
// rounded up to a multiple of DEPTH with masked dummies), so the register
// ring slot of every page is known at compile time; loads run DEPTH pages
// ahead and page ids 2*DEPTH pages ahead, across piece boundaries.
struct DecodeArgs {
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const uint16_t* q;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  const uint8_t* abort;
  void* out;
  float* ws_o;     // [slots][C][128] unnormalised weighted V
  float* ws_ml;    // [slots][C][2]   (max in log2 units, sum)
  int32_t* ws_pre; // [B+1] prefix sums of the live requests' work-list items
  // log2-sum-exp of each written output row ([B][qlen][Hq], -inf for +0 rows),
  // or null: what a caller needs to merge these rows with attention over
  // other tokens
  float* lse;
  int64_t page_stride;
  // qlen: new tokens (queries) per request; C = G * qlen MFMA columns used
  int32_t batch, max_pages, num_pages, Hq, Hkv, G, qlen, C, out_f32;
  float sm_scale;
};

// Q and the output are [B][qlen][Hq][128].  Column n < C of the MFMA tiles of
// (request b, kv-head g) holds query n / G of q-head g*G + n % G: this is the
// row of Q and of the output it reads and writes.  With several queries per
// request (several new tokens checked at once, speculative decoding) query i
// sees the cache up to its own token: it ignores the last qlen-1-i tokens.
__device__ __forceinline__ int64_t column_row(const DecodeArgs& a, int b, int g, int n) {
  const int qi = n / a.G;
  return (static_cast<int64_t>(b) * a.qlen + qi) * a.Hq + g * a.G + (n - qi * a.G);
}

constexpr int kMaxBatch = 4096;

// Per-request and per-head constants (context lengths, scales) that the
// decode kernel never writes, read at a wave-uniform index through the scalar
// cache.  Vector loads retire in order, so waiting for one of them would also
// wait for every K/V load issued before it; a scalar load is waited on with
// the LDS counter instead and leaves the K/V prefetch in flight.
template <class T>
__device__ __forceinline__ T uniform_load(const T* p, int i) {
  typedef const __attribute__((address_space(4))) T ConstT;
  return ((ConstT*)p)[__builtin_amdgcn_readfirstlane(i)];
}

// Barrier for hand-offs through LDS only: it waits for this wave's LDS
// accesses but not for its global loads and stores (a full __syncthreads
// fence would drain the K/V prefetch of the next piece).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Prompts shared by groups of requests.  Requests [req_start[k], req_end[k])
// continue prompt k of prefix_len[k] tokens, on the pages their tables list
// first (read from the table of the group's first request).  Group k's
// prompt-pass workgroups are [wg_start[k], wg_start[k+1]): S[k] page ranges x
// Hkv x blocks[k] column blocks; its partial states start at row
// part_base[k] of the workspace.
constexpr int kMaxPromptGroups = 32;
// the fused shared-prompt grid runs the decode over the views with this
// fraction of the plain decode grid's workgroups: a third, with the default
// grid one workgroup per CU beside the prompt pass's two (the full grid, a
// quarter and a sixth measured 2%, 6% and 24% slower)
#ifndef FP8KV_FUSED_DECODE_DIV
#define FP8KV_FUSED_DECODE_DIV 3
#endif
constexpr int kFusedDecodeDiv = FP8KV_FUSED_DECODE_DIV;
struct PromptGroups {
  int32_t n;
  int32_t req_start[kMaxPromptGroups];
  int32_t req_end[kMaxPromptGroups];
  int32_t prefix_len[kMaxPromptGroups];
  int32_t S[kMaxPromptGroups];
  int32_t tiles[kMaxPromptGroups];
  int32_t blocks[kMaxPromptGroups];
  int32_t wg_start[kMaxPromptGroups + 1];
  int64_t part_base[kMaxPromptGroups + 1];
};

// the group of request b, or -1
__device__ __forceinline__ int prompt_group(const PromptGroups& pg, int b) {
  for (int k = 0; k < pg.n; ++k)
    if (b >= pg.req_start[k] && b < pg.req_end[k]) return k;
  return -1;
}

// pages of request b's table the decode skips: its prompt's, when the body
// runs over the own tokens of a shared-prompt call (VIEWS), else none
template <bool VIEWS>
__device__ __forceinline__ int view_skip(const PromptGroups* pg, int b) {
  if constexpr (!VIEWS) {
    return 0;
  } else {
    const int k = prompt_group(*pg, b);
    return k < 0 ? 0 : pg->prefix_len[k] / kPage;
  }
}

// pages the decode reads for request b past the `skip` pages it skips
__device__ __forceinline__ int live_pages(const DecodeArgs& a, int b, int skip) {
  // the flag is loaded next to the length (without an abort array, from a
  // byte of the length itself, and ignored), not after it
  const int64_t ctx = static_cast<int64_t>(a.ctx_lens[b]) - static_cast<int64_t>(skip) * kPage;
  const uint8_t flag =
      *(a.abort ? a.abort + b : reinterpret_cast<const uint8_t*>(a.ctx_lens + b));
  const int64_t n = ctx > 0 ? (ctx + kPage - 1) / kPage : 0;
  // nothing read for: no context, a length that does not fit the table (fail
  // closed), an aborted request (+0 rows)
  const bool none = n == 0 || n + skip > a.max_pages || (a.abort != nullptr && flag != 0);
  return none ? 0 : static_cast<int>(n);
}

__device__ __forceinline__ void store_out8(const DecodeArgs& a, int64_t idx, const float* v) {
  if (a.out_f32) {
    f32x4_t* o = reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + idx);
    o[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    o[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  } else {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned lo = __builtin_bit_cast(unsigned short, static_cast<__bf16>(v[2 * i]));
      const unsigned hi = __builtin_bit_cast(unsigned short, static_cast<__bf16>(v[2 * i + 1]));
      w[i] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.out) + idx) = w;
  }
}

// The work list: segment (b, g) of a live request holds kPieceItems items
// that read nothing, then one item per page.  Those items stand for a
// piece's fixed cost (its Q load waits for the page loads already in flight,
// and its waves merge through LDS), so the equal-work split gives a slice
// that spans many short segments fewer pages.
#ifndef FP8KV_PIECE_ITEMS
#define FP8KV_PIECE_ITEMS 16
#endif
constexpr int kPieceItems = FP8KV_PIECE_ITEMS;

// A piece: the part of segment (b, g) inside this workgroup's slice.
struct Piece {
  int b, g, n;   // request, kv-head, items of the segment
  int64_t sx;    // work-list index of the segment's first page
  int64_t ps;    // first item of the piece
  int64_t pe;    // one past its last item
};

__device__ __forceinline__ Piece first_piece(const int* s_pre, int B, int Hkv, int64_t X0,
                                             int64_t X1) {
  int lo = 0, hi = B;  // largest b with Hkv*pre[b] <= X0 (a live request since X0 < W)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(Hkv) * s_pre[mid] <= X0)
      lo = mid;
    else
      hi = mid;
  }
  Piece p;
  p.b = lo;
  p.n = s_pre[lo + 1] - s_pre[lo];
  const int64_t sb = static_cast<int64_t>(Hkv) * s_pre[lo];
  p.g = static_cast<int>((X0 - sb) / p.n);
  p.sx = sb + static_cast<int64_t>(p.g) * p.n;
  p.ps = X0;
  p.pe = min(X1, p.sx + p.n);
  return p;
}

// the piece after p inside [.., X1); returns false at the end of the slice
__device__ __forceinline__ bool next_piece(Piece& p, const int* s_pre, int B, int Hkv,
                                           int64_t X1) {
  if (p.pe >= X1) return false;
  if (p.g + 1 < Hkv) {
    ++p.g;
    p.sx += p.n;
  } else {
    int b = p.b;
    do {
      ++b;
    } while (b < B && s_pre[b + 1] == s_pre[b]);
    if (b >= B) return false;
    p.b = b;
    p.g = 0;
    p.n = s_pre[b + 1] - s_pre[b];
    p.sx = static_cast<int64_t>(Hkv) * s_pre[b];
  }
  p.ps = p.sx;
  p.pe = min(X1, p.sx + p.n);
  return true;
}

// page index (within the request) of piece p's first page
__device__ __forceinline__ int piece_first_page(const Piece& p) {
  const int64_t r = p.ps - p.sx - kPieceItems;
  return r > 0 ? static_cast<int>(r) : 0;
}

// pages of piece p that wave `wave` takes (round robin from its first page)
__device__ __forceinline__ int wave_count(const Piece& p, int wave) {
  const int64_t r0 = p.sx + kPieceItems > p.ps ? p.sx + kPieceItems : p.ps;  // first page item
  const int len = p.pe > r0 ? static_cast<int>(p.pe - r0) : 0;
  return len > wave ? (len - wave + kWaves - 1) / kWaves : 0;
}

// position in a wave's padded page sequence
template <int DEPTH>
struct SeqCursor {
  Piece p;
  int i;       // index within the piece's padded run
  int cnt;     // real pages of this wave in the piece
  bool done;

  __device__ __forceinline__ void settle(const int* s_pre, int B, int Hkv, int64_t X1,
                                         int wave) {
    // skip pieces in which this wave has nothing to do
    while (!done && (cnt + DEPTH - 1) / DEPTH * DEPTH <= i) {
      if (!next_piece(p, s_pre, B, Hkv, X1)) {
        done = true;
        break;
      }
      i = 0;
      cnt = wave_count(p, wave);
    }
  }
  __device__ __forceinline__ void advance(const int* s_pre, int B, int Hkv, int64_t X1,
                                          int wave) {
    ++i;
    settle(s_pre, B, Hkv, X1, wave);
  }
  __device__ __forceinline__ bool real() const { return !done && i < cnt; }
  // page index within the request
  __device__ __forceinline__ int page(int wave) const {
    return piece_first_page(p) + wave + kWaves * i;
  }
};

// Slices get at least this many pages' worth of items (one page per wave,
// plus one piece's items): with fewer pages than workgroups, one page per
// slice would cut every segment into pieces that the merge then walks one by
// one, and longer slices chain more dependent loads per workgroup.  Both
// kernels derive the count from the item total alone.
constexpr int64_t kMinSlice = 4;
__device__ __forceinline__ int64_t slice_count(int64_t W, int64_t grid) {
  const int64_t want = (W + kMinSlice + kPieceItems - 1) / (kMinSlice + kPieceItems);
  return want < 1 ? 1 : (want < grid ? want : grid);
}

// workgroups w in [wf, wl] whose slices hold pages of the segment whose items
// are [first, last]; the ones with an empty slice are skipped by callers
__device__ __forceinline__ void segment_workgroups(int64_t first, int64_t last, int64_t W,
                                                   int64_t NWG, int64_t& wf, int64_t& wl) {
  // workgroup holding item x: largest w with w*W/NWG <= x
  wf = ((first + 1) * NWG - 1) / W;
  wl = ((last + 1) * NWG - 1) / W;
}

// The decode kernel's body, run as workgroup wg_id of wg_count: by its own
// kernel, or by the decode part of the shared-prompt call's fused grid, which
// sets VIEWS: each request's table and context are then read past its
// prompt's pages (pg).
template <int CACHE, int DEPTH, int NT, bool VIEWS = false>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, int wg_id, int wg_count,
                                            const PromptGroups* pg = nullptr) {
  constexpr int TB = Tile<CACHE>::kBytes;
  constexpr int NC = Tile<CACHE>::kChunks;
  __shared__ int s_pre[kMaxBatch + 1];
  __shared__ int s_part[kThreads];
  __shared__ float s_acc[kWaves][32][64];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the ring's two pages as one step with PV on the 16x16x32 MFMA: half the PV
  // instructions, which the two-tile form (2 waves per SIMD, twice the MFMA
  // work per page) gains from; the one-tile form refills its first slot a
  // page later that way and measured slower
  constexpr bool kPairPV = DEPTH == 2 && NT == 2;
  const int n = lane & 15;   // MFMA column: (query, head) pair 16*ct + n of tile ct
  const int qd = lane >> 4;  // lane quarter
  const int B = a.batch;
  // trailing tokens of the context the query of column 16*ct + n does not see
  int lag[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int col = kTileCols * ct + n;
    lag[ct] = col < a.C ? a.qlen - 1 - col / a.G : 0;
  }

  // ---- prologue: work-list item prefix sums of the live requests --------
  {
    const int per = (B + kThreads - 1) / kThreads;
    const int b0 = min(B, static_cast<int>(threadIdx.x) * per);
    const int b1 = min(B, b0 + per);
    int sum = 0;
    for (int b = b0; b < b1; ++b) {
      const int np = live_pages(a, b, view_skip<VIEWS>(pg, b));
      const int items = np > 0 ? np + kPieceItems : 0;  // per kv-head segment
      s_pre[b] = items;
      sum += items;
    }
    s_part[threadIdx.x] = sum;
    __syncthreads();
    if (threadIdx.x < 64) {
      int v[4], t = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = s_part[4 * threadIdx.x + i];
        t += v[i];
      }
      int inc = t;  // inclusive scan of the 64 lane totals
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      int run = inc - t;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_part[4 * threadIdx.x + i] = run;
        run += v[i];
      }
      if (threadIdx.x == 63) s_pre[B] = inc;
    }
    __syncthreads();
    int run = s_part[threadIdx.x];
    for (int b = b0; b < b1; ++b) {
      const int np = s_pre[b];
      s_pre[b] = run;
      run += np;
    }
    __syncthreads();
    if (wg_id == 0)
      for (int b = threadIdx.x; b <= B; b += kThreads) a.ws_pre[b] = s_pre[b];
    // requests with nothing to read get +0 rows (aborted, empty, invalid)
    for (int b = wg_id; b < B; b += wg_count) {
      if (s_pre[b + 1] != s_pre[b]) continue;
      const int64_t base = static_cast<int64_t>(b) * a.qlen * a.Hq * kHeadDim;
      for (int i = threadIdx.x; i < a.qlen * a.Hq * kHeadDim; i += kThreads) {
        if (a.out_f32)
          static_cast<float*>(a.out)[base + i] = 0.0f;
        else
          static_cast<uint16_t*>(a.out)[base + i] = 0;
      }
      if (a.lse)
        for (int i = threadIdx.x; i < a.qlen * a.Hq; i += kThreads)
          a.lse[static_cast<int64_t>(b) * a.qlen * a.Hq + i] = -INFINITY;
    }
  }

  // ---- this workgroup's slice --------------------------------------------
  const int64_t W = static_cast<int64_t>(a.Hkv) * s_pre[B];
  const int64_t NWG = slice_count(W, wg_count);
  const int64_t bw = wg_id;
  if (bw >= NWG) return;  // fewer slices than workgroups (uniform: no barrier follows)
  const int64_t X0 = bw * W / NWG;
  const int64_t X1 = (bw + 1) * W / NWG;
  if (X0 >= X1) return;

  const Piece first = first_piece(s_pre, B, a.Hkv, X0, X1);
  SeqCursor<DEPTH> I{first, 0, wave_count(first, wave), false};  // next page to load
  I.settle(s_pre, B, a.Hkv, X1, wave);
  SeqCursor<DEPTH> J = I;  // next page id to fetch

  u32x4_t kr[DEPTH][NC], vr[DEPTH][NC];
  bool okp[DEPTH];
  int pid_ring[DEPTH];

  auto fetch_pid = [&]() -> int {
    int pid = -1;
    // a vector load: it retires right after the page loads issued before it,
    // which are waited for first anyway (page ids through the scalar cache
    // measured slower: 12 waves per CU contend for it)
    if (J.real())
      pid = a.page_table[static_cast<int64_t>(J.p.b) * a.max_pages + view_skip<VIEWS>(pg, J.p.b) +
                         J.page(wave)];
    J.advance(s_pre, B, a.Hkv, X1, wave);
    return pid;
  };
  // A page's K and V loads: together (one-tile form), or K as soon as the
  // slot's K has been used and V after PV (two-tile pair step: its K refill
  // then overlaps the softmax and PV of the pair); the V offset waits per slot
  int64_t voff[DEPTH];
  auto issue_k = [&](int slot, int pid) {
    const bool ok = I.real() && static_cast<unsigned>(pid) < static_cast<unsigned>(a.num_pages);
    const int64_t off =
        ok ? static_cast<int64_t>(pid) * a.page_stride + static_cast<int64_t>(I.p.g) * TB : 0;
    const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.k_cache + off),
                                                       (short)0, ok ? TB : 0, kRsrcWord3);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kr[slot][c] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, c * 1024 + lane * 16, 0, kKvLoadPolicy));
    okp[slot] = ok;
    voff[slot] = off;
    I.advance(s_pre, B, a.Hkv, X1, wave);
  };
  auto issue_v = [&](int slot) {
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.v_cache + voff[slot]), (short)0, okp[slot] ? TB : 0, kRsrcWord3);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      vr[slot][c] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, c * 1024 + lane * 16, 0, kKvLoadPolicy));
  };
  auto issue = [&](int slot, int pid) {
    issue_k(slot, pid);
    issue_v(slot);
  };

  // prime: loads for the first DEPTH pages, page ids for the next DEPTH
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) {
    const int pid = __builtin_amdgcn_readfirstlane(fetch_pid());
    issue(s, pid);
  }
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) pid_ring[s] = fetch_pid();

  // Q fragments (B operands of the QK^T MFMA) of a piece: lane (n, qd) holds,
  // for tile ct and step kk, q[column 16 ct + n][32 qd + 8 kk + i], i < 8;
  // columns past C are 0
  auto load_q = [&](const Piece& pc, u32x4_t (&dst)[NT][4]) {
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const int col = kTileCols * ct + n;
      const u32x4_t* qrow = reinterpret_cast<const u32x4_t*>(
          a.q + column_row(a, pc.b, pc.g, col < a.C ? col : 0) * kHeadDim + 32 * qd);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        dst[ct][kk] = col < a.C ? qrow[kk] : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  Piece P = first;  // piece being processed (all waves visit every piece)
  for (;;) {
    const int cnt = wave_count(P, wave);
    const int iters = (cnt + DEPTH - 1) / DEPTH * DEPTH;
    const int pg0 = piece_first_page(P) + wave;  // my first page in the piece
    const int ctx = uniform_load(a.ctx_lens, P.b) - kPage * view_skip<VIEWS>(pg, P.b);
    // Q is waited for here, once per piece: vector loads retire in order, so
    // this also waits for the pages already in flight (a slice holds only a
    // few pieces).  Waiting at the first MFMA instead would put the wait
    // inside the page loop, where the compiler cannot count the loads issued
    // after Q and drains the prefetch every step.
    u32x4_t qcur[NT][4];
    load_q(P, qcur);
    if constexpr (CACHE == FP8KV_E4M3) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) asm volatile("" ::"v"(qcur[ct][kk]));
    }
    Piece Pn = P;
    const bool has_next = next_piece(Pn, s_pre, B, a.Hkv, X1);

    f32x4_t acc[NT][8];
    float m_run[NT];  // running max of column 16 ct + n (log2 units)
    float l_run[NT];  // this lane's share of the softmax denominator
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[ct][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_run[ct] = -INFINITY;
      l_run[ct] = 0.f;
    }

    if (cnt > 0) {
      // scores in log2 units: s = (q.k_code) * sm_scale * k_scale * log2(e).
      // The scale's sign goes into Q (negating bf16 is exact), so the running
      // max is taken on the raw MFMA scores and |scale| joins the subtraction
      // of the max in one FMA (a zero scale is kept just above 0 so that
      // masked scores stay -inf)
      const float sc = a.sm_scale * (a.k_scale ? uniform_load(a.k_scale, P.g) : 1.0f) * kLog2e;
      const float asc = sc != sc ? sc : fmaxf(fabsf(sc), FLT_MIN);
      const unsigned qflip = sc < 0.f ? 0x80008000u : 0u;
      bf16x8_t qf[NT][4];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x4_t w = qcur[ct][kk];
          qf[ct][kk] = __builtin_bit_cast(bf16x8_t, u32x4_t{w.x ^ qflip, w.y ^ qflip, w.z ^ qflip,
                                                            w.w ^ qflip});
        }

      for (int i0 = 0; i0 < iters; i0 += DEPTH) {
        if constexpr (kPairPV) {
          // the ring's two pages as one 32-token step: joint softmax update, PV
          // on the 16x16x32 MFMA whose k index 8 qd + j holds token
          // 4 qd + (j % 4) of page j / 4 (the lane's own V and P of both pages)
          float sv[2][NT][4];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int i = i0 + s;
            const int page = pg0 + kWaves * i;
            const int left = (i < cnt && okp[s]) ? ctx - page * kPage : 0;
            const int valid = min(left, kPage);
            f32x4_t st[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) st[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              bf16x8_t kfrag;
              if constexpr (CACHE == FP8KV_E4M3) {
                const u32x4_t w = kr[s][kk >> 1];
                kfrag = (kk & 1) ? e4m3x8_to_bf16(w.z, w.w) : e4m3x8_to_bf16(w.x, w.y);
              } else {
                kfrag = __builtin_bit_cast(bf16x8_t, kr[s][kk]);
              }
#pragma unroll
              for (int ct = 0; ct < NT; ++ct)
                st[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qf[ct][kk], st[ct], 0, 0, 0);
            }
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r) sv[s][ct][r] = st[ct][r];
            if (left - (a.qlen - 1) < kPage) {
#pragma unroll
              for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (4 * qd + r >= left - lag[ct]) sv[s][ct][r] = -INFINITY;
              // tokens past the end may hold any bytes: clear their V (in the
              // ring, on this page only) so 0*x stays 0
              const int keep = min(max(valid - 4 * qd, 0), 4);
              u32x4_t vmask;
              if constexpr (CACHE == FP8KV_E4M3) {
                const unsigned m = keep >= 4 ? ~0u : ((1u << (8 * keep)) - 1u);
                vmask = u32x4_t{m, m, m, m};
              } else {
                const unsigned m0 = keep >= 2 ? ~0u : (keep == 1 ? 0xFFFFu : 0u);
                const unsigned m1 = keep >= 4 ? ~0u : (keep == 3 ? 0xFFFFu : 0u);
                vmask = u32x4_t{m0, m1, m0, m1};
              }
#pragma unroll
              for (int c = 0; c < NC; ++c) vr[s][c] &= vmask;
            }
          }
          // both pages' K is used: refill K a pair ahead (V follows after PV)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            issue_k(s, __builtin_amdgcn_readfirstlane(pid_ring[s]));
            pid_ring[s] = fetch_pid();
          }
          float p[NT][8];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            float mx = fmaxf(fmaxf(fmaxf(sv[0][ct][0], sv[0][ct][1]), fmaxf(sv[0][ct][2], sv[0][ct][3])),
                             fmaxf(fmaxf(sv[1][ct][0], sv[1][ct][1]), fmaxf(sv[1][ct][2], sv[1][ct][3])));
            mx = wave_max_rows_swap(mx) * asc;
            const float m_new = fmaxf(m_run[ct], mx);
            if (__any(m_new > m_run[ct] + kLazyRescale)) {
              const float alpha = (m_run[ct] == -INFINITY) ? 0.f : fast_exp2(m_run[ct] - m_new);
#pragma unroll
              for (int t = 0; t < 8; ++t) acc[ct][t] *= alpha;
              l_run[ct] *= alpha;
              m_run[ct] = m_new;
            }
            const float mref = (m_run[ct] == -INFINITY) ? 0.f : m_run[ct];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[ct][j] = fast_exp2(__builtin_fmaf(sv[j / 4][ct][j % 4], asc, -mref));
            l_run[ct] += ((p[ct][0] + p[ct][1]) + (p[ct][2] + p[ct][3])) +
                         ((p[ct][4] + p[ct][5]) + (p[ct][6] + p[ct][7]));
          }
          if constexpr (CACHE == FP8KV_E4M3) {
            f16x8_t ph[NT], pl[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float h = __uint_as_float(__float_as_uint(p[ct][j]) & 0xFFFFE000u);
                ph[ct][j] = static_cast<_Float16>(h);
                pl[ct][j] = static_cast<_Float16>(p[ct][j] - h);
              }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const f16x4_t va = e4m3x4_to_f16(vr[0][t >> 2][t & 3]);
              const f16x4_t vb = e4m3x4_to_f16(vr[1][t >> 2][t & 3]);
              const f16x8_t vfrag = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
#pragma unroll
              for (int ct = 0; ct < NT; ++ct) {
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vfrag, ph[ct], acc[ct][t], 0, 0, 0);
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vfrag, pl[ct], acc[ct][t], 0, 0, 0);
              }
            }
          } else {
            bf16x8_t ph[NT], pl[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float h = __uint_as_float(__float_as_uint(p[ct][j]) & 0xFFFF0000u);
                ph[ct][j] = static_cast<__bf16>(h);
                pl[ct][j] = static_cast<__bf16>(p[ct][j] - h);
              }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const u32x4_t wa = vr[0][t >> 1], wb = vr[1][t >> 1];
              const u32x4_t w = (t & 1) ? u32x4_t{wa.z, wa.w, wb.z, wb.w}
                                        : u32x4_t{wa.x, wa.y, wb.x, wb.y};
              const bf16x8_t vfrag = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
              for (int ct = 0; ct < NT; ++ct) {
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag, ph[ct], acc[ct][t], 0, 0, 0);
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag, pl[ct], acc[ct][t], 0, 0, 0);
              }
            }
          }
#pragma unroll
          for (int s = 0; s < 2; ++s) issue_v(s);
          continue;
        }
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
          const int i = i0 + s;
          const int page = pg0 + kWaves * i;
          // context tokens from this page on (not clamped to the page: a column's
          // limit ctx - lag can fall on this page even when ctx lies beyond it)
          const int left = (i < cnt && okp[s]) ? ctx - page * kPage : 0;
          const int valid = min(left, kPage);

          // ---- S^T = K Q^T : rows = 16 tokens, cols = 16 (query, head) ----
          f32x4_t st[NT];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) st[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            bf16x8_t kfrag;
            if constexpr (CACHE == FP8KV_E4M3) {
              const u32x4_t w = kr[s][kk >> 1];
              kfrag = (kk & 1) ? e4m3x8_to_bf16(w.z, w.w) : e4m3x8_to_bf16(w.x, w.y);
            } else {
              kfrag = __builtin_bit_cast(bf16x8_t, kr[s][kk]);
            }
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
              st[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qf[ct][kk], st[ct], 0, 0, 0);
          }
          // lane (n, qd) now holds scores of column n for tokens 4qd + r
          float sv[NT][4];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[ct][r] = st[ct][r];
          if (left - (a.qlen - 1) < kPage) {  // some column stops inside this page
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * qd + r >= left - lag[ct]) sv[ct][r] = -INFINITY;
            // tokens past the end may hold any bytes: clear their V (in the
            // ring, on this page only) so 0*x stays 0
            const int keep = min(max(valid - 4 * qd, 0), 4);  // tokens 4qd+j, j<keep
            u32x4_t vmask;
            if constexpr (CACHE == FP8KV_E4M3) {
              const unsigned m = keep >= 4 ? ~0u : ((1u << (8 * keep)) - 1u);
              vmask = u32x4_t{m, m, m, m};
            } else {
              const unsigned m0 = keep >= 2 ? ~0u : (keep == 1 ? 0xFFFFu : 0u);
              const unsigned m1 = keep >= 4 ? ~0u : (keep == 3 ? 0xFFFFu : 0u);
              vmask = u32x4_t{m0, m1, m0, m1};
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) vr[s][c] &= vmask;
          }
          float p[NT][4];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            float mx = fmaxf(fmaxf(sv[ct][0], sv[ct][1]), fmaxf(sv[ct][2], sv[ct][3]));
            mx = wave_max_rows_swap(mx) * asc;
            const float m_new = fmaxf(m_run[ct], mx);
            if (__any(m_new > m_run[ct] + kLazyRescale)) {
              const float alpha = (m_run[ct] == -INFINITY) ? 0.f : fast_exp2(m_run[ct] - m_new);
#pragma unroll
              for (int t = 0; t < 8; ++t) acc[ct][t] *= alpha;
              l_run[ct] *= alpha;
              m_run[ct] = m_new;
            }
            const float mref = (m_run[ct] == -INFINITY) ? 0.f : m_run[ct];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[ct][r] = fast_exp2(__builtin_fmaf(sv[ct][r], asc, -mref));
            l_run[ct] += (p[ct][0] + p[ct][1]) + (p[ct][2] + p[ct][3]);
          }

          // ---- O^T += V^T P^T : rows = dims 8m + t (tile t), cols = columns
          if constexpr (CACHE == FP8KV_E4M3) {
            // P split into two f16 terms (hi + lo) so the weights keep ~22 bits:
            // hi is P with its low mantissa bits cleared (exact in f16 over the
            // weights' range), lo the exact remainder
            f16x4_t ph[NT], pl[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float h = __uint_as_float(__float_as_uint(p[ct][r]) & 0xFFFFE000u);
                ph[ct][r] = static_cast<_Float16>(h);
                pl[ct][r] = static_cast<_Float16>(p[ct][r] - h);
              }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const unsigned w = vr[s][t >> 2][t & 3];
              const f16x4_t vfrag = e4m3x4_to_f16(w);
#pragma unroll
              for (int ct = 0; ct < NT; ++ct) {
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x16f16(vfrag, ph[ct], acc[ct][t], 0, 0, 0);
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x16f16(vfrag, pl[ct], acc[ct][t], 0, 0, 0);
              }
            }
          } else {
            s16x4_t ph[NT], pl[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float h = __uint_as_float(__float_as_uint(p[ct][r]) & 0xFFFF0000u);
                ph[ct][r] = __builtin_bit_cast(short, static_cast<__bf16>(h));
                pl[ct][r] = __builtin_bit_cast(short, static_cast<__bf16>(p[ct][r] - h));
              }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const u32x4_t w = vr[s][t >> 1];
              u32x2_t pair;
              pair.x = (t & 1) ? w.z : w.x;
              pair.y = (t & 1) ? w.w : w.y;
              const s16x4_t vfrag = __builtin_bit_cast(s16x4_t, pair);
#pragma unroll
              for (int ct = 0; ct < NT; ++ct) {
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vfrag, ph[ct], acc[ct][t], 0, 0, 0);
                acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vfrag, pl[ct], acc[ct][t], 0, 0, 0);
              }
            }
          }
          // refill this slot DEPTH pages ahead; its page id was fetched DEPTH
          // pages ago; fetch the id 2*DEPTH pages ahead
          issue(s, __builtin_amdgcn_readfirstlane(pid_ring[s]));
          pid_ring[s] = fetch_pid();
        }
      }
    }

    // ---- merge the 4 waves' states for this piece through LDS, one tile of
    // columns at a time -------------------------------------------------------
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const float l_tot = wave_sum_rows(l_run[ct]);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_acc[wave][t * 4 + r][lane] = acc[ct][t][r];
      if (qd == 0) {
        s_m[wave][n] = m_run[ct];
        s_l[wave][n] = l_tot;
      }
      lds_barrier();
      {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][n]);
        float e[kWaves];
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = s_m[w][n];
          e[w] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
          L += e[w] * s_l[w][n];
        }
        // wave `wave` merges accumulator row r = wave: dims 32 qd + 8 wave + t
        float O[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          float o = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) o += e[w] * s_acc[w][t * 4 + wave][lane];
          O[t] = o;
        }
        const int col = kTileCols * ct + n;
        if (col < a.C) {
          const int d0 = 32 * qd + 8 * wave;
          if (P.ps == P.sx && P.pe == P.sx + P.n) {
            // the whole segment sits in this slice: write the output
            const float vsc = a.v_scale ? uniform_load(a.v_scale, P.g) : 1.0f;
            const float inv = L > 0.f ? vsc / L : 0.f;
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = O[t] * inv;
            store_out8(a, column_row(a, P.b, P.g, col) * kHeadDim + d0, v);
            if (a.lse && qd == 0 && wave == 0)
              a.lse[column_row(a, P.b, P.g, col)] = L > 0.f ? M + __log2f(L) : -INFINITY;
          } else {
            const int64_t pidx = (bw + static_cast<int64_t>(P.b) * a.Hkv + P.g) * a.C + col;
            f32x4_t* po = reinterpret_cast<f32x4_t*>(a.ws_o + pidx * kHeadDim + d0);
            po[0] = f32x4_t{O[0], O[1], O[2], O[3]};
            po[1] = f32x4_t{O[4], O[5], O[6], O[7]};
            if (qd == 0 && wave == 0) {
              a.ws_ml[pidx * 2] = M;
              a.ws_ml[pidx * 2 + 1] = L;
            }
          }
        }
      }
      lds_barrier();  // LDS is reused by the next tile or piece
    }
    if (!has_next) break;
    P = Pn;
  }
}

// NT: 16-column tiles of (query, head) pairs per kv-head (1 or 2).  Two tiles
// double the Q fragments and accumulators, so that form runs 2 waves per SIMD
// instead of 3; each page's K/V fragments are converted once for both tiles.
template <int CACHE, int DEPTH, int NT>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(NT == 1 ? 3 : 2, NT == 1 ? 3 : 2)))
void decode_kernel(DecodeArgs a) {
  decode_body<CACHE, DEPTH, NT>(a, static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
}

// ---------------------------------------------------------------------------
// 5. merge of the pieces of split segments (fixed order: deterministic)
// ---------------------------------------------------------------------------
// Workgroups stride over (request, kv-head) segments.  Two forms: a flat one
// (a thread per (head, 4 dims) pair walks all of the segment's pieces) for
// segments of a few pieces, and a grouped one for segments cut into many
// pieces (few long requests): there a thread takes one (head, 4 dims) pair and
// one group of consecutive pieces, and the groups' states meet in LDS in group
// order.  Both are deterministic.  A separate pass: ordering the partial
// writes of other workgroups inside the decode kernel would need a device-scope
// release/acquire per piece, which on this part writes back and invalidates
// the L2 and costs far more than this launch.
constexpr int kMergeUnroll = 8;
// flat form: a thread per (column, 4 dims) pair, 256 to 1024 threads (C*32)
constexpr int kMergeFlatMaxThreads = 1024;
constexpr int kMergeGroupedThreads = 1024;
// segments average at least this many pieces: the grouped form
constexpr int kMergeGroupedMinPieces = 4;
// workgroups per (request, kv-head) segment at most, with the default grid
constexpr int kDefaultPiecesPerSegment = 24;

// fold one piece's (max, sum, weighted V) into a running state
__device__ __forceinline__ void merge_state(float& M, float& L, f32x4_t& O, float m, float l,
                                            f32x4_t o) {
  if (m == -INFINITY) return;
  if (m > M) {
    const float r = (M == -INFINITY) ? 0.f : fast_exp2(M - m);
    L *= r;
    O *= r;
    M = m;
  }
  const float e = fast_exp2(m - M);
  L += e * l;
  O += e * o;
}

// the pieces of workgroups [w0, w1) of segment seg, for head n, dims d..d+3
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int64_t seg, int n, int d,
                                             int64_t w0, int64_t w1, float& M, float& L,
                                             f32x4_t& O) {
  for (int64_t w = w0; w < w1; w += kMergeUnroll) {
    // issue the loads of several pieces before using any of them
    float m[kMergeUnroll], l[kMergeUnroll];
    f32x4_t o[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const bool has = w + u < w1;
      const int64_t pidx = (w + u + seg) * a.C + n;
      m[u] = has ? a.ws_ml[pidx * 2] : -INFINITY;
      l[u] = has ? a.ws_ml[pidx * 2 + 1] : 0.f;
      o[u] = has ? *reinterpret_cast<const f32x4_t*>(a.ws_o + pidx * kHeadDim + d)
                 : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) merge_state(M, L, O, m[u], l[u], o[u]);
  }
}

__device__ __forceinline__ void merge_store(const DecodeArgs& a, int b, int g, int n, int d,
                                            float M, float L, f32x4_t O) {
  const float vsc = a.v_scale ? a.v_scale[g] : 1.0f;
  const float inv = L > 0.f ? vsc / L : 0.f;
  if (a.lse && d == 0) a.lse[column_row(a, b, g, n)] = L > 0.f ? M + __log2f(L) : -INFINITY;
  const int64_t io = column_row(a, b, g, n) * kHeadDim + d;
  if (a.out_f32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + io) = O * inv;
  } else {
    u32x2_t w;
    w.x = __builtin_bit_cast(unsigned short, static_cast<__bf16>(O[0] * inv)) |
          (static_cast<unsigned>(__builtin_bit_cast(unsigned short, static_cast<__bf16>(O[1] * inv))) << 16);
    w.y = __builtin_bit_cast(unsigned short, static_cast<__bf16>(O[2] * inv)) |
          (static_cast<unsigned>(__builtin_bit_cast(unsigned short, static_cast<__bf16>(O[3] * inv))) << 16);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + io) = w;
  }
}

// The workgroups holding pieces of segment seg (false: nothing to merge, the
// segment is empty or one workgroup wrote it whole).  With at least one page
// per workgroup no slice is empty, so every workgroup in [wf, wl] holds one.
__device__ __forceinline__ bool segment_span(const DecodeArgs& a, int seg, int64_t W,
                                             int64_t NWG, int64_t& wf, int64_t& wl) {
  const int b = seg / a.Hkv;
  const int g = seg % a.Hkv;
  const int pre_b = a.ws_pre[b];
  const int np = a.ws_pre[b + 1] - pre_b;
  if (np == 0) return false;
  const int64_t first = static_cast<int64_t>(a.Hkv) * pre_b + static_cast<int64_t>(g) * np;
  segment_workgroups(first, first + np - 1, W, NWG, wf, wl);
  return wf != wl;
}

__global__ __launch_bounds__(kMergeFlatMaxThreads) void merge_flat_kernel(DecodeArgs a,
                                                                          int64_t grid) {
  const int64_t W = static_cast<int64_t>(a.Hkv) * a.ws_pre[a.batch];
  const int64_t NWG = slice_count(W, grid);
  for (int seg = blockIdx.x; seg < a.batch * a.Hkv; seg += gridDim.x) {
    int64_t wf, wl;
    if (!segment_span(a, seg, W, NWG, wf, wl)) continue;
    for (int idx = threadIdx.x; idx < a.C * (kHeadDim / 4); idx += blockDim.x) {
      const int n = idx / (kHeadDim / 4);
      const int d = 4 * (idx % (kHeadDim / 4));
      float M = -INFINITY, L = 0.f;
      f32x4_t O = {0.f, 0.f, 0.f, 0.f};
      merge_pieces(a, seg, n, d, wf, wl + 1, M, L, O);
      merge_store(a, seg / a.Hkv, seg % a.Hkv, n, d, M, L, O);
    }
  }
}

__global__ __launch_bounds__(kMergeGroupedThreads) void merge_grouped_kernel(DecodeArgs a,
                                                                             int64_t grid) {
  __shared__ float s_m[kMergeGroupedThreads];
  __shared__ float s_l[kMergeGroupedThreads];
  __shared__ f32x4_t s_o[kMergeGroupedThreads];
  const int64_t W = static_cast<int64_t>(a.Hkv) * a.ws_pre[a.batch];
  const int64_t NWG = slice_count(W, grid);
  const int items = a.C * (kHeadDim / 4);            // (column, 4 dims) pairs, at most 1024
  const int groups = kMergeGroupedThreads / items;   // at least 1
  const int t = threadIdx.x;
  const bool active = t < items * groups;
  const int idx = t % items, grp = t / items;
  const int n = idx / (kHeadDim / 4);
  const int d = 4 * (idx % (kHeadDim / 4));
  for (int seg = blockIdx.x; seg < a.batch * a.Hkv; seg += gridDim.x) {
    int64_t wf, wl;
    if (!segment_span(a, seg, W, NWG, wf, wl)) continue;  // uniform: no barrier skipped
    const int64_t chunk = (wl - wf + groups) / groups;
    const int64_t w0 = wf + grp * chunk;
    const int64_t w1 = (w0 + chunk < wl + 1) ? w0 + chunk : wl + 1;
    float M = -INFINITY, L = 0.f;
    f32x4_t O = {0.f, 0.f, 0.f, 0.f};
    if (active) merge_pieces(a, seg, n, d, w0, w1, M, L, O);
    s_m[t] = M;
    s_l[t] = L;
    s_o[t] = O;
    __syncthreads();
    if (active && grp == 0) {
      for (int k = 1; k < groups; ++k)
        merge_state(M, L, O, s_m[k * items + idx], s_l[k * items + idx], s_o[k * items + idx]);
      merge_store(a, seg / a.Hkv, seg % a.Hkv, n, d, M, L, O);
    }
    __syncthreads();  // LDS is reused for the next segment
  }
}

// ---------------------------------------------------------------------------
// 6. prompts shared by groups of requests (cache reuse)
// ---------------------------------------------------------------------------
// When a group of requests continues one prompt whose pages they all map,
// each of those pages is read once per kv-head for the whole group: the MFMA
// columns are the group's (request, q-head) pairs of the kv-head (16 per
// wave), so the prompt part is a dense product instead of separate reads.  A
// workgroup takes 4 column tiles (one per wave) and a range of the prompt's
// pages; its waves read the same pages at the same time, which the caches
// serve once.  Each (column, page range) leaves (max, sum, weighted V) for
// the combine pass.  The requests' own tokens go through decode_kernel over
// the rest of their tables, with its log-sum-exp output.
// The groups are described by PromptGroups (before the decode kernel, whose
// body can skip each request's prompt pages).
struct PrefixArgs {
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const uint16_t* q;           // [B][Hq][128]
  const int32_t* page_table;   // [B][max_pages]
  const int32_t* ctx_lens;     // [B]
  int32_t* view_pt;            // [B][max_pages]: each table past its prompt
  int32_t* view_ctx;           // [B]: each context past its prompt
  uint8_t* member_ok;          // [B]: a grouped request's table lists its prompt's pages
  float* ws_o;                 // [rows][128], rows as in PromptGroups
  float* ws_ml;                // [rows][2]
  int64_t page_stride;
  int32_t batch, Hq, Hkv, G, max_pages, num_pages;
  float sm_scale;
  PromptGroups pg;
};

// The own-token view of every request: its table past its prompt's pages and
// its context past the prompt (the plain decode then runs on it).  A
// workgroup per request.
__global__ __launch_bounds__(256) void view_kernel(PrefixArgs a) {
  const int b = blockIdx.x;
  const int k = prompt_group(a.pg, b);
  const int p0 = k < 0 ? 0 : a.pg.prefix_len[k] / kPage;
  const int64_t row = static_cast<int64_t>(b) * a.max_pages;
  for (int j = threadIdx.x; j < a.max_pages; j += 256)
    a.view_pt[row + j] = j + p0 < a.max_pages ? a.page_table[row + j + p0] : -1;
  if (threadIdx.x == 0) a.view_ctx[b] = a.ctx_lens[b] - p0 * kPage;
}

// NT column tiles per wave: each page's K and V fragments are loaded and
// converted once for NT x 16 columns.  Two tiles run two waves per SIMD (an
// e4m3 cache would fit three, which measured slower: 1.5x the page ranges,
// hence 1.5x the partial states written and merged).
template <int CACHE, int NT>
__device__ __forceinline__ void prefix_body(const PrefixArgs& a, int wg_id) {
  constexpr int TB = Tile<CACHE>::kBytes;
  constexpr int NC = Tile<CACHE>::kChunks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qd = lane >> 4;
  // workgroup -> (prompt group k, kv-head g, page range s, column block): the
  // blocks reading the same pages are Hkv*S apart, so with Hkv*S a multiple of
  // 8 they land on one XCD (workgroups go round robin over the 8) and share
  // its L2
  int k = 0;
  while (k + 1 < a.pg.n && wg_id >= a.pg.wg_start[k + 1]) ++k;
  const int S = a.pg.S[k];
  const int P0 = a.pg.prefix_len[k] / kPage;
  const int wg = wg_id - a.pg.wg_start[k];
  // Fail closed: the prompt's pages are read through the table of the group's
  // first request, while each member's tag check covered its own table; a
  // member whose table does not list the same pages first gets +0 rows.  The
  // last wave of each of the group's workgroups compares a share of the
  // members' tables with the first one (before any of its page loads).
  if (wave == kWaves - 1) {
    const int nwg = a.pg.wg_start[k + 1] - a.pg.wg_start[k];
    const int first = a.pg.req_start[k];
    const int32_t* pt0 = a.page_table + static_cast<int64_t>(first) * a.max_pages;
    for (int r = first + wg; r < a.pg.req_end[k]; r += nwg) {
      const int32_t* ptr = a.page_table + static_cast<int64_t>(r) * a.max_pages;
      int diff = 0;
      for (int j = lane; j < P0; j += 64) diff |= ptr[j] != pt0[j] ? 1 : 0;
      diff = __any(diff);
      if (lane == 0) a.member_ok[r] = diff ? 0 : 1;
    }
  }
  const int gs = wg % (a.Hkv * S);
  const int blk = wg / (a.Hkv * S);
  const int g = gs / S, s = gs % S;
  const int tile0 = (blk * kWaves + wave) * NT;
  if (tile0 >= a.pg.tiles[k]) return;  // no barrier in this kernel
  const int b0 = a.pg.req_start[k];
  const int nreq = a.pg.req_end[k] - b0;
  const int cols = nreq * a.G;
  const int32_t* prefix_pages = a.page_table + static_cast<int64_t>(b0) * a.max_pages;
  // the score scale's sign goes into Q (negating bf16 is exact), so the
  // running max is taken on the raw MFMA scores and |scale| joins the
  // subtraction of the max in one FMA (a zero scale is kept just above 0 so
  // that masked scores stay -inf)
  const float sc = a.sm_scale * (a.k_scale ? uniform_load(a.k_scale, g) : 1.0f) * kLog2e;
  const float asc = sc != sc ? sc : fmaxf(fabsf(sc), FLT_MIN);
  const unsigned qflip = sc < 0.f ? 0x80008000u : 0u;
  int col[NT], bl[NT];
  int64_t row[NT];
  bf16x8_t qf[NT][4];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    col[ct] = (tile0 + ct) * kTileCols + n;
    bl[ct] = col[ct] / a.G;  // request within the group
    row[ct] = static_cast<int64_t>(b0 + bl[ct]) * a.Hq + g * a.G + (col[ct] - bl[ct] * a.G);
    const bool has = col[ct] < cols;
    const u32x4_t* qrow = reinterpret_cast<const u32x4_t*>(a.q + (has ? row[ct] : 0) * kHeadDim +
                                                           32 * qd);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4_t w = has ? qrow[kk] : u32x4_t{0u, 0u, 0u, 0u};
      qf[ct][kk] = __builtin_bit_cast(bf16x8_t, u32x4_t{w.x ^ qflip, w.y ^ qflip, w.z ^ qflip,
                                                        w.w ^ qflip});
    }
  }
  const int p0 = static_cast<int>(static_cast<int64_t>(s) * P0 / S);
  const int p1 = static_cast<int>(static_cast<int64_t>(s + 1) * P0 / S);

  // pages in flight: the two of one step (a deeper ring measured no faster:
  // this kernel is bound by its per-page arithmetic, not by load latency)
  constexpr int R = 2;
  u32x4_t kr[R][NC], vr[R][NC];
  bool okp[R];
  auto issue = [&](int slot, int p) {
    const int pid = p < p1 ? uniform_load(prefix_pages, p) : -1;
    const bool ok = static_cast<unsigned>(pid) < static_cast<unsigned>(a.num_pages);
    const int64_t off = ok ? static_cast<int64_t>(pid) * a.page_stride + static_cast<int64_t>(g) * TB : 0;
    const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.k_cache + off),
                                                       (short)0, ok ? TB : 0, kRsrcWord3);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.v_cache + off),
                                                       (short)0, ok ? TB : 0, kRsrcWord3);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kr[slot][c] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, c * 1024 + lane * 16, 0, 0));
#pragma unroll
    for (int c = 0; c < NC; ++c)
      vr[slot][c] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, c * 1024 + lane * 16, 0, 0));
    okp[slot] = ok;
  };
#pragma unroll
  for (int r = 0; r < R; ++r) issue(r, p0 + r);

  f32x4_t acc[NT][8];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[ct][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
  }
  // the two pages of the ring are one 32-token step: PV runs on the 16x16x32
  // MFMA, whose k index 8 qd + j holds token 4 qd + (j % 4) of page j / 4 --
  // the lane's own V and P values of the two pages side by side
  for (int p = p0; p < p1; p += 2) {
    float sv[NT][2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      f32x4_t st[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) st[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t kfrag;
        if constexpr (CACHE == FP8KV_E4M3) {
          const u32x4_t w = kr[r][kk >> 1];
          kfrag = (kk & 1) ? e4m3x8_to_bf16(w.z, w.w) : e4m3x8_to_bf16(w.x, w.y);
        } else {
          kfrag = __builtin_bit_cast(bf16x8_t, kr[r][kk]);
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          st[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qf[ct][kk], st[ct], 0, 0, 0);
      }
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[ct][r][i] = st[ct][i];
      // the prompt's pages are full; a page past the range or with an id
      // outside the pool adds nothing (a wave-uniform, rare branch)
      if (!(okp[r] && p + r < p1)) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[ct][r][i] = -INFINITY;
      }
    }
    // softmax of every tile first, so that each V fragment below is
    // converted once and feeds all tiles' PV products (one live fragment)
    using PFrag = std::conditional_t<CACHE == FP8KV_E4M3, f16x8_t, bf16x8_t>;
    PFrag ph[NT], pl[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      float mx = fmaxf(fmaxf(fmaxf(sv[ct][0][0], sv[ct][0][1]), fmaxf(sv[ct][0][2], sv[ct][0][3])),
                       fmaxf(fmaxf(sv[ct][1][0], sv[ct][1][1]), fmaxf(sv[ct][1][2], sv[ct][1][3])));
      mx = wave_max_rows_swap(mx) * asc;
      // lazy rescale: the reference max moves only when a column's max
      // passes it by more than 2^kLazyRescale, so the weights stay below that
      // bound and most steps leave the accumulators alone
      const float m_new = fmaxf(m_run[ct], mx);
      if (__any(m_new > m_run[ct] + kLazyRescale)) {
        const float alpha = (m_run[ct] == -INFINITY) ? 0.f : fast_exp2(m_run[ct] - m_new);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[ct][t] *= alpha;
        l_run[ct] *= alpha;
        m_run[ct] = m_new;
      }
      const float mref = (m_run[ct] == -INFINITY) ? 0.f : m_run[ct];
      float pr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pr[j] = fast_exp2(__builtin_fmaf(sv[ct][j / 4][j % 4], asc, -mref));
      l_run[ct] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      // P in two terms (hi + lo) so the weights keep ~22 bits (16 for bf16):
      // hi is P with its low mantissa bits cleared (exact in the 16-bit type
      // over the weights' range), lo the exact remainder
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (CACHE == FP8KV_E4M3) {
          const float h = __uint_as_float(__float_as_uint(pr[j]) & 0xFFFFE000u);
          ph[ct][j] = static_cast<_Float16>(h);
          pl[ct][j] = static_cast<_Float16>(pr[j] - h);
        } else {
          const float h = __uint_as_float(__float_as_uint(pr[j]) & 0xFFFF0000u);
          ph[ct][j] = static_cast<__bf16>(h);
          pl[ct][j] = static_cast<__bf16>(pr[j] - h);
        }
      }
    }
    // PV: V of the step's two pages in the MFMA's operand order
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if constexpr (CACHE == FP8KV_E4M3) {
        const f16x4_t va = e4m3x4_to_f16(vr[0][t >> 2][t & 3]);
        const f16x4_t vb = e4m3x4_to_f16(vr[1][t >> 2][t & 3]);
        const f16x8_t vfrag = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vfrag, ph[ct], acc[ct][t], 0, 0, 0);
          acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vfrag, pl[ct], acc[ct][t], 0, 0, 0);
        }
      } else {
        const u32x4_t wa = vr[0][t >> 1], wb = vr[1][t >> 1];
        const u32x4_t w = (t & 1) ? u32x4_t{wa.z, wa.w, wb.z, wb.w} : u32x4_t{wa.x, wa.y, wb.x, wb.y};
        const bf16x8_t vfrag = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag, ph[ct], acc[ct][t], 0, 0, 0);
          acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag, pl[ct], acc[ct][t], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) issue(r, p + r + 2);
  }
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const float l_tot = wave_sum_rows(l_run[ct]);
    if (col[ct] < cols) {
      // acc[t][i] of lane (n, qd) holds dim 32 qd + 8 i + t
      const int64_t pidx = a.pg.part_base[k] + (static_cast<int64_t>(s) * nreq + bl[ct]) * a.Hq +
                           (row[ct] - static_cast<int64_t>(b0 + bl[ct]) * a.Hq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4_t* po = reinterpret_cast<f32x4_t*>(a.ws_o + pidx * kHeadDim + 32 * qd + 8 * i);
        po[0] = f32x4_t{acc[ct][0][i], acc[ct][1][i], acc[ct][2][i], acc[ct][3][i]};
        po[1] = f32x4_t{acc[ct][4][i], acc[ct][5][i], acc[ct][6][i], acc[ct][7][i]};
      }
      if (qd == 0) {
        a.ws_ml[pidx * 2] = m_run[ct];
        a.ws_ml[pidx * 2 + 1] = l_tot;
      }
    }
  }
}

template <int CACHE, int NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 3 : 2, NT == 1 ? 3 : 2)))
void prefix_kernel(PrefixArgs a) {
  prefix_body<CACHE, NT>(a, static_cast<int>(blockIdx.x));
}

// The prompt pass and the own-token decode in one grid (e4m3 cache, at most
// 16 columns): workgroups [0, prefix_wgs) run the prompt pass, the others the
// decode over the views (its slices numbered from 0).  Workgroups go out in
// index order, so the decode's fill the slots the prompt pass leaves (three
// waves per SIMD here) and its memory-bound work runs beside the prompt
// pass's issue-bound work instead of after it.
template <int NTP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void shared_fused_kernel(PrefixArgs pa, DecodeArgs da, int32_t prefix_wgs, int32_t decode_wgs) {
  const int w = static_cast<int>(blockIdx.x);
  if (w < prefix_wgs)
    prefix_body<FP8KV_E4M3, NTP>(pa, w);
  else
    decode_body<FP8KV_E4M3, FP8KV_DEPTH_E4M3, 1, true>(da, w - prefix_wgs, decode_wgs, &pa.pg);
}

// Output rows of the shared-prompt call: the prompt's S partial states and
// the own-token rows (normalised, with their log-sum-exp) in one log-sum-exp.
// A thread per (row, 4 dims).  Rows of aborted requests, of contexts that do
// not extend past the prompt, of contexts the table cannot hold and of group
// members whose table does not list the prompt's pages are +0.
struct CombineArgs {
  const float* ws_o;
  const float* ws_ml;
  const float* suf_out;   // [B][Hq][128] f32
  const float* suf_lse;   // [B][Hq]
  const int32_t* ctx_lens;
  const uint8_t* abort;
  const uint8_t* member_ok;  // [B], written by the prompt pass for grouped requests
  const float* v_scale;
  void* out;
  int32_t batch, Hq, G, out_f32;
  int64_t max_tokens;     // the table's width in tokens
  PromptGroups pg;
  // fold_merge: the own-token decode's split segments are merged here from
  // its pieces (decode = its arguments, decode_grid = its workgroups); the
  // rows it wrote whole are read as above
  int32_t fold_merge;
  int64_t decode_grid;
  DecodeArgs decode;
};

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rows = static_cast<int64_t>(a.batch) * a.Hq;
  if (idx >= rows * (kHeadDim / 4)) return;
  const int64_t row = idx / (kHeadDim / 4);
  const int d = 4 * static_cast<int>(idx % (kHeadDim / 4));
  const int b = static_cast<int>(row / a.Hq);
  const int h = static_cast<int>(row % a.Hq);
  const int k = prompt_group(a.pg, b);
  const int S = k < 0 ? 0 : a.pg.S[k];
  const int prefix_len = k < 0 ? 0 : a.pg.prefix_len[k];
  const int64_t nreq = k < 0 ? 0 : a.pg.req_end[k] - a.pg.req_start[k];
  const int64_t base = k < 0 ? 0 : a.pg.part_base[k] + (b - a.pg.req_start[k]) * a.Hq + h;
  const int ctx = a.ctx_lens[b];
  const bool aborted = a.abort != nullptr && a.abort[b] != 0;
  const bool member = k < 0 || a.member_ok[b] != 0;  // its table lists the prompt's pages
  f32x4_t res = {0.f, 0.f, 0.f, 0.f};
  if (!aborted && member && ctx > prefix_len && ctx <= a.max_tokens) {
    const float vsc = a.v_scale ? a.v_scale[h / a.G] : 1.0f;
    float M = -INFINITY, L = 0.f;
    f32x4_t O = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kMergeUnroll) {
      // issue the loads of several ranges before using any of them
      float m[kMergeUnroll], l[kMergeUnroll];
      f32x4_t o[kMergeUnroll];
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const bool has = s0 + u < S;
        const int64_t pidx = base + (s0 + u) * nreq * a.Hq;
        m[u] = has ? a.ws_ml[pidx * 2] : -INFINITY;
        l[u] = has ? a.ws_ml[pidx * 2 + 1] : 0.f;
        o[u] = has ? *reinterpret_cast<const f32x4_t*>(a.ws_o + pidx * kHeadDim + d)
                   : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) merge_state(M, L, O, m[u], l[u], o[u]);
    }
    O *= vsc;  // the prompt's partial sums are in cache units
    int64_t wf = 0, wl = 0;
    bool split = false;
    const int g = h / a.G;
    const int seg = b * a.decode.Hkv + g;
    if (a.fold_merge) {
      const int64_t W = static_cast<int64_t>(a.decode.Hkv) * a.decode.ws_pre[a.batch];
      split = segment_span(a.decode, seg, W, slice_count(W, a.decode_grid), wf, wl);
    }
    if (split) {
      // the own-token pieces' states (sums in cache units)
      float Ms = -INFINITY, Ls = 0.f;
      f32x4_t Os = {0.f, 0.f, 0.f, 0.f};
      merge_pieces(a.decode, seg, h - g * a.G, d, wf, wl + 1, Ms, Ls, Os);
      merge_state(M, L, O, Ms, Ls, Os * vsc);
    } else {
      // the own-token rows are normalised: as a state, (lse, 1, row)
      merge_state(M, L, O, a.suf_lse[row], 1.0f,
                  *reinterpret_cast<const f32x4_t*>(a.suf_out + row * kHeadDim + d));
    }
    if (L > 0.f) res = O * (1.0f / L);
  }
  const int64_t io = row * kHeadDim + d;
  if (a.out_f32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + io) = res;
  } else {
    u32x2_t w;
    w.x = __builtin_bit_cast(unsigned short, static_cast<__bf16>(res[0])) |
          (static_cast<unsigned>(__builtin_bit_cast(unsigned short, static_cast<__bf16>(res[1]))) << 16);
    w.y = __builtin_bit_cast(unsigned short, static_cast<__bf16>(res[2])) |
          (static_cast<unsigned>(__builtin_bit_cast(unsigned short, static_cast<__bf16>(res[3]))) << 16);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + io) = w;
  }
}

// ---------------------------------------------------------------------------
// self-test of the conversions used above
// ---------------------------------------------------------------------------
// Streaming-read reference: every byte of a buffer read once, as the tile
// loads read (16-byte buffer loads with their cache policy, each wave a 4 KiB
// block at a time, 4 blocks in flight), but in order and with no page
// indirection; XOR-folded to one word per thread so nothing is optimised away.
__global__ __launch_bounds__(256) void read_bandwidth_kernel(const uint8_t* buf, int64_t bytes,
                                                             uint32_t* sink) {
  constexpr int kBlock = 4096;
  const int lane = threadIdx.x & 63;
  const int64_t wave =
      __builtin_amdgcn_readfirstlane(static_cast<int>((blockIdx.x * 256 + threadIdx.x) >> 6));
  const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t blocks = (bytes + kBlock - 1) / kBlock;
  uint32_t x = 0;
  for (int64_t b0 = wave; b0 < blocks; b0 += 4 * waves) {
    u32x4_t v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t b = b0 + u * waves;
      const int64_t base = b < blocks ? b * kBlock : 0;
      const int n = b < blocks ? static_cast<int>(bytes - base < kBlock ? bytes - base : kBlock) : 0;
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf + base), (short)0, n,
                                                        kRsrcWord3);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[u][k] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, k * 1024 + lane * 16, 0, kKvLoadPolicy));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) x ^= v[u][k].x ^ v[u][k].y ^ v[u][k].z ^ v[u][k].w;
  }
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = x;
}

__global__ void debug_convert_kernel(const uint8_t* codes, float* out, int n, int which) {
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const unsigned w = *reinterpret_cast<const unsigned*>(codes + i);
  if (which == 0) {
    const bf16x8_t v = e4m3x8_to_bf16(w, 0u);
    for (int j = 0; j < 4; ++j) out[i + j] = static_cast<float>(v[j]);
  } else {
    const f16x4_t v = e4m3x4_to_f16(w);
    for (int j = 0; j < 4; ++j) out[i + j] = static_cast<float>(v[j]);
  }
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
fp8kv_status hip_status(hipError_t e) {
  if (e == hipSuccess) return FP8KV_OK;
  fp8kv_detail::record_hip_error(static_cast<int32_t>(e));
  return FP8KV_HIP_ERROR;
}

fp8kv_status launched() { return hip_status(hipGetLastError()); }

fp8kv_status check_desc(const fp8kv_cache_desc* d) {
  if (!d) return FP8KV_INVALID_ARG;
  if (d->page_size != kPage || d->head_dim != kHeadDim) return FP8KV_UNSUPPORTED;
  if (d->cache_dtype != FP8KV_E4M3 && d->cache_dtype != FP8KV_BF16) return FP8KV_UNSUPPORTED;
  if (d->num_pages <= 0 || d->num_kv_heads <= 0) return FP8KV_INVALID_ARG;
  return FP8KV_OK;
}

int tile_bytes(const fp8kv_cache_desc* d) {
  return d->cache_dtype == FP8KV_E4M3 ? Tile<FP8KV_E4M3>::kBytes : Tile<FP8KV_BF16>::kBytes;
}

// Workers (waves) of the decode kernel: all of them resident at once.
int32_t device_workers() {
  // compute-unit count per device, queried once
  constexpr int kMaxDevices = 64;
  static std::atomic<int32_t> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int32_t c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c * FP8KV_WAVES_PER_CU;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus * FP8KV_WAVES_PER_CU;
}

struct WorkspaceLayout {
  size_t o, ml, pre, total;
};

// C = (Hq / Hkv) * qlen columns per partial
WorkspaceLayout workspace_layout(int64_t batch, int64_t Hq, int64_t Hkv, int64_t qlen,
                                 int64_t workers) {
  const int64_t C = Hq / Hkv * qlen;
  const int64_t slots = workers / kWaves + batch * Hkv;  // (workgroup + segment) slots
  WorkspaceLayout L;
  L.o = 0;
  L.ml = L.o + static_cast<size_t>(slots * C * kHeadDim) * sizeof(float);
  L.pre = L.ml + static_cast<size_t>(slots * C * 2) * sizeof(float);
  L.pre = (L.pre + 255) / 256 * 256;
  L.total = L.pre + static_cast<size_t>(batch + 1) * sizeof(int32_t);
  return L;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* fp8kv_status_string(fp8kv_status s) {
  switch (s) {
    case FP8KV_OK: return "ok";
    case FP8KV_INVALID_ARG: return "invalid argument";
    case FP8KV_UNSUPPORTED: return "unsupported shape or dtype";
    case FP8KV_OUT_OF_PAGES: return "out of pages";
    case FP8KV_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FP8KV_HIP_ERROR: return "HIP error";
    default: return "unknown status";
  }
}

int32_t fp8kv_last_hip_error(void) { return fp8kv_detail::g_last_hip_error; }

size_t fp8kv_cache_bytes(const fp8kv_cache_desc* d) {
  if (check_desc(d) != FP8KV_OK) return 0;
  return static_cast<size_t>(d->num_pages) * d->num_kv_heads * tile_bytes(d);
}

int64_t fp8kv_cache_offset(const fp8kv_cache_desc* d, int32_t is_v, int32_t page,
                           int32_t kv_head, int32_t slot, int32_t dim) {
  if (check_desc(d) != FP8KV_OK) return -1;
  if (page < 0 || page >= d->num_pages || kv_head < 0 || kv_head >= d->num_kv_heads ||
      slot < 0 || slot >= kPage || dim < 0 || dim >= kHeadDim)
    return -1;
  const int E = d->cache_dtype == FP8KV_E4M3 ? 1 : 2;
  const int C = 16 / E;
  int f, lane;
  if (is_v) {
    f = 4 * (dim % 8) + slot % 4;
    lane = 16 * (slot / 4) + dim / 8;
  } else {
    f = dim % 32;
    lane = 16 * (dim / 32) + slot;
  }
  const int64_t tile = (static_cast<int64_t>(page) * d->num_kv_heads + kv_head) * tile_bytes(d);
  return tile + (f / C) * 1024 + 16 * lane + E * (f % C);
}

fp8kv_status fp8kv_verify_tags(const int32_t* d_page_table, const uint32_t* d_expected_tags,
                               int32_t max_pages_per_seq, const int32_t* d_ctx_lens,
                               int32_t batch, const uint32_t* d_pool_tags, int32_t num_pages,
                               int32_t page_size, uint8_t* d_abort, hipStream_t stream) {
  if (batch < 0 || max_pages_per_seq < 0 || num_pages < 0 || page_size <= 0)
    return FP8KV_INVALID_ARG;
  if (batch == 0) return FP8KV_OK;
  if (!d_ctx_lens || !d_abort || (max_pages_per_seq > 0 && (!d_page_table || !d_expected_tags)) ||
      (num_pages > 0 && !d_pool_tags))
    return FP8KV_INVALID_ARG;
  VerifyArgs a{d_page_table, d_expected_tags, d_ctx_lens, d_pool_tags, d_abort,
               max_pages_per_seq, num_pages, page_size};
  hipLaunchKernelGGL(verify_tags_kernel, dim3(batch), dim3(kVerifyThreads), 0, stream, a);
  return launched();
}

fp8kv_status fp8kv_append(const fp8kv_cache_desc* desc, void* d_k_cache, void* d_v_cache,
                          const float* d_k_scale, const float* d_v_scale,
                          const uint16_t* d_k_new, const uint16_t* d_v_new, int32_t num_tokens,
                          const int32_t* d_token_seq, const int32_t* d_token_pos,
                          int32_t num_seqs, const int32_t* d_page_table,
                          int32_t max_pages_per_seq, const uint8_t* d_abort,
                          hipStream_t stream) {
  fp8kv_status st = check_desc(desc);
  if (st != FP8KV_OK) return st;
  if (num_tokens < 0 || num_seqs < 0 || max_pages_per_seq < 0) return FP8KV_INVALID_ARG;
  if (num_tokens == 0) return FP8KV_OK;
  if (!d_k_cache || !d_v_cache || !d_k_new || !d_v_new || !d_token_seq || !d_token_pos ||
      !d_page_table)
    return FP8KV_INVALID_ARG;
  if (desc->cache_dtype == FP8KV_E4M3 && (!d_k_scale || !d_v_scale)) return FP8KV_INVALID_ARG;
  AppendArgs a;
  a.k_cache = static_cast<uint8_t*>(d_k_cache);
  a.v_cache = static_cast<uint8_t*>(d_v_cache);
  a.k_scale = d_k_scale;
  a.v_scale = d_v_scale;
  a.k_new = d_k_new;
  a.v_new = d_v_new;
  a.token_seq = d_token_seq;
  a.token_pos = d_token_pos;
  a.page_table = d_page_table;
  a.abort = d_abort;
  a.page_stride = static_cast<int64_t>(desc->num_kv_heads) * tile_bytes(desc);
  a.total_items = static_cast<int64_t>(num_tokens) * desc->num_kv_heads * (kHeadDim / 4);
  a.num_seqs = num_seqs;
  a.max_pages = max_pages_per_seq;
  a.num_pages = desc->num_pages;
  a.Hkv = desc->num_kv_heads;
  // a grid-stride kernel: at most kAppendMaxBlocks workgroups of 256 threads
  const int64_t need = (a.total_items + 255) / 256;
  const int64_t blocks = need < kAppendMaxBlocks ? need : kAppendMaxBlocks;
  if (desc->cache_dtype == FP8KV_E4M3)
    hipLaunchKernelGGL(append_kernel<FP8KV_E4M3>, dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<FP8KV_BF16>, dim3(blocks), dim3(256), 0, stream, a);
  return launched();
}

int32_t fp8kv_decode_num_workers(int32_t requested) {
  if (requested < 0) return -1;
  int32_t w = requested > 0 ? requested : device_workers();
  if (w <= 0) return -1;
  return (w + kWaves - 1) / kWaves * kWaves;
}

}  // extern "C"

namespace {

size_t decode_workspace(const fp8kv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                        int32_t q_len, int32_t num_workers) {
  if (check_desc(desc) != FP8KV_OK || batch < 0 || num_q_heads <= 0 || q_len <= 0 ||
      num_q_heads % desc->num_kv_heads != 0 ||
      num_q_heads / desc->num_kv_heads * q_len > kMaxGroup)
    return 0;
  const int32_t w = fp8kv_decode_num_workers(num_workers);
  if (w <= 0) return 0;
  return workspace_layout(batch, num_q_heads, desc->num_kv_heads, q_len, w).total;
}

// Checks one decode call's arguments and fills its kernel arguments (the
// whole table from token 0, no log-sum-exp output).
fp8kv_status decode_setup(const fp8kv_cache_desc* desc, const void* d_k_cache,
                          const void* d_v_cache, const float* d_k_scale, const float* d_v_scale,
                          const uint16_t* d_q, int32_t num_q_heads, int32_t q_len,
                          const int32_t* d_page_table, int32_t max_pages_per_seq,
                          const int32_t* d_ctx_lens, int32_t batch, float sm_scale,
                          const uint8_t* d_abort, void* d_out, int32_t out_dtype,
                          int32_t num_workers, void* d_workspace, size_t workspace_bytes,
                          DecodeArgs& a, int32_t& workers) {
  fp8kv_status st = check_desc(desc);
  if (st != FP8KV_OK) return st;
  if (batch < 0 || max_pages_per_seq < 0 || num_q_heads <= 0 || num_workers < 0 || q_len <= 0)
    return FP8KV_INVALID_ARG;
  if (num_q_heads % desc->num_kv_heads != 0) return FP8KV_UNSUPPORTED;
  const int G = num_q_heads / desc->num_kv_heads;
  // the (query, head) pairs of a kv-head fill one or two 16-column MFMA tiles
  if (G * q_len > kMaxGroup || batch > kMaxBatch) return FP8KV_UNSUPPORTED;
  // the work split's prefix sums are 32-bit: each request counts at most the
  // table's width in pages plus its segments' fixed items
  if (static_cast<int64_t>(batch) * (static_cast<int64_t>(max_pages_per_seq) + kPieceItems) >
      static_cast<int64_t>(INT32_MAX))
    return FP8KV_UNSUPPORTED;
  if (out_dtype != FP8KV_OUT_BF16 && out_dtype != FP8KV_OUT_F32) return FP8KV_INVALID_ARG;
  if (batch == 0) return FP8KV_OK;
  if (!d_k_cache || !d_v_cache || !d_q || !d_ctx_lens || !d_out ||
      (max_pages_per_seq > 0 && !d_page_table))
    return FP8KV_INVALID_ARG;
  if (desc->cache_dtype == FP8KV_E4M3 && (!d_k_scale || !d_v_scale)) return FP8KV_INVALID_ARG;
  workers = fp8kv_decode_num_workers(num_workers);
  if (workers <= 0) return FP8KV_HIP_ERROR;
  const WorkspaceLayout L =
      workspace_layout(batch, num_q_heads, desc->num_kv_heads, q_len, workers);
  if (!d_workspace || workspace_bytes < L.total) return FP8KV_WORKSPACE_TOO_SMALL;
  a.k_cache = static_cast<const uint8_t*>(d_k_cache);
  a.v_cache = static_cast<const uint8_t*>(d_v_cache);
  // a BF16 cache holds the values themselves: no scales
  a.k_scale = desc->cache_dtype == FP8KV_E4M3 ? d_k_scale : nullptr;
  a.v_scale = desc->cache_dtype == FP8KV_E4M3 ? d_v_scale : nullptr;
  a.q = d_q;
  a.page_table = d_page_table;
  a.ctx_lens = d_ctx_lens;
  a.abort = d_abort;
  a.out = d_out;
  char* ws = static_cast<char*>(d_workspace);
  a.ws_o = reinterpret_cast<float*>(ws + L.o);
  a.ws_ml = reinterpret_cast<float*>(ws + L.ml);
  a.ws_pre = reinterpret_cast<int32_t*>(ws + L.pre);
  a.lse = nullptr;
  a.page_stride = static_cast<int64_t>(desc->num_kv_heads) * tile_bytes(desc);
  a.batch = batch;
  a.max_pages = max_pages_per_seq;
  a.num_pages = desc->num_pages;
  a.Hq = num_q_heads;
  a.Hkv = desc->num_kv_heads;
  a.G = G;
  a.qlen = q_len;
  a.C = G * q_len;
  a.out_f32 = out_dtype == FP8KV_OUT_F32 ? 1 : 0;
  a.sm_scale = sm_scale;
  return FP8KV_OK;
}

// The decode kernel and its merge pass.
// Workgroups of the decode grid.
int64_t decode_grid(const DecodeArgs& a, int32_t workers, int32_t num_workers) {
  const int segs = a.batch * a.Hkv;
  // More than 16 (query, head) columns: two column tiles, 2 waves per SIMD
  // instead of 3, so the default grid holds 2/3 as many workgroups.  With the
  // default grid, long segments shared by many workgroups leave the merge a
  // long chain of pieces per segment (one request of 8k tokens: ~100), which
  // costs more than the extra workgroups gain: the default grid is capped at
  // kDefaultPiecesPerSegment workgroups per segment.  An explicit worker
  // count is used as given.
  const bool two_tiles = a.C > kTileCols;
  int blocks = workers / kWaves;
  if (num_workers == 0 && two_tiles) blocks = blocks / 3 * 2;
  if (num_workers == 0 && static_cast<int64_t>(kDefaultPiecesPerSegment) * segs < blocks)
    blocks = kDefaultPiecesPerSegment * segs;
  return blocks;
}

// The merge pass after a decode grid of `blocks` workgroups.
fp8kv_status merge_launch(const DecodeArgs& a, int64_t blocks, hipStream_t stream) {
  const int segs = a.batch * a.Hkv;
  // at least 256 threads, one per (column, 4 dims) pair up to 1024
  const int pairs = a.C * (kHeadDim / 4);
  const int flat_threads =
      pairs < 256 ? 256 : (pairs > kMergeFlatMaxThreads ? kMergeFlatMaxThreads : pairs);
  const dim3 mgrid(segs < 1024 ? segs : 1024);
  if (blocks >= static_cast<int64_t>(kMergeGroupedMinPieces) * segs)
    hipLaunchKernelGGL(merge_grouped_kernel, mgrid, dim3(kMergeGroupedThreads), 0, stream, a,
                       blocks);
  else
    hipLaunchKernelGGL(merge_flat_kernel, mgrid, dim3(flat_threads), 0, stream, a, blocks);
  return launched();
}

fp8kv_status decode_launch(const DecodeArgs& a, int32_t cache_dtype, int32_t workers,
                           int32_t num_workers, hipStream_t stream) {
  const bool two_tiles = a.C > kTileCols;
  const int64_t blocks = decode_grid(a, workers, num_workers);
  if (cache_dtype == FP8KV_E4M3) {
    if (two_tiles)
      hipLaunchKernelGGL((decode_kernel<FP8KV_E4M3, FP8KV_DEPTH_E4M3_2T, 2>), dim3(blocks),
                         dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<FP8KV_E4M3, FP8KV_DEPTH_E4M3, 1>), dim3(blocks),
                         dim3(kThreads), 0, stream, a);
  } else {
    if (two_tiles)
      hipLaunchKernelGGL((decode_kernel<FP8KV_BF16, FP8KV_DEPTH_BF16_2T, 2>), dim3(blocks),
                         dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<FP8KV_BF16, FP8KV_DEPTH_BF16, 1>), dim3(blocks),
                         dim3(kThreads), 0, stream, a);
  }
  fp8kv_status st = launched();
  if (st != FP8KV_OK) return st;
  return merge_launch(a, blocks, stream);
}

fp8kv_status decode_impl(const fp8kv_cache_desc* desc, const void* d_k_cache,
                         const void* d_v_cache, const float* d_k_scale, const float* d_v_scale,
                         const uint16_t* d_q, int32_t num_q_heads, int32_t q_len,
                         const int32_t* d_page_table, int32_t max_pages_per_seq,
                         const int32_t* d_ctx_lens, int32_t batch, float sm_scale,
                         const uint8_t* d_abort, void* d_out, int32_t out_dtype,
                         int32_t num_workers, void* d_workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  DecodeArgs a;
  int32_t workers = 0;
  const fp8kv_status st = decode_setup(desc, d_k_cache, d_v_cache, d_k_scale, d_v_scale, d_q,
                                       num_q_heads, q_len, d_page_table, max_pages_per_seq,
                                       d_ctx_lens, batch, sm_scale, d_abort, d_out, out_dtype,
                                       num_workers, d_workspace, workspace_bytes, a, workers);
  if (st != FP8KV_OK || batch == 0) return st;
  return decode_launch(a, desc->cache_dtype, workers, num_workers, stream);
}

// ---- the shared-prompt call ------------------------------------------------
// page ranges of a prompt: enough workgroups to fill the device, at least
// kPrefixMinPages pages each
constexpr int kPrefixMinPages = 8;

struct SharedLayout {
  size_t o, ml, suf_out, suf_lse, view_pt, view_ctx, ok, total;
  PromptGroups pg;
  int64_t grid;
  int nt;  // column tiles per prefix wave
};

// Checks the group description (host arrays) and lays out the workspace.
// Groups with an empty prompt are dropped (their requests attend as usual).
fp8kv_status shared_layout(int32_t batch, int32_t Hq, int32_t Hkv, int32_t max_pages,
                           int32_t num_groups, const int32_t* h_group_start,
                           const int32_t* h_prefix_len, int32_t workers, SharedLayout& L) {
  if (num_groups < 0 || num_groups > kMaxPromptGroups || (num_groups > 0 && (!h_group_start ||
                                                                           !h_prefix_len)))
    return FP8KV_INVALID_ARG;
  if (num_groups > 0 && (h_group_start[0] < 0 || h_group_start[num_groups] > batch))
    return FP8KV_INVALID_ARG;
  const int32_t G = Hq / Hkv;
  PromptGroups& pg = L.pg;
  pg.n = 0;
  pg.wg_start[0] = 0;
  pg.part_base[0] = 0;
  int64_t wgs = 0, part = 0;
  // two column tiles per prefix wave when every group has at least two per
  // wave of a workgroup (two waves per SIMD then, so 2/3 as many resident)
  L.nt = 2;
  for (int k = 0; k < num_groups; ++k) {
    const int64_t r = static_cast<int64_t>(h_group_start[k + 1]) - h_group_start[k];
    if (r > 0 && h_prefix_len[k] > 0 && (r * G + kTileCols - 1) / kTileCols < 2 * kWaves) L.nt = 1;
  }
  const int64_t resident = L.nt == 1 ? workers / kWaves : workers * 2 / 3 / kWaves;
  for (int k = 0; k < num_groups; ++k) {
    const int32_t r0 = h_group_start[k], r1 = h_group_start[k + 1], len = h_prefix_len[k];
    if (r1 < r0 || len < 0 || len % kPage != 0 || len / kPage > max_pages)
      return FP8KV_INVALID_ARG;
    if (len == 0 || r1 == r0) continue;
    const int m = pg.n++;
    pg.req_start[m] = r0;
    pg.req_end[m] = r1;
    pg.prefix_len[m] = len;
    const int32_t P0 = len / kPage;
    pg.tiles[m] = static_cast<int32_t>((static_cast<int64_t>(r1 - r0) * G + kTileCols - 1) / kTileCols);
    pg.blocks[m] = (pg.tiles[m] + kWaves * L.nt - 1) / (kWaves * L.nt);
    const int64_t base = static_cast<int64_t>(Hkv) * pg.blocks[m];
    const int64_t want = (resident + base - 1) / base;
    const int64_t most = P0 / kPrefixMinPages > 1 ? P0 / kPrefixMinPages : 1;
    pg.S[m] = static_cast<int32_t>(want < 1 ? 1 : (want < most ? want : most));
    pg.wg_start[m] = static_cast<int32_t>(wgs);
    pg.part_base[m] = part;
    wgs += base * pg.S[m];
    part += static_cast<int64_t>(pg.S[m]) * (r1 - r0) * Hq;
    if (wgs > 0x7FFFFFFF) return FP8KV_UNSUPPORTED;
  }
  pg.wg_start[pg.n] = static_cast<int32_t>(wgs);
  pg.part_base[pg.n] = part;
  L.grid = wgs;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = static_cast<size_t>(batch) * Hq;
  L.o = up(workspace_layout(batch, Hq, Hkv, 1, workers).total);
  L.ml = L.o + up(static_cast<size_t>(part) * kHeadDim * sizeof(float));
  L.suf_out = L.ml + up(static_cast<size_t>(part) * 2 * sizeof(float));
  L.suf_lse = L.suf_out + up(rows * kHeadDim * sizeof(float));
  L.view_pt = L.suf_lse + up(rows * sizeof(float));
  L.view_ctx = L.view_pt + up(static_cast<size_t>(batch) * max_pages * sizeof(int32_t));
  L.ok = L.view_ctx + up(static_cast<size_t>(batch) * sizeof(int32_t));
  L.total = L.ok + up(static_cast<size_t>(batch));
  return FP8KV_OK;
}

fp8kv_status shared_impl(const fp8kv_cache_desc* desc, const void* d_k_cache,
                         const void* d_v_cache, const float* d_k_scale, const float* d_v_scale,
                         const uint16_t* d_q, int32_t num_q_heads, int32_t num_groups,
                         const int32_t* h_group_start, const int32_t* h_prefix_len,
                         const int32_t* d_page_table, int32_t max_pages_per_seq,
                         const int32_t* d_ctx_lens, int32_t batch, float sm_scale,
                         const uint8_t* d_abort, void* d_out, int32_t out_dtype,
                         int32_t num_workers, void* d_workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  // the plain call's checks first (the workspace size once the groups are known)
  DecodeArgs a;
  int32_t workers = 0;
  fp8kv_status st = decode_setup(desc, d_k_cache, d_v_cache, d_k_scale, d_v_scale, d_q,
                                 num_q_heads, 1, d_page_table, max_pages_per_seq, d_ctx_lens,
                                 batch, sm_scale, d_abort, d_out, out_dtype, num_workers,
                                 d_workspace, d_workspace ? SIZE_MAX : 0, a, workers);
  if (st != FP8KV_OK) return st;
  SharedLayout L;
  st = shared_layout(batch, num_q_heads, desc->num_kv_heads, max_pages_per_seq, num_groups,
                     h_group_start, h_prefix_len, workers, L);
  if (st != FP8KV_OK || batch == 0) return st;
  const size_t need = L.pg.n == 0
                          ? workspace_layout(batch, num_q_heads, desc->num_kv_heads, 1, workers).total
                          : L.total;
  if (workspace_bytes < need) return FP8KV_WORKSPACE_TOO_SMALL;
  if (L.pg.n == 0) return decode_launch(a, desc->cache_dtype, workers, num_workers, stream);
  char* ws = static_cast<char*>(d_workspace);

  PrefixArgs pa;
  pa.k_cache = a.k_cache;
  pa.v_cache = a.v_cache;
  pa.k_scale = a.k_scale;
  pa.v_scale = a.v_scale;
  pa.q = d_q;
  pa.page_table = d_page_table;
  pa.ctx_lens = d_ctx_lens;
  pa.view_pt = reinterpret_cast<int32_t*>(ws + L.view_pt);
  pa.view_ctx = reinterpret_cast<int32_t*>(ws + L.view_ctx);
  pa.member_ok = reinterpret_cast<uint8_t*>(ws + L.ok);
  pa.ws_o = reinterpret_cast<float*>(ws + L.o);
  pa.ws_ml = reinterpret_cast<float*>(ws + L.ml);
  pa.page_stride = a.page_stride;
  pa.batch = batch;
  pa.Hq = num_q_heads;
  pa.Hkv = a.Hkv;
  pa.G = a.G;
  pa.max_pages = max_pages_per_seq;
  pa.num_pages = desc->num_pages;
  pa.sm_scale = sm_scale;
  pa.pg = L.pg;

  // the own tokens: the decode past each request's prompt pages, f32 rows
  // with their log-sum-exp, into the workspace
  int64_t fused_decode_grid = 0;
  a.out = ws + L.suf_out;
  a.out_f32 = 1;
  a.lse = reinterpret_cast<float*>(ws + L.suf_lse);
  if (desc->cache_dtype == FP8KV_E4M3 && a.C <= kTileCols) {
    // one grid: the prompt pass, then the decode's workgroups beside it (the
    // decode skips the prompt pages of the original tables itself)
    const int64_t dblocks = decode_grid(a, workers, num_workers) / kFusedDecodeDiv;
    const int64_t d = dblocks < 1 ? 1 : dblocks;
    if (L.grid + d > 0x7FFFFFFF) return FP8KV_UNSUPPORTED;
    if (L.nt == 2)
      hipLaunchKernelGGL(shared_fused_kernel<2>, dim3(L.grid + d), dim3(kThreads), 0, stream, pa,
                         a, static_cast<int32_t>(L.grid), static_cast<int32_t>(d));
    else
      hipLaunchKernelGGL(shared_fused_kernel<1>, dim3(L.grid + d), dim3(kThreads), 0, stream, pa,
                         a, static_cast<int32_t>(L.grid), static_cast<int32_t>(d));
    st = launched();
    fused_decode_grid = d;  // combine_kernel merges the split segments
  } else {
    // the plain decode over materialised views of the tables
    hipLaunchKernelGGL(view_kernel, dim3(batch), dim3(256), 0, stream, pa);
    st = launched();
    if (st != FP8KV_OK) return st;
    a.page_table = pa.view_pt;
    a.ctx_lens = pa.view_ctx;
    if (desc->cache_dtype == FP8KV_E4M3) {
      if (L.nt == 2)
        hipLaunchKernelGGL((prefix_kernel<FP8KV_E4M3, 2>), dim3(L.grid), dim3(kThreads), 0, stream, pa);
      else
        hipLaunchKernelGGL((prefix_kernel<FP8KV_E4M3, 1>), dim3(L.grid), dim3(kThreads), 0, stream, pa);
    } else {
      if (L.nt == 2)
        hipLaunchKernelGGL((prefix_kernel<FP8KV_BF16, 2>), dim3(L.grid), dim3(kThreads), 0, stream, pa);
      else
        hipLaunchKernelGGL((prefix_kernel<FP8KV_BF16, 1>), dim3(L.grid), dim3(kThreads), 0, stream, pa);
    }
    st = launched();
    if (st != FP8KV_OK) return st;
    st = decode_launch(a, desc->cache_dtype, workers, num_workers, stream);
  }
  if (st != FP8KV_OK) return st;

  CombineArgs ca;
  ca.ws_o = pa.ws_o;
  ca.ws_ml = pa.ws_ml;
  ca.suf_out = reinterpret_cast<const float*>(ws + L.suf_out);
  ca.suf_lse = a.lse;
  ca.ctx_lens = d_ctx_lens;
  ca.abort = d_abort;
  ca.member_ok = pa.member_ok;
  ca.v_scale = a.v_scale;
  ca.out = d_out;
  ca.batch = batch;
  ca.Hq = num_q_heads;
  ca.G = a.G;
  ca.max_tokens = static_cast<int64_t>(max_pages_per_seq) * kPage;
  ca.out_f32 = out_dtype == FP8KV_OUT_F32 ? 1 : 0;
  ca.pg = L.pg;
  ca.fold_merge = fused_decode_grid > 0 ? 1 : 0;
  ca.decode_grid = fused_decode_grid;
  ca.decode = a;
  const int64_t threads = static_cast<int64_t>(batch) * num_q_heads * (kHeadDim / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((threads + 255) / 256), dim3(256), 0, stream, ca);
  return launched();
}

}  // namespace

extern "C" {

size_t fp8kv_decode_workspace_size(const fp8kv_cache_desc* desc, int32_t batch,
                                   int32_t num_q_heads, int32_t num_workers) {
  return decode_workspace(desc, batch, num_q_heads, 1, num_workers);
}

size_t fp8kv_decode_workspace_size_q(const fp8kv_cache_desc* desc, int32_t batch,
                                     int32_t num_q_heads, int32_t q_len, int32_t num_workers) {
  return decode_workspace(desc, batch, num_q_heads, q_len, num_workers);
}

size_t fp8kv_decode_workspace_size_shared(const fp8kv_cache_desc* desc, int32_t batch,
                                          int32_t num_q_heads, int32_t max_pages_per_seq,
                                          int32_t num_groups, const int32_t* h_group_start,
                                          const int32_t* h_prefix_len, int32_t num_workers) {
  const size_t plain = decode_workspace(desc, batch, num_q_heads, 1, num_workers);
  if (plain == 0 || max_pages_per_seq < 0) return 0;
  SharedLayout L;
  if (shared_layout(batch, num_q_heads, desc->num_kv_heads, max_pages_per_seq, num_groups,
                    h_group_start, h_prefix_len, fp8kv_decode_num_workers(num_workers),
                    L) != FP8KV_OK)
    return 0;
  return L.pg.n == 0 ? plain : L.total;
}

fp8kv_status fp8kv_decode_attention_shared(
    const fp8kv_cache_desc* desc, const void* d_k_cache, const void* d_v_cache,
    const float* d_k_scale, const float* d_v_scale, const uint16_t* d_q, int32_t num_q_heads,
    int32_t num_groups, const int32_t* h_group_start, const int32_t* h_prefix_len,
    const int32_t* d_page_table, int32_t max_pages_per_seq, const int32_t* d_ctx_lens,
    int32_t batch, float sm_scale, const uint8_t* d_abort, void* d_out, int32_t out_dtype,
    int32_t num_workers, void* d_workspace, size_t workspace_bytes, hipStream_t stream) {
  return shared_impl(desc, d_k_cache, d_v_cache, d_k_scale, d_v_scale, d_q, num_q_heads,
                     num_groups, h_group_start, h_prefix_len, d_page_table, max_pages_per_seq,
                     d_ctx_lens, batch, sm_scale, d_abort, d_out, out_dtype, num_workers,
                     d_workspace, workspace_bytes, stream);
}

fp8kv_status fp8kv_decode_attention(const fp8kv_cache_desc* desc, const void* d_k_cache,
                                    const void* d_v_cache, const float* d_k_scale,
                                    const float* d_v_scale, const uint16_t* d_q,
                                    int32_t num_q_heads, const int32_t* d_page_table,
                                    int32_t max_pages_per_seq, const int32_t* d_ctx_lens,
                                    int32_t batch, float sm_scale, const uint8_t* d_abort,
                                    void* d_out, int32_t out_dtype, int32_t num_workers,
                                    void* d_workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return decode_impl(desc, d_k_cache, d_v_cache, d_k_scale, d_v_scale, d_q, num_q_heads, 1,
                     d_page_table, max_pages_per_seq, d_ctx_lens, batch, sm_scale, d_abort,
                     d_out, out_dtype, num_workers, d_workspace, workspace_bytes, stream);
}

// Scratch address on the current device, looked up once per device with that
// device current; nullptr (and the HIP error recorded) if the lookup fails.
static void* device_scratch() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fp8kv_detail::record_hip_error(static_cast<int32_t>(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    fp8kv_detail::record_hip_error(static_cast<int32_t>(e != hipSuccess ? e : hipErrorUnknown));
    return nullptr;
  }
  ptrs[dev].store(p, std::memory_order_release);
  return p;
}

fp8kv_status fp8kv_decode_attention_noalloc(const fp8kv_cache_desc* desc, const void* d_k_cache,
                                            const void* d_v_cache, const float* d_k_scale,
                                            const float* d_v_scale, const uint16_t* d_q,
                                            int32_t num_q_heads, const int32_t* d_page_table,
                                            int32_t max_pages_per_seq, const int32_t* d_ctx_lens,
                                            int32_t batch, float sm_scale, const uint8_t* d_abort,
                                            void* d_out, int32_t out_dtype, int32_t num_workers,
                                            hipStream_t stream) {
  // the same checks as the workspace form, then the size against the scratch
  const size_t need = decode_workspace(desc, batch, num_q_heads, 1, num_workers);
  if (batch > 0 && need > FP8KV_NOALLOC_SCRATCH_BYTES) return FP8KV_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (batch > 0 && need > 0) {
    ws = device_scratch();
    if (!ws) return FP8KV_HIP_ERROR;
  }
  return decode_impl(desc, d_k_cache, d_v_cache, d_k_scale, d_v_scale, d_q, num_q_heads, 1,
                     d_page_table, max_pages_per_seq, d_ctx_lens, batch, sm_scale, d_abort,
                     d_out, out_dtype, num_workers, ws, ws ? FP8KV_NOALLOC_SCRATCH_BYTES : 0,
                     stream);
}

fp8kv_status fp8kv_decode_attention_q(const fp8kv_cache_desc* desc, const void* d_k_cache,
                                      const void* d_v_cache, const float* d_k_scale,
                                      const float* d_v_scale, const uint16_t* d_q,
                                      int32_t num_q_heads, int32_t q_len,
                                      const int32_t* d_page_table, int32_t max_pages_per_seq,
                                      const int32_t* d_ctx_lens, int32_t batch, float sm_scale,
                                      const uint8_t* d_abort, void* d_out, int32_t out_dtype,
                                      int32_t num_workers, void* d_workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(desc, d_k_cache, d_v_cache, d_k_scale, d_v_scale, d_q, num_q_heads, q_len,
                     d_page_table, max_pages_per_seq, d_ctx_lens, batch, sm_scale, d_abort,
                     d_out, out_dtype, num_workers, d_workspace, workspace_bytes, stream);
}

fp8kv_status fp8kv_verify_append_q(const fp8kv_cache_desc* desc, void* d_k_cache, void* d_v_cache,
                                 const float* d_k_scale, const float* d_v_scale,
                                 const uint16_t* d_k_new, const uint16_t* d_v_new,
                                 const int32_t* d_new_pos, int32_t q_len, const int32_t* d_page_table,
                                 const uint32_t* d_expected_tags, int32_t max_pages_per_seq,
                                 const int32_t* d_ctx_lens, int32_t batch,
                                 const uint32_t* d_pool_tags, uint8_t* d_abort,
                                 hipStream_t stream) {
  fp8kv_status st = check_desc(desc);
  if (st != FP8KV_OK) return st;
  if (batch < 0 || max_pages_per_seq < 0 || q_len <= 0) return FP8KV_INVALID_ARG;
  if (batch == 0) return FP8KV_OK;
  if (!d_k_cache || !d_v_cache || !d_k_new || !d_v_new || !d_new_pos || !d_ctx_lens ||
      !d_abort || !d_pool_tags || (max_pages_per_seq > 0 && (!d_page_table || !d_expected_tags)))
    return FP8KV_INVALID_ARG;
  if (desc->cache_dtype == FP8KV_E4M3 && (!d_k_scale || !d_v_scale)) return FP8KV_INVALID_ARG;
  if (desc->num_kv_heads * (kHeadDim / 4) > kVerifyThreads) return FP8KV_UNSUPPORTED;
  VerifyAppendArgs a;
  a.v = VerifyArgs{d_page_table, d_expected_tags, d_ctx_lens, d_pool_tags, d_abort,
                   max_pages_per_seq, desc->num_pages, kPage};
  a.w.k_cache = static_cast<uint8_t*>(d_k_cache);
  a.w.v_cache = static_cast<uint8_t*>(d_v_cache);
  a.w.k_scale = d_k_scale;
  a.w.v_scale = d_v_scale;
  a.w.k_new = d_k_new;
  a.w.v_new = d_v_new;
  a.w.token_seq = nullptr;
  a.w.token_pos = nullptr;
  a.w.page_table = d_page_table;
  a.w.abort = nullptr;
  a.w.page_stride = static_cast<int64_t>(desc->num_kv_heads) * tile_bytes(desc);
  a.w.total_items = static_cast<int64_t>(batch) * desc->num_kv_heads * 8;
  a.w.num_seqs = batch;
  a.w.max_pages = max_pages_per_seq;
  a.w.num_pages = desc->num_pages;
  a.w.Hkv = desc->num_kv_heads;
  a.new_pos = d_new_pos;
  a.qlen = q_len;
  if (desc->cache_dtype == FP8KV_E4M3)
    hipLaunchKernelGGL(verify_append_kernel<FP8KV_E4M3>, dim3(batch), dim3(kVerifyThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(verify_append_kernel<FP8KV_BF16>, dim3(batch), dim3(kVerifyThreads), 0,
                       stream, a);
  return launched();
}

fp8kv_status fp8kv_verify_append(const fp8kv_cache_desc* desc, void* d_k_cache, void* d_v_cache,
                                 const float* d_k_scale, const float* d_v_scale,
                                 const uint16_t* d_k_new, const uint16_t* d_v_new,
                                 const int32_t* d_new_pos, const int32_t* d_page_table,
                                 const uint32_t* d_expected_tags, int32_t max_pages_per_seq,
                                 const int32_t* d_ctx_lens, int32_t batch,
                                 const uint32_t* d_pool_tags, uint8_t* d_abort,
                                 hipStream_t stream) {
  return fp8kv_verify_append_q(desc, d_k_cache, d_v_cache, d_k_scale, d_v_scale, d_k_new, d_v_new,
                               d_new_pos, 1, d_page_table, d_expected_tags, max_pages_per_seq,
                               d_ctx_lens, batch, d_pool_tags, d_abort, stream);
}

int32_t fp8kv_debug_read_sink_words(void) { return device_workers() / kWaves * 256; }

fp8kv_status fp8kv_debug_read_bandwidth(const void* d_buf, size_t bytes, uint32_t* d_sink,
                                        hipStream_t stream) {
  if (!d_buf || !d_sink || bytes % 16 != 0) return FP8KV_INVALID_ARG;
  if (bytes == 0) return FP8KV_OK;
  const int32_t words = fp8kv_debug_read_sink_words();
  if (words <= 0) return FP8KV_HIP_ERROR;
  hipLaunchKernelGGL(read_bandwidth_kernel, dim3(words / 256), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(d_buf), static_cast<int64_t>(bytes), d_sink);
  return launched();
}

fp8kv_status fp8kv_debug_convert_e4m3(const uint8_t* d_codes, float* d_out, int32_t n,
                                      int32_t which, hipStream_t stream) {
  if (!d_codes || !d_out || n < 0 || n % 4 != 0 || (which != 0 && which != 1))
    return FP8KV_INVALID_ARG;
  if (n == 0) return FP8KV_OK;
  const int blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(debug_convert_kernel, dim3(blocks), dim3(256), 0, stream, d_codes, d_out, n,
                     which);
  return launched();
}

}  // extern "C"
