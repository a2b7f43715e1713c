// fp8kv page pool: free list and per-page generation tags (host side).
//
// The integrity scheme tags every physical KV page; the tag changes each time
// the page is handed out again, and a request remembers the (page, tag) pairs
// it was given (Cloudflare, "Smaller, faster, safer: running Kimi and GLM at
// scale", integrity section; commentary page, "Giving Every Physical Cache
// Page a 'Generation Number'").  Here: a uint32 counter per page, seeded
// random at creation, +1 (mod 2^32) on every allocation; freed pages are
// reused first-in first-out so a stale mapping lives as long as possible
// before its page is reissued (and then it is caught by the tag).
//
// Pages can be shared (a common prefix mapped by several requests, the cache
// reuse the same pages warn widens the reach of a bad mapping): every holder
// records the same tag; a page goes back to the free list when its last
// holder releases it, and only its next allocation changes the tag.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "fp8kv.h"
#include "fp8kv_internal.h"

struct fp8kv_pool {
  int32_t n = 0;
  std::vector<uint32_t> tags;
  std::vector<int32_t> refs;   // holders of the page (0: free)
  std::vector<uint8_t> seen;   // scratch of one call: duplicate ids
  std::vector<int32_t> ring;  // free ids, FIFO
  int64_t head = 0;           // index of the oldest free id
  int64_t count = 0;          // free ids in the ring
  int32_t dirty_lo = 0, dirty_hi = -1;
  uint32_t* staging = nullptr;  // pinned, n entries
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
};

namespace {

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void mark_dirty(fp8kv_pool* p, int32_t id) {
  if (p->dirty_hi < p->dirty_lo) {
    p->dirty_lo = p->dirty_hi = id;
  } else {
    if (id < p->dirty_lo) p->dirty_lo = id;
    if (id > p->dirty_hi) p->dirty_hi = id;
  }
}

fp8kv_status fail(hipError_t e) {
  fp8kv_detail::record_hip_error(static_cast<int32_t>(e));
  return FP8KV_HIP_ERROR;
}

}  // namespace

extern "C" {

fp8kv_status fp8kv_pool_create(int32_t num_pages, uint64_t seed, fp8kv_pool** out) {
  if (!out || num_pages <= 0) return FP8KV_INVALID_ARG;
  fp8kv_pool* p = new (std::nothrow) fp8kv_pool();
  if (!p) return FP8KV_INVALID_ARG;
  p->n = num_pages;
  p->tags.resize(num_pages);
  p->refs.assign(num_pages, 0);
  p->seen.assign(num_pages, 0);
  p->ring.resize(num_pages);
  uint64_t s = seed;
  for (int32_t i = 0; i < num_pages; ++i) {
    p->tags[i] = static_cast<uint32_t>(splitmix64(s) >> 32);
    p->ring[i] = i;
  }
  p->head = 0;
  p->count = num_pages;
  p->dirty_lo = 0;
  p->dirty_hi = num_pages - 1;  // the first sync uploads every tag
  *out = p;
  return FP8KV_OK;
}

void fp8kv_pool_destroy(fp8kv_pool* p) {
  if (!p) return;
  if (p->upload_done) {
    if (p->upload_pending) (void)hipEventSynchronize(p->upload_done);
    (void)hipEventDestroy(p->upload_done);
  }
  if (p->staging) (void)hipHostFree(p->staging);
  delete p;
}

fp8kv_status fp8kv_pool_alloc(fp8kv_pool* p, int32_t n, int32_t* ids, uint32_t* tags) {
  if (!p || n < 0 || (n > 0 && (!ids || !tags))) return FP8KV_INVALID_ARG;
  if (n > p->count) return FP8KV_OUT_OF_PAGES;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t id = p->ring[p->head];
    p->head = (p->head + 1) % p->n;
    --p->count;
    p->tags[id] += 1u;  // a new lifetime of this page
    p->refs[id] = 1;
    mark_dirty(p, id);
    ids[k] = id;
    tags[k] = p->tags[id];
  }
  return FP8KV_OK;
}

namespace {

// Every id in range, currently held, listed once (and, when adding a holder,
// not at the counter's limit); on failure nothing is marked.
bool valid_held_list(fp8kv_pool* p, int32_t n, const int32_t* ids, bool adding) {
  bool ok = true;
  int32_t k = 0;
  for (; k < n; ++k) {
    const int32_t id = ids[k];
    if (id < 0 || id >= p->n || p->refs[id] <= 0 || p->seen[id] ||
        (adding && p->refs[id] == INT32_MAX)) {
      ok = false;
      break;
    }
    p->seen[id] = 1;
  }
  for (int32_t j = 0; j < k; ++j) p->seen[ids[j]] = 0;
  return ok;
}

}  // namespace

fp8kv_status fp8kv_pool_share(fp8kv_pool* p, int32_t n, const int32_t* ids) {
  if (!p || n < 0 || (n > 0 && !ids)) return FP8KV_INVALID_ARG;
  if (!valid_held_list(p, n, ids, true)) return FP8KV_INVALID_ARG;
  for (int32_t k = 0; k < n; ++k) ++p->refs[ids[k]];
  return FP8KV_OK;
}

fp8kv_status fp8kv_pool_free(fp8kv_pool* p, int32_t n, const int32_t* ids) {
  if (!p || n < 0 || (n > 0 && !ids)) return FP8KV_INVALID_ARG;
  if (!valid_held_list(p, n, ids, false)) return FP8KV_INVALID_ARG;  // all-or-nothing
  for (int32_t k = 0; k < n; ++k) {
    const int32_t id = ids[k];
    if (--p->refs[id] > 0) continue;  // other holders keep it
    p->ring[(p->head + p->count) % p->n] = id;
    ++p->count;
  }
  return FP8KV_OK;
}

int32_t fp8kv_pool_refcount(const fp8kv_pool* p, int32_t id) {
  if (!p || id < 0 || id >= p->n) return -1;
  return p->refs[id];
}

uint32_t fp8kv_pool_tag(const fp8kv_pool* p, int32_t id) {
  if (!p || id < 0 || id >= p->n) return 0;
  return p->tags[id];
}

int32_t fp8kv_pool_num_free(const fp8kv_pool* p) {
  return p ? static_cast<int32_t>(p->count) : 0;
}

fp8kv_status fp8kv_pool_read_tags(const fp8kv_pool* p, uint32_t* h_tags) {
  if (!p || !h_tags) return FP8KV_INVALID_ARG;
  std::memcpy(h_tags, p->tags.data(), sizeof(uint32_t) * p->n);
  return FP8KV_OK;
}

fp8kv_status fp8kv_pool_sync(fp8kv_pool* p, uint32_t* d_tags, hipStream_t stream) {
  if (!p || !d_tags) return FP8KV_INVALID_ARG;
  if (p->dirty_hi < p->dirty_lo) return FP8KV_OK;
  hipError_t e;
  if (!p->staging) {
    e = hipHostMalloc(reinterpret_cast<void**>(&p->staging), sizeof(uint32_t) * p->n,
                      hipHostMallocDefault);
    if (e != hipSuccess) {
      p->staging = nullptr;
      return fail(e);
    }
    e = hipEventCreateWithFlags(&p->upload_done, hipEventDisableTiming);
    if (e != hipSuccess) return fail(e);
  }
  if (p->upload_pending) {
    e = hipEventSynchronize(p->upload_done);  // staging still being read
    if (e != hipSuccess) return fail(e);
    p->upload_pending = false;
  }
  const int32_t lo = p->dirty_lo, cnt = p->dirty_hi - p->dirty_lo + 1;
  std::memcpy(p->staging + lo, p->tags.data() + lo, sizeof(uint32_t) * cnt);
  e = hipMemcpyAsync(d_tags + lo, p->staging + lo, sizeof(uint32_t) * cnt,
                     hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(e);
  e = hipEventRecord(p->upload_done, stream);
  if (e != hipSuccess) return fail(e);
  p->upload_pending = true;
  p->dirty_lo = 0;
  p->dirty_hi = -1;
  return FP8KV_OK;
}

}  // extern "C"
