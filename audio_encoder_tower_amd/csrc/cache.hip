// Embeddings cache: encoder outputs kept on the device under caller-given
// content keys, so a clip the encoder has already seen is served by a copy.
//
// Serving stacks keep such a cache next to a separately scheduled encoder
// (the "Multimodal Embeddings Cache" and "Multimodal Encoder Side Stream" of
// TRT-LLM, cited by the "Kimi-Audio-7B-Instruct" and "Qwen2-Audio-7B-Instruct"
// records, (1) under SERVICEABILITY JOIN). Here:
//   - the pool is one device allocation of `capacity` slots of `entry_bytes`
//     (one clip's output), made at create time; lookups and inserts allocate
//     nothing and only enqueue device-to-device copies on the caller's stream;
//   - slots are recycled least recently used first;
//   - every slot carries an event recorded after its last copy; the next copy
//     touching the slot first waits for that event on its own stream, so an
//     insert on one stream and a lookup on another are ordered;
//   - a mutex makes the bookkeeping safe for concurrent host threads.
#include <cstring>
#include <list>
#include <mutex>
#include <unordered_map>
#include <vector>

#include <hip/hip_runtime.h>

#include "aenc.h"

namespace aenc {
void set_kernel_error(const char* msg);
}

struct aenc_cache {
  int64_t entry_bytes = 0;
  int64_t capacity = 0;
  char* pool = nullptr;
  std::vector<hipEvent_t> last_use;          // per slot
  std::vector<uint64_t> slot_key;
  std::vector<std::list<int64_t>::iterator> where;
  std::list<int64_t> lru;                    // front: most recently used slot
  std::unordered_map<uint64_t, int64_t> index;
  std::vector<int64_t> free_slots;
  int64_t hits = 0, misses = 0, inserts = 0, evictions = 0;
  std::mutex mu;
};

namespace {

void cache_error(const char* msg) { aenc::set_kernel_error(msg); }

void touch(aenc_cache* c, int64_t slot) {
  c->lru.erase(c->where[slot]);
  c->lru.push_front(slot);
  c->where[slot] = c->lru.begin();
}

// Copy `bytes` between device buffers on `s`, ordered after the slot's last use.
hipError_t slot_copy(aenc_cache* c, int64_t slot, void* dst, const void* src, hipStream_t s) {
  hipError_t e = hipStreamWaitEvent(s, c->last_use[slot], 0);
  if (e == hipSuccess) e = hipMemcpyAsync(dst, src, (size_t)c->entry_bytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(c->last_use[slot], s);
  return e;
}

}  // namespace

extern "C" aenc_cache* aenc_cache_create(int64_t entry_bytes, int64_t capacity) {
  if (entry_bytes <= 0 || capacity <= 0 || entry_bytes > ((int64_t)1 << 40) / capacity) {
    cache_error("cache: entry_bytes and capacity must be positive (and their product at most 1 TiB)");
    return nullptr;
  }
  auto* c = new aenc_cache;
  c->entry_bytes = entry_bytes;
  c->capacity = capacity;
  hipError_t e = hipMalloc(&c->pool, (size_t)(entry_bytes * capacity));
  c->last_use.assign(capacity, nullptr);
  for (int64_t i = 0; e == hipSuccess && i < capacity; ++i)
    e = hipEventCreateWithFlags(&c->last_use[i], hipEventDisableTiming);
  if (e != hipSuccess) {
    cache_error(hipGetErrorString(e));
    aenc_cache_destroy(c);
    return nullptr;
  }
  c->slot_key.assign(capacity, 0);
  c->where.resize(capacity);
  c->free_slots.reserve(capacity);
  for (int64_t i = capacity - 1; i >= 0; --i) c->free_slots.push_back(i);
  return c;
}

extern "C" void aenc_cache_destroy(aenc_cache* c) {
  if (!c) return;
  for (hipEvent_t ev : c->last_use)
    if (ev) (void)hipEventDestroy(ev);
  if (c->pool) (void)hipFree(c->pool);
  delete c;
}

extern "C" int aenc_cache_contains(aenc_cache* c, uint64_t key) {
  if (!c) { cache_error("cache is NULL"); return AENC_E_INVAL; }
  std::lock_guard<std::mutex> g(c->mu);
  return c->index.count(key) ? 1 : 0;
}

namespace {
// Lookup with the cache's mutex held: 1 hit (copy enqueued), 0 miss, < 0 error.
int lookup_locked(aenc_cache* c, uint64_t key, void* dst, hipStream_t stream) {
  auto it = c->index.find(key);
  if (it == c->index.end()) {
    ++c->misses;
    return 0;
  }
  const int64_t slot = it->second;
  touch(c, slot);
  const hipError_t e = slot_copy(c, slot, dst, c->pool + slot * c->entry_bytes, stream);
  if (e != hipSuccess) { cache_error(hipGetErrorString(e)); return AENC_E_HIP; }
  ++c->hits;
  return 1;
}
}  // namespace

extern "C" int aenc_cache_lookup(aenc_cache* c, uint64_t key, void* dst, void* stream) {
  if (!c || !dst) { cache_error("cache and dst must not be NULL"); return AENC_E_INVAL; }
  std::lock_guard<std::mutex> g(c->mu);
  return lookup_locked(c, key, dst, (hipStream_t)stream);
}

extern "C" int aenc_cache_insert(aenc_cache* c, uint64_t key, const void* src, void* stream) {
  if (!c || !src) { cache_error("cache and src must not be NULL"); return AENC_E_INVAL; }
  std::lock_guard<std::mutex> g(c->mu);
  int64_t slot;
  auto it = c->index.find(key);
  if (it != c->index.end()) {
    slot = it->second;                      // refresh the entry in place
    touch(c, slot);
  } else {
    if (!c->free_slots.empty()) {
      slot = c->free_slots.back();
      c->free_slots.pop_back();
    } else {                                // recycle the least recently used slot
      slot = c->lru.back();
      c->lru.pop_back();
      c->index.erase(c->slot_key[slot]);
      ++c->evictions;
    }
    c->lru.push_front(slot);
    c->where[slot] = c->lru.begin();
    c->index[key] = slot;
    c->slot_key[slot] = key;
  }
  const hipError_t e = slot_copy(c, slot, c->pool + slot * c->entry_bytes, src, (hipStream_t)stream);
  if (e != hipSuccess) { cache_error(hipGetErrorString(e)); return AENC_E_HIP; }
  ++c->inserts;
  return AENC_OK;
}

extern "C" int aenc_cache_stats(aenc_cache* c, int64_t out[5]) {
  if (!c || !out) { cache_error("cache and out must not be NULL"); return AENC_E_INVAL; }
  std::lock_guard<std::mutex> g(c->mu);
  out[0] = c->hits;
  out[1] = c->misses;
  out[2] = c->inserts;
  out[3] = c->evictions;
  out[4] = (int64_t)c->index.size();
  return AENC_OK;
}

extern "C" int aenc_forward_cached(aenc_handle* h, aenc_cache* c, const uint64_t* keys, const void* mel,
                                   const uint8_t* mask, void* out, void* stream, int32_t* hits) {
  if (!h || !c || !keys || !mel || !out) { cache_error("handle, cache, keys, mel and out must not be NULL"); return AENC_E_INVAL; }
  aenc_geometry g;
  if (aenc_handle_geometry(h, &g) != AENC_OK) return AENC_E_INVAL;
  int64_t shape[3];
  if (aenc_output_shape(&g, shape) != AENC_OK) return AENC_E_INVAL;
  const int64_t clip_bytes = shape[1] * shape[2] * (g.out_dtype == AENC_BF16 ? 2 : 4);
  if (clip_bytes != c->entry_bytes) { cache_error("cache entry size differs from one clip's output"); return AENC_E_INVAL; }
  int n_hit = 0;
  {
    // Decide and copy under one hold of the lock, so that no other thread can
    // evict an entry between the check and its copy.
    std::lock_guard<std::mutex> lk(c->mu);
    for (int b = 0; b < g.batch; ++b) n_hit += c->index.count(keys[b]) ? 1 : 0;
    if (n_hit == g.batch) {                 // every clip cached: copies only
      for (int b = 0; b < g.batch; ++b) {
        const int st = lookup_locked(c, keys[b], (char*)out + b * clip_bytes, (hipStream_t)stream);
        if (st < 0) return st;
      }
      if (hits) *hits = n_hit;
      return AENC_OK;
    }
  }
  // Any miss runs the whole batch (its shape is fixed), then stores the new clips.
  const int st = aenc_forward(h, mel, mask, out, stream);
  if (st != AENC_OK) return st;
  {
    std::lock_guard<std::mutex> lk(c->mu);
    c->hits += n_hit;
    c->misses += g.batch - n_hit;
  }
  for (int b = 0; b < g.batch; ++b) {
    if (aenc_cache_contains(c, keys[b]) == 1) continue;
    const int s2 = aenc_cache_insert(c, keys[b], (const char*)out + b * clip_bytes, stream);
    if (s2 != AENC_OK) return s2;
  }
  if (hits) *hits = n_hit;
  return AENC_OK;
}
