// Memoized cascade plans [cascade-PR, "What I left out, and where I was
// unsure": detection re-runs for every layer of every step although the page
// table is already cached; a plan slot in the plan cache is named as the
// follow-up]. Every layer of a decode step reads the same page table, so one
// plan (and its upload) serves them all.
//
// The key is the whole host page table - indptr, indices and kv_len - with
// the page size and the plan parameters. The KV lengths are part of the key
// on purpose: partitions, the full-page cap and the level-1 ranges depend on
// them, so two steps with the same rows but different lengths need different
// plans [FreeToken issue "Layer-major prefill for offloaded MoE", the fix
// to a plan cache keyed by rows although split-KV depends on KV length].
// A lookup compares the table with each cached key (sizes first, then the
// lengths, the row offsets and the page ids: memcmp, a few microseconds for a
// batch of 72 with 20k page ids), so an equal key is never missed and a
// different one never returned; a hash over the same bytes would cost more
// than the comparisons it saves at these cache sizes.

#include <cstring>
#include <list>
#include <mutex>
#include <vector>

#include "internal.h"
#include "pdk.h"

using namespace pdk;

namespace {

struct Key {
  int32_t page_size = 0;
  pdk_cascade_params params{};
  std::vector<int32_t> indptr, indices, kv_len;
};

bool same_table(const Key& k, const pdk_csr* csr, int32_t P, const pdk_cascade_params& pr) {
  if (k.page_size != P || std::memcmp(&k.params, &pr, sizeof(pr)) != 0) return false;
  if ((int)k.kv_len.size() != csr->batch || (int)k.indices.size() != csr->nnz) return false;
  return std::memcmp(k.kv_len.data(), csr->kv_len, sizeof(int32_t) * csr->batch) == 0 &&
         std::memcmp(k.indptr.data(), csr->indptr, sizeof(int32_t) * (csr->batch + 1)) == 0 &&
         (csr->nnz == 0 ||
          std::memcmp(k.indices.data(), csr->indices, sizeof(int32_t) * csr->nnz) == 0);
}

struct Entry {
  int64_t id;
  Key key;
  pdk_cascade_plan* plan;
};

}  // namespace

struct pdk_plan_cache {
  int capacity = 0;
  std::list<Entry> lru;  // most recently used first
  mutable std::mutex mu;
  int64_t next_id = 1;
  int64_t lookups = 0, hits = 0, builds = 0, evictions = 0;
};

extern "C" {

int pdk_plan_cache_create(int32_t capacity, pdk_plan_cache** out) {
  if (!out) return fail(PDK_ERR_ARG, "NULL cache_out");
  *out = nullptr;
  if (capacity < 1) return fail(PDK_ERR_ARG, "plan cache capacity %d < 1", capacity);
  auto c = new pdk_plan_cache();
  c->capacity = capacity;
  *out = c;
  return PDK_OK;
}

void pdk_plan_cache_free(pdk_plan_cache* cache) {
  if (!cache) return;
  for (auto& e : cache->lru) pdk_cascade_plan_free(e.plan);
  delete cache;
}

int pdk_plan_cache_get(pdk_plan_cache* cache, const pdk_csr* csr, int32_t P,
                       const pdk_cascade_params* params, pdk_cascade_plan** plan_out,
                       int64_t* entry_id, int32_t* hit) {
  if (!cache || !params || !plan_out) return fail(PDK_ERR_ARG, "NULL argument");
  *plan_out = nullptr;
  if (!csr || csr->batch < 0 || csr->nnz < 0 || !csr->indptr || (csr->batch > 0 && !csr->kv_len) ||
      (csr->nnz > 0 && !csr->indices))
    return fail(PDK_ERR_ARG, "NULL or negative-size page table");
  // a table equal to a cached key passed the planner's validation when that
  // key was built; a new one is validated by the planner below
  std::lock_guard<std::mutex> lock(cache->mu);
  ++cache->lookups;
  for (auto it = cache->lru.begin(); it != cache->lru.end(); ++it) {
    if (!same_table(it->key, csr, P, *params)) continue;
    ++cache->hits;
    cache->lru.splice(cache->lru.begin(), cache->lru, it);
    *plan_out = cache->lru.front().plan;
    if (entry_id) *entry_id = cache->lru.front().id;
    if (hit) *hit = 1;
    return PDK_OK;
  }
  pdk_cascade_plan* plan = nullptr;
  if (int st = pdk_cascade_plan_create(csr, P, params, &plan)) return st;
  ++cache->builds;
  Entry e{cache->next_id++, Key{}, plan};
  e.key.page_size = P;
  e.key.params = *params;
  e.key.indptr.assign(csr->indptr, csr->indptr + csr->batch + 1);
  e.key.indices.assign(csr->indices, csr->indices + csr->nnz);
  e.key.kv_len.assign(csr->kv_len, csr->kv_len + csr->batch);
  cache->lru.push_front(std::move(e));
  while ((int)cache->lru.size() > cache->capacity) {
    pdk_cascade_plan_free(cache->lru.back().plan);
    cache->lru.pop_back();
    ++cache->evictions;
  }
  *plan_out = cache->lru.front().plan;
  if (entry_id) *entry_id = cache->lru.front().id;
  if (hit) *hit = 0;
  return PDK_OK;
}

int pdk_plan_cache_stats(const pdk_plan_cache* cache, int64_t stats[5]) {
  if (!cache || !stats) return fail(PDK_ERR_ARG, "NULL argument");
  std::lock_guard<std::mutex> lock(cache->mu);
  stats[0] = cache->lookups;
  stats[1] = cache->hits;
  stats[2] = cache->builds;
  stats[3] = cache->evictions;
  stats[4] = (int64_t)cache->lru.size();
  return PDK_OK;
}

}  // extern "C"
