// Host-side block pool: the allocator behind a paged cache, with reference
// counts for shared blocks and a prefix cache keyed by chained block hashes.
//
// The cache lives in fixed-size blocks handed out as a sequence grows, and
// sequences that share a prefix can share its blocks ("Serving" section
// 23.4).  Prefix caching finds those blocks by content: each full block is
// named by a hash of its tokens chained with the hash of the block before it
// (the block-and-hash-chain scheme of the prompt-caching articles on the
// pagedattention tag page), so one changed token renames every later block.
//
// Policy, fixed so that results are reproducible:
//  * a fresh block is the lowest-numbered free block that holds no cached
//    prefix; when there is none, the cached free block released longest ago
//    is reused and its hash forgotten;
//  * a block whose reference count drops to zero is free; if it carries a
//    hash it stays findable by that hash until it is reused.
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <deque>
#include <map>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_block_pool {
  int32_t n_blocks = 0;
  std::vector<int32_t> ref;            // reference count per block
  std::vector<uint64_t> hash;          // content hash, valid where cached[b]
  std::vector<uint8_t> cached;
  std::vector<uint64_t> released_at;   // key in lru while free and cached
  std::set<int32_t> free_plain;        // free, no hash: lowest id first
  std::map<uint64_t, int32_t> lru;     // free and cached, by release order
  std::unordered_map<uint64_t, int32_t> by_hash;
  uint64_t clock = 0;

  int32_t available() const { return (int32_t)(free_plain.size() + lru.size()); }

  // A block for new content (reference count 1, no hash).
  int32_t take_fresh() {
    int32_t b;
    if (!free_plain.empty()) {
      b = *free_plain.begin();
      free_plain.erase(free_plain.begin());
    } else {
      auto it = lru.begin();
      b = it->second;
      lru.erase(it);
      by_hash.erase(hash[b]);
      cached[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  void drop_ref(int32_t b) {
    if (--ref[b] > 0) return;
    if (cached[b]) {
      released_at[b] = ++clock;
      lru.emplace(released_at[b], b);
    } else {
      free_plain.insert(b);
    }
  }
};

namespace {

constexpr uint64_t kFnvOffset = 14695981039346656037ull;  // FNV-1a, 64-bit
constexpr uint64_t kFnvPrime = 1099511628211ull;

uint64_t fnv1a(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

bool valid_ids(const pa_block_pool* p, const int32_t* ids, int32_t n, bool need_ref) {
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->n_blocks) return false;
    if (need_ref && p->ref[ids[i]] < 1) return false;
  }
  return true;
}

}  // namespace

extern "C" {

int pa_block_hashes(const int32_t* tokens, int32_t n_tokens, int32_t block_size,
                    uint64_t parent, uint64_t* hashes, int32_t* n_full) {
  if (n_tokens < 0 || block_size < 1) return PA_ERR_SHAPE;
  if (!n_full || (n_tokens >= block_size && (!tokens || !hashes))) return PA_ERR_NULL;
  const int32_t nf = n_tokens / block_size;
  uint64_t h = parent;
  for (int32_t i = 0; i < nf; ++i) {
    unsigned char head[8];
    for (int k = 0; k < 8; ++k) head[k] = (unsigned char)(h >> (8 * k));  // little endian
    uint64_t x = fnv1a(kFnvOffset, head, 8);
    for (int32_t t = 0; t < block_size; ++t) {
      const uint32_t v = (uint32_t)tokens[(int64_t)i * block_size + t];
      unsigned char w[4] = {(unsigned char)v, (unsigned char)(v >> 8),
                            (unsigned char)(v >> 16), (unsigned char)(v >> 24)};
      x = fnv1a(x, w, 4);
    }
    hashes[i] = h = x;
  }
  *n_full = nf;
  return PA_OK;
}

pa_block_pool* pa_pool_create(int32_t n_blocks) {
  if (n_blocks < 1) return nullptr;
  pa_block_pool* p = new (std::nothrow) pa_block_pool();
  if (!p) return nullptr;
  try {
    p->n_blocks = n_blocks;
    p->ref.assign(n_blocks, 0);
    p->hash.assign(n_blocks, 0);
    p->cached.assign(n_blocks, 0);
    p->released_at.assign(n_blocks, 0);
    for (int32_t b = 0; b < n_blocks; ++b) p->free_plain.insert(p->free_plain.end(), b);
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

int32_t pa_pool_available(const pa_block_pool* pool) {
  return pool ? pool->available() : PA_ERR_NULL;
}

int32_t pa_pool_refcount(const pa_block_pool* pool, int32_t block) {
  if (!pool) return PA_ERR_NULL;
  if (block < 0 || block >= pool->n_blocks) return PA_ERR_SHAPE;
  return pool->ref[block];
}

int pa_pool_alloc(pa_block_pool* pool, int32_t n, int32_t* ids) {
  if (!pool) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && !ids) return PA_ERR_NULL;
  if (n > pool->available()) return PA_ERR_NOSPACE;
  for (int32_t i = 0; i < n; ++i) ids[i] = pool->take_fresh();
  return PA_OK;
}

int pa_pool_fork(pa_block_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && !ids) return PA_ERR_NULL;
  if (!valid_ids(pool, ids, n, true)) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) ++pool->ref[ids[i]];
  return PA_OK;
}

int pa_pool_release(pa_block_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && !ids) return PA_ERR_NULL;
  if (!valid_ids(pool, ids, n, true)) return PA_ERR_SHAPE;
  // a block listed twice must hold two references
  std::unordered_map<int32_t, int32_t> count;
  for (int32_t i = 0; i < n; ++i)
    if (++count[ids[i]] > pool->ref[ids[i]]) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) pool->drop_ref(ids[i]);
  return PA_OK;
}

int pa_pool_map_prefix(pa_block_pool* pool, const uint64_t* hashes, int32_t n, int32_t* ids,
                       int32_t* n_hit) {
  if (!pool || !n_hit) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && (!hashes || !ids)) return PA_ERR_NULL;
  // the cached prefix, and how many of its blocks are free now
  int32_t hit = 0, hit_free = 0;
  while (hit < n) {
    auto it = pool->by_hash.find(hashes[hit]);
    if (it == pool->by_hash.end()) break;
    hit_free += pool->ref[it->second] == 0;
    ++hit;
  }
  if (n - hit > pool->available() - hit_free) return PA_ERR_NOSPACE;
  for (int32_t i = 0; i < hit; ++i) {
    const int32_t b = pool->by_hash[hashes[i]];
    if (pool->ref[b] == 0) pool->lru.erase(pool->released_at[b]);
    ++pool->ref[b];
    ids[i] = b;
  }
  for (int32_t i = hit; i < n; ++i) {
    const int32_t b = pool->take_fresh();
    ids[i] = b;
    if (pool->by_hash.count(hashes[i])) continue;  // the same content twice
    pool->hash[b] = hashes[i];
    pool->cached[b] = 1;
    pool->by_hash.emplace(hashes[i], b);
  }
  *n_hit = hit;
  return PA_OK;
}

int pa_pool_simulate(const int32_t* arrivals, const int32_t* prompt_lens,
                     const int32_t* final_lens, int32_t n_requests, int32_t n_blocks,
                     int32_t block_size, int32_t policy, int32_t max_len, int32_t* start,
                     int32_t* finish, int32_t* running, int32_t max_steps, int32_t* n_steps,
                     int64_t* util_tokens, int64_t* util_capacity) {
  if (!n_steps || !util_tokens || !util_capacity) return PA_ERR_NULL;
  if (n_requests < 0 || n_blocks < 1 || block_size < 1 || max_steps < 0) return PA_ERR_SHAPE;
  if (policy != PA_SIM_RESERVE && policy != PA_SIM_PAGED) return PA_ERR_SHAPE;
  if (n_requests > 0 && (!arrivals || !prompt_lens || !final_lens || !start || !finish))
    return PA_ERR_NULL;
  if (max_steps > 0 && !running) return PA_ERR_NULL;
  const int32_t reserve = policy == PA_SIM_RESERVE ? (max_len + block_size - 1) / block_size : 0;
  for (int32_t i = 0; i < n_requests; ++i) {
    if (arrivals[i] < 0 || prompt_lens[i] < 1 || final_lens[i] < prompt_lens[i])
      return PA_ERR_SHAPE;
    if (policy == PA_SIM_RESERVE && final_lens[i] > max_len) return PA_ERR_SHAPE;
    const int32_t need =
        policy == PA_SIM_RESERVE ? reserve : (prompt_lens[i] + block_size - 1) / block_size;
    if (need > n_blocks) return PA_ERR_NOSPACE;  // could never start
  }
  pa_block_pool* pool = pa_pool_create(n_blocks);
  if (!pool) return PA_ERR_NOSPACE;
  // requests in arrival order (ties by index): the order waiting requests start in
  std::vector<int32_t> order(n_requests);
  for (int32_t i = 0; i < n_requests; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return arrivals[x] < arrivals[y]; });
  std::vector<std::vector<int32_t>> held(n_requests);
  std::vector<int32_t> tokens(n_requests, 0);
  std::vector<int32_t> live;    // running requests, in start order
  std::deque<int32_t> waiting;  // arrived, not started
  int32_t next = 0, done = 0, step = 0, status = PA_OK;
  int64_t tok_sum = 0, cap_sum = 0;
  for (int32_t i = 0; i < n_requests; ++i) start[i] = finish[i] = -1;
  while (done < n_requests) {
    while (next < n_requests && arrivals[order[next]] == step) waiting.push_back(order[next++]);
    // start waiting requests in arrival order while their blocks are free
    while (!waiting.empty()) {
      const int32_t i = waiting.front();
      const int32_t need =
          policy == PA_SIM_RESERVE ? reserve : (prompt_lens[i] + block_size - 1) / block_size;
      if (need > pool->available()) break;
      waiting.pop_front();
      held[i].resize(need);
      pa_pool_alloc(pool, need, held[i].data());
      tokens[i] = prompt_lens[i];
      start[i] = step;
      live.push_back(i);
    }
    if (step < max_steps) running[step] = (int32_t)live.size();
    for (int32_t i : live) {
      tok_sum += tokens[i];
      cap_sum += (int64_t)held[i].size() * block_size;
    }
    // each running request finishes, or gains a token (and a block when its
    // tokens pass the blocks it holds)
    std::vector<int32_t> still;
    still.reserve(live.size());
    for (int32_t i : live) {
      if (tokens[i] >= final_lens[i]) {
        finish[i] = step;
        pa_pool_release(pool, held[i].data(), (int32_t)held[i].size());
        held[i].clear();
        ++done;
        continue;
      }
      ++tokens[i];
      if (policy == PA_SIM_PAGED && (int64_t)tokens[i] > (int64_t)held[i].size() * block_size) {
        int32_t b;
        if (pa_pool_alloc(pool, 1, &b) != PA_OK) {
          status = PA_ERR_NOSPACE;  // the pool ran out while requests grew
          break;
        }
        held[i].push_back(b);
      }
      still.push_back(i);
    }
    if (status != PA_OK) break;
    live.swap(still);
    ++step;
  }
  pa_pool_destroy(pool);
  *n_steps = step;
  *util_tokens = tok_sum;
  *util_capacity = cap_sum;
  if (status == PA_OK && step > max_steps) status = PA_ERR_SHAPE;  // trace cut short
  return status;
}

}  // extern "C"
