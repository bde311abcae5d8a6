// Host-side page allocator of the paged cache (the pkv_pool_* calls of
// include/pkv.h): reference counts, prefix reuse at job admission, prompt
// caching of released pages with least-recently-released eviction, and
// defragmentation planning. Host memory only; the data movement a
// defragmentation plans runs on the GPU (pool_kernels.hip).
//
// Sources: ExLlamaV2 "Dynamic Generator" page, "Continuous Batching" (jobs
// start while their pages fit, finished jobs free pages, later jobs fill the
// holes; unreferenced pages are defragmented when the queue is empty),
// "Deduplication" (a new job references the K/V already cached for its prompt
// prefix) and "Prompt caching" (the most recently used pages are the last to
// be overwritten).
//
// A full prompt page is found again by its prefix: all token ids up to the end
// of the page. The index keys it by a 64-bit FNV-1a hash chained over the
// prompt's pages (the previous page's chain value, then this page's 256 token
// ids as little-endian int32), and a hit is confirmed against the page's own
// chain predecessor, position and 256 tokens.

#include "pkv.h"

#include <algorithm>
#include <cstring>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

namespace {

constexpr int kPage = PKV_PAGE_SIZE;
constexpr uint64_t kFnvBasis = 1469598103934665603ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

enum State : uint8_t { kFree = 0, kCached = 1, kUsed = 2 };

uint64_t chain_hash(uint64_t prev, const int32_t* toks) {
  uint64_t h = kFnvBasis;
  for (int i = 0; i < 8; ++i) {
    h ^= (prev >> (8 * i)) & 0xFF;
    h *= kFnvPrime;
  }
  for (int t = 0; t < kPage; ++t) {
    const uint32_t v = static_cast<uint32_t>(toks[t]);
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xFF;
      h *= kFnvPrime;
    }
  }
  return h;
}

}  // namespace

struct pkv_pool {
  int32_t P = 0;
  std::vector<int32_t> ref;
  std::vector<uint8_t> state;
  std::vector<uint64_t> stamp;        // release counter when the page became cached
  std::vector<uint8_t> keyed;         // 1: the page carries a prefix key
  std::vector<uint64_t> hash;         // chain value of the page's prefix
  std::vector<uint64_t> prev_hash;    // chain value of the prefix before it
  std::vector<int32_t> first_tok;     // position of the page's first token in its prompt
  std::vector<int32_t> toks;          // [P][256] the page's own token ids
  std::unordered_map<uint64_t, int32_t> index;
  std::set<int32_t> free_set;                          // lowest index first
  std::set<std::pair<uint64_t, int32_t>> cached_set;   // oldest release first
  uint64_t clock = 0;
  int32_t n_used = 0;

  explicit pkv_pool(int32_t n)
      : P(n), ref(n, 0), state(n, kFree), stamp(n, 0), keyed(n, 0), hash(n, 0), prev_hash(n, 0),
        first_tok(n, 0), toks(static_cast<size_t>(n) * kPage, 0) {
    for (int32_t p = 0; p < n; ++p) free_set.insert(free_set.end(), p);
  }

  int32_t allocatable() const { return P - n_used; }

  void unkey(int32_t p) {
    if (!keyed[p]) return;
    auto it = index.find(hash[p]);
    if (it != index.end() && it->second == p) index.erase(it);
    keyed[p] = 0;
  }

  void use(int32_t p) {
    ref[p] = 1;
    state[p] = kUsed;
    ++n_used;
  }

  // One page for new content: the lowest free page, else the cached page
  // released longest ago (lowest index on ties), which forgets its key.
  int32_t take() {
    int32_t p;
    if (!free_set.empty()) {
      p = *free_set.begin();
      free_set.erase(free_set.begin());
    } else {
      p = cached_set.begin()->second;
      cached_set.erase(cached_set.begin());
      unkey(p);
    }
    state[p] = kFree;
    return p;
  }

  // The page holding the prompt prefix that ends with page j (chain value h,
  // predecessor value prev, page tokens t), or -1.
  int32_t lookup(uint64_t h, uint64_t prev, int32_t pos, const int32_t* t) const {
    auto it = index.find(h);
    if (it == index.end()) return -1;
    const int32_t p = it->second;
    if (!keyed[p] || prev_hash[p] != prev || first_tok[p] != pos) return -1;
    if (std::memcmp(&toks[static_cast<size_t>(p) * kPage], t, kPage * sizeof(int32_t)) != 0) return -1;
    return p;
  }

  void drop_ref(int32_t p) {
    if (--ref[p] > 0) return;
    --n_used;
    if (keyed[p]) {
      state[p] = kCached;
      stamp[p] = ++clock;
      cached_set.insert({stamp[p], p});
    } else {
      state[p] = kFree;
      free_set.insert(p);
    }
  }
};

extern "C" {

pkv_pool* pkv_pool_create(int32_t num_pages) {
  if (num_pages < 1 || num_pages > (1 << 23)) return nullptr;
  try {
    return new pkv_pool(num_pages);
  } catch (...) {
    return nullptr;
  }
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int pkv_pool_stats(const pkv_pool* pool, int32_t* out) {
  if (!pool || !out) return PKV_ERR_NULL;
  out[0] = static_cast<int32_t>(pool->free_set.size());
  out[1] = static_cast<int32_t>(pool->cached_set.size());
  out[2] = pool->n_used;
  return PKV_OK;
}

int pkv_pool_admit(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, int32_t* pages, int32_t max_pages,
                   int32_t* n_pages_out, int32_t* cached_tokens) {
  if (!pool || !pages || !n_pages_out || !cached_tokens || (n_tokens > 0 && !tokens)) return PKV_ERR_NULL;
  if (n_tokens < 0) return PKV_ERR_SHAPE;
  const int32_t n_pages = (n_tokens + kPage - 1) / kPage;
  if (n_pages > max_pages) return PKV_ERR_SHAPE;
  try {
    // match full pages from the start while a prompt token follows them
    std::vector<int32_t> matched;
    std::vector<uint64_t> chain(n_pages + 1, kFnvBasis);  // chain[j]: value before page j
    const int32_t matchable = n_tokens > 0 ? (n_tokens - 1) / kPage : 0;
    for (int32_t j = 0; j < n_pages && (j + 1) * kPage <= n_tokens; ++j)
      chain[j + 1] = chain_hash(chain[j], tokens + static_cast<size_t>(j) * kPage);
    for (int32_t j = 0; j < matchable; ++j) {
      const int32_t p = pool->lookup(chain[j + 1], chain[j], j * kPage, tokens + static_cast<size_t>(j) * kPage);
      if (p < 0) break;
      matched.push_back(p);
    }
    int32_t revived = 0;
    for (int32_t p : matched) revived += pool->state[p] == kCached;
    const int32_t fresh = n_pages - static_cast<int32_t>(matched.size());
    if (fresh > pool->allocatable() - revived) return PKV_ERR_SPACE;
    int32_t k = 0;
    for (int32_t p : matched) {
      if (pool->state[p] == kCached) {
        pool->cached_set.erase({pool->stamp[p], p});
        pool->use(p);
      } else {
        ++pool->ref[p];
      }
      pages[k++] = p;
    }
    for (int32_t j = static_cast<int32_t>(matched.size()); j < n_pages; ++j) {
      const int32_t p = pool->take();
      pool->use(p);
      if ((j + 1) * kPage <= n_tokens) {  // a full page gets its prefix key
        const uint64_t h = chain[j + 1];
        if (pool->index.find(h) == pool->index.end()) {
          pool->index.emplace(h, p);
          pool->keyed[p] = 1;
          pool->hash[p] = h;
          pool->prev_hash[p] = chain[j];
          pool->first_tok[p] = j * kPage;
          std::memcpy(&pool->toks[static_cast<size_t>(p) * kPage], tokens + static_cast<size_t>(j) * kPage,
                      kPage * sizeof(int32_t));
        }
      }
      pages[k++] = p;
    }
    *n_pages_out = n_pages;
    *cached_tokens = static_cast<int32_t>(matched.size()) * kPage;
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_STATE;
  }
}

int pkv_pool_alloc(pkv_pool* pool, int32_t n, int32_t* pages) {
  if (!pool || (n > 0 && !pages)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n > pool->allocatable()) return PKV_ERR_SPACE;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = pool->take();
    pool->use(p);
    pages[i] = p;
  }
  return PKV_OK;
}

int pkv_pool_retain(pkv_pool* pool, const int32_t* pages, int32_t n) {
  if (!pool || (n > 0 && !pages)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (pages[i] < 0 || pages[i] >= pool->P || pool->state[pages[i]] != kUsed) return PKV_ERR_STATE;
  for (int32_t i = 0; i < n; ++i) ++pool->ref[pages[i]];
  return PKV_OK;
}

int pkv_pool_release(pkv_pool* pool, const int32_t* pages, int32_t n) {
  if (!pool || (n > 0 && !pages)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  try {
    std::unordered_map<int32_t, int32_t> need;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t p = pages[i];
      if (p < 0 || p >= pool->P) return PKV_ERR_STATE;
      if (++need[p] > pool->ref[p]) return PKV_ERR_STATE;
    }
  } catch (...) {
    return PKV_ERR_STATE;
  }
  for (int32_t i = 0; i < n; ++i) pool->drop_ref(pages[i]);
  return PKV_OK;
}

int pkv_pool_defrag(pkv_pool* pool, int32_t move_referenced, int32_t* remap, int32_t* src, int32_t* dst,
                    int32_t* n_moves) {
  if (!pool || !remap || !src || !dst || !n_moves) return PKV_ERR_NULL;
  const int32_t P = pool->P;
  const int32_t n_occ = P - static_cast<int32_t>(pool->free_set.size());
  int32_t k = 0;
  auto hole = pool->free_set.begin();  // free pages, ascending; the ones below n_occ are the holes
  for (int32_t p = 0; p < P; ++p) remap[p] = p;
  for (int32_t s = n_occ; s < P; ++s) {
    const uint8_t st = pool->state[s];
    if (st == kFree || (st == kUsed && !move_referenced)) continue;
    if (hole == pool->free_set.end() || *hole >= n_occ) break;
    const int32_t d = *hole;
    ++hole;
    src[k] = s;
    dst[k] = d;
    ++k;
  }
  for (int32_t i = 0; i < k; ++i) {
    const int32_t s = src[i], d = dst[i];
    remap[s] = d;
    pool->free_set.erase(d);
    pool->free_set.insert(s);
    pool->ref[d] = pool->ref[s];
    pool->state[d] = pool->state[s];
    pool->stamp[d] = pool->stamp[s];
    pool->keyed[d] = pool->keyed[s];
    pool->hash[d] = pool->hash[s];
    pool->prev_hash[d] = pool->prev_hash[s];
    pool->first_tok[d] = pool->first_tok[s];
    std::memcpy(&pool->toks[static_cast<size_t>(d) * kPage], &pool->toks[static_cast<size_t>(s) * kPage],
                kPage * sizeof(int32_t));
    if (pool->state[d] == kCached) {
      pool->cached_set.erase({pool->stamp[s], s});
      pool->cached_set.insert({pool->stamp[d], d});
    }
    if (pool->keyed[d]) pool->index[pool->hash[d]] = d;
    pool->ref[s] = 0;
    pool->state[s] = kFree;
    pool->stamp[s] = 0;
    pool->keyed[s] = 0;
  }
  *n_moves = k;
  return PKV_OK;
}

}  // extern "C"
