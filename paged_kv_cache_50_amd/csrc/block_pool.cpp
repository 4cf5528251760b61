// Host KV block pool: hands out the physical blocks of the paged cache and
// produces block tables and slot mappings for the attention calls (vLLM
// book, ch. 4.1 "Structures de données du planificateur", ch. 4.4
// "Détermination des touches du cache de préfixe et cycle de vie des blocs";
// «Khám phá vLLM», "Scheduler", the allocate_slots steps).
//
//   * Free blocks form a doubly linked queue in eviction order (intrusive
//     prev/next indices, O(1) removal).  At creation it holds every block in
//     id order; the first block taken from its head is the null block (0), a
//     placeholder for block-table padding that is never handed out or freed.
//   * New blocks are popped from the head; a popped block that still carries
//     a prefix-cache hash is evicted from the cache.
//   * Releasing a request walks its blocks last to first; a block whose
//     reference count drops to 0 returns to the head when it has no hash
//     (LIFO: the most recently used memory is reused first) and to the tail
//     when it has one (FIFO: cached blocks are evicted least recently used
//     first).
//   * A prefix-cache hit takes the block out of the free queue if it was in
//     it and raises its count.  At most num_tokens - 1 tokens of a new request
//     come from the cache.  Full blocks are entered into the cache under a
//     hash chained over the previous block's hash and the block's token ids
//     (64-bit FNV-1a: parent hash as 8 little-endian bytes, then each token id
//     as 4 little-endian bytes; 0 is the parent of the first block); an
//     existing entry for the same hash is kept.
//   * A request of n tokens owns ceil(n / block_size) blocks; an allocation
//     that cannot be met in full changes nothing.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int32_t n) {
  unsigned char buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = (unsigned char)(parent >> (8 * i));
  uint64_t h = fnv_bytes(kFnvOffset, buf, 8);
  for (int32_t t = 0; t < n; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    for (int i = 0; i < 4; ++i) buf[i] = (unsigned char)(v >> (8 * i));
    h = fnv_bytes(h, buf, 4);
  }
  return h;
}

struct Block {
  int32_t prev = -1, next = -1;   // free-queue links
  int32_t ref = 0;
  bool in_free = false;
  bool hashed = false;
  uint64_t hash = 0;
};

struct Request {
  std::vector<int32_t> blocks;
  std::vector<uint64_t> hashes;   // hash chain of the full blocks entered so far
  int64_t cached = 0;             // full blocks already entered into the cache
};

}  // namespace

struct pkv_block_pool {
  std::mutex mu;
  int32_t bs = 0;
  bool caching = false;
  std::vector<Block> blk;
  int32_t head = -1, tail = -1;
  int64_t nfree = 0;
  int32_t null_block = -1;
  std::unordered_map<uint64_t, int32_t> cache;
  std::unordered_map<int64_t, Request> reqs;

  void push_front(int32_t b) {
    Block& x = blk[b];
    x.prev = -1;
    x.next = head;
    if (head >= 0) blk[head].prev = b; else tail = b;
    head = b;
    x.in_free = true;
    ++nfree;
  }
  void push_back(int32_t b) {
    Block& x = blk[b];
    x.next = -1;
    x.prev = tail;
    if (tail >= 0) blk[tail].next = b; else head = b;
    tail = b;
    x.in_free = true;
    ++nfree;
  }
  void unlink(int32_t b) {
    Block& x = blk[b];
    if (x.prev >= 0) blk[x.prev].next = x.next; else head = x.next;
    if (x.next >= 0) blk[x.next].prev = x.prev; else tail = x.prev;
    x.prev = x.next = -1;
    x.in_free = false;
    --nfree;
  }
  int32_t pop_front() {
    const int32_t b = head;
    unlink(b);
    return b;
  }

  // take n blocks from the head (caller checked nfree >= n)
  void take(int64_t n, std::vector<int32_t>& out) {
    for (int64_t i = 0; i < n; ++i) {
      const int32_t b = pop_front();
      Block& x = blk[b];
      if (x.hashed) {
        auto it = cache.find(x.hash);
        if (it != cache.end() && it->second == b) cache.erase(it);
        x.hashed = false;
        x.hash = 0;
      }
      x.ref = 1;
      out.push_back(b);
    }
  }
  void touch(int32_t b) {
    if (blk[b].ref == 0) unlink(b);
    ++blk[b].ref;
  }
  void release(const std::vector<int32_t>& blocks) {
    for (size_t i = blocks.size(); i-- > 0;) {
      const int32_t b = blocks[i];
      if (--blk[b].ref == 0) {
        if (blk[b].hashed) push_back(b); else push_front(b);
      }
    }
  }
};

extern "C" {

pkv_block_pool* pkv_pool_create(int64_t num_blocks, int32_t block_size, int32_t prefix_caching) {
  if (num_blocks < 2 || num_blocks > INT32_MAX || block_size <= 0) return nullptr;
  pkv_block_pool* p = new (std::nothrow) pkv_block_pool();
  if (!p) return nullptr;
  p->bs = block_size;
  p->caching = prefix_caching != 0;
  p->blk.resize((size_t)num_blocks);
  for (int64_t b = 0; b < num_blocks; ++b) p->push_back((int32_t)b);
  p->null_block = p->pop_front();
  return p;
}

void pkv_pool_destroy(pkv_block_pool* p) { delete p; }

int64_t pkv_pool_num_free(pkv_block_pool* p) {
  if (!p) return -1;
  std::lock_guard<std::mutex> lk(p->mu);
  return p->nfree;
}

int64_t pkv_pool_allocate(pkv_block_pool* p, int64_t req, int64_t num_tokens,
                          const int32_t* token_ids) {
  if (!p || num_tokens < 0) return -2;
  std::lock_guard<std::mutex> lk(p->mu);
  const int64_t bs = p->bs;
  auto found = p->reqs.find(req);
  const bool fresh = found == p->reqs.end();
  // prefix-cache hits of a new request (at most num_tokens - 1 tokens)
  std::vector<int32_t> hits;
  std::vector<uint64_t> hit_hashes;
  if (fresh && p->caching && token_ids && num_tokens > 0) {
    uint64_t parent = 0;
    const int64_t max_blocks = (num_tokens - 1) / bs;
    for (int64_t i = 0; i < max_blocks; ++i) {
      const uint64_t h = chain_hash(parent, token_ids + i * bs, (int32_t)bs);
      auto it = p->cache.find(h);
      if (it == p->cache.end()) break;
      hits.push_back(it->second);
      hit_hashes.push_back(h);
      parent = h;
    }
  }
  const int64_t have = fresh ? (int64_t)hits.size() : (int64_t)found->second.blocks.size();
  const int64_t need = std::max<int64_t>(0, (num_tokens + bs - 1) / bs - have);
  int64_t evictable_hits = 0;
  for (int32_t b : hits) evictable_hits += p->blk[b].ref == 0 ? 1 : 0;
  if (need > p->nfree - evictable_hits) return -1;
  Request& r = p->reqs[req];
  if (fresh) {
    for (int32_t b : hits) p->touch(b);
    r.blocks = hits;
    r.hashes = hit_hashes;
    r.cached = (int64_t)hits.size();
  }
  p->take(need, r.blocks);
  return fresh ? (int64_t)hits.size() * bs : 0;
}

pkv_status pkv_pool_cache_full_blocks(pkv_block_pool* p, int64_t req, const int32_t* token_ids,
                                      int64_t num_tokens) {
  if (!p || num_tokens < 0 || (num_tokens > 0 && !token_ids)) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> lk(p->mu);
  auto it = p->reqs.find(req);
  if (it == p->reqs.end()) return PKV_ERR_SHAPE;
  if (!p->caching) return PKV_OK;
  Request& r = it->second;
  const int64_t bs = p->bs;
  const int64_t full = std::min<int64_t>(num_tokens / bs, (int64_t)r.blocks.size());
  for (int64_t i = r.cached; i < full; ++i) {
    const uint64_t parent = i > 0 ? r.hashes[(size_t)i - 1] : 0;
    const uint64_t h = chain_hash(parent, token_ids + i * bs, (int32_t)bs);
    r.hashes.push_back(h);
    Block& x = p->blk[r.blocks[(size_t)i]];
    if (!x.hashed) {
      x.hashed = true;
      x.hash = h;
      p->cache.emplace(h, r.blocks[(size_t)i]);   // an existing entry is kept
    }
  }
  r.cached = std::max(r.cached, full);
  return PKV_OK;
}

pkv_status pkv_pool_free(pkv_block_pool* p, int64_t req) {
  if (!p) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> lk(p->mu);
  auto it = p->reqs.find(req);
  if (it == p->reqs.end()) return PKV_ERR_SHAPE;
  p->release(it->second.blocks);
  p->reqs.erase(it);
  return PKV_OK;
}

int64_t pkv_pool_num_blocks_of(pkv_block_pool* p, int64_t req) {
  if (!p) return -1;
  std::lock_guard<std::mutex> lk(p->mu);
  auto it = p->reqs.find(req);
  return it == p->reqs.end() ? -1 : (int64_t)it->second.blocks.size();
}

pkv_status pkv_pool_block_table(pkv_block_pool* p, const int64_t* reqs, int32_t n,
                                int32_t max_blocks, int32_t* out) {
  if (!p || (n > 0 && (!reqs || !out))) return PKV_ERR_NULL;
  if (n < 0 || max_blocks <= 0) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(p->mu);
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->reqs.find(reqs[i]);
    if (it == p->reqs.end() || (int64_t)it->second.blocks.size() > max_blocks) return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& b = p->reqs.find(reqs[i])->second.blocks;
    int32_t* row = out + (int64_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < (int32_t)b.size() ? b[j] : p->null_block;
  }
  return PKV_OK;
}

pkv_status pkv_pool_slot_mapping(pkv_block_pool* p, int64_t req, int64_t first_pos, int64_t count,
                                 int64_t* out) {
  if (!p || (count > 0 && !out)) return PKV_ERR_NULL;
  if (first_pos < 0 || count < 0) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(p->mu);
  auto it = p->reqs.find(req);
  if (it == p->reqs.end()) return PKV_ERR_SHAPE;
  const std::vector<int32_t>& b = it->second.blocks;
  const int64_t bs = p->bs;
  if (first_pos + count > (int64_t)b.size() * bs) return PKV_ERR_SHAPE;
  for (int64_t k = 0; k < count; ++k) {
    const int64_t pos = first_pos + k;
    out[k] = (int64_t)b[(size_t)(pos / bs)] * bs + pos % bs;
  }
  return PKV_OK;
}

int64_t pkv_pool_free_queue(pkv_block_pool* p, int32_t* out, int64_t cap) {
  if (!p) return -1;
  std::lock_guard<std::mutex> lk(p->mu);
  int64_t n = 0;
  for (int32_t b = p->head; b >= 0; b = p->blk[b].next) {
    if (out && n < cap) out[n] = b;
    ++n;
  }
  return n;
}

}  // extern "C"
