// Randomised stress of the host KV block pool, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_block_pool_sanitized.py.
// Thousands of random operations (allocate, grow, cache full blocks, free,
// block tables, slot mappings, the free queue, and calls with bad arguments)
// on pools of several sizes, block sizes and both prefix-caching modes; after
// every operation the pool's invariants are checked against a model of the
// live requests.  Exits non-zero on the first violated invariant.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "../../include/pagedkv.h"

#define REQUIRE(c)                                                                 \
  do {                                                                             \
    if (!(c)) {                                                                    \
      std::fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #c);    \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

namespace {

struct Req {
  std::vector<int32_t> tokens;
};

int64_t blocks_for(int64_t n, int32_t bs) { return (n + bs - 1) / bs; }

void check(pkv_block_pool* p, const std::map<int64_t, Req>& live, int64_t num_blocks, int32_t bs) {
  // free queue: distinct, never the null block, its length the free count
  std::vector<int32_t> fq((size_t)num_blocks + 4, -7);
  const int64_t nfree = pkv_pool_free_queue(p, fq.data(), (int64_t)fq.size());
  REQUIRE(nfree == pkv_pool_num_free(p));
  REQUIRE(nfree >= 0 && nfree <= num_blocks - 1);
  std::set<int32_t> freeset;
  for (int64_t i = 0; i < nfree; ++i) {
    REQUIRE(fq[i] >= 1 && fq[i] < num_blocks);
    REQUIRE(freeset.insert(fq[i]).second);
  }
  REQUIRE(fq[nfree] == -7);                       // nothing written past the length
  // every live request: ceil(n / bs) distinct blocks, none of them free
  std::set<int32_t> owned;
  for (const auto& [req, r] : live) {
    const int64_t nb = pkv_pool_num_blocks_of(p, req);
    REQUIRE(nb == blocks_for((int64_t)r.tokens.size(), bs));
    if (nb == 0) continue;
    std::vector<int32_t> row((size_t)nb + 2, -9);
    const int64_t one = req;
    REQUIRE(pkv_pool_block_table(p, &one, 1, (int32_t)nb + 2, row.data()) == PKV_OK);
    std::set<int32_t> mine;
    for (int64_t i = 0; i < nb; ++i) {
      REQUIRE(row[i] >= 1 && row[i] < num_blocks);
      REQUIRE(!freeset.count(row[i]));
      REQUIRE(mine.insert(row[i]).second);
      owned.insert(row[i]);
    }
    REQUIRE(row[nb] == 0 && row[nb + 1] == 0);      // padded with the null block
    if (nb > 1)                                     // a table that is too narrow is refused
      REQUIRE(pkv_pool_block_table(p, &one, 1, (int32_t)nb - 1, row.data()) == PKV_ERR_SHAPE);
    // slots of every token lie in the request's blocks
    const int64_t n = (int64_t)r.tokens.size();
    std::vector<int64_t> slots((size_t)n);
    REQUIRE(pkv_pool_slot_mapping(p, req, 0, n, slots.data()) == PKV_OK);
    for (int64_t t = 0; t < n; ++t) {
      REQUIRE(slots[t] / bs == row[t / bs]);
      REQUIRE(slots[t] % bs == t % bs);
    }
  }
  // blocks are owned, free, or cached and evicted later: never both
  REQUIRE((int64_t)owned.size() + nfree <= num_blocks - 1);
}

int run(int64_t num_blocks, int32_t bs, int32_t caching, uint32_t seed, int steps) {
  pkv_block_pool* p = pkv_pool_create(num_blocks, bs, caching);
  REQUIRE(p);
  std::mt19937 rng(seed);
  std::map<int64_t, Req> live;
  int64_t next_req = 0;
  auto rnd = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  // a few shared prompt prefixes, so that cached blocks are found again
  std::vector<std::vector<int32_t>> prompts(4);
  for (auto& pr : prompts)
    for (int i = 0; i < 5 * bs + 3; ++i) pr.push_back(rnd(0, 50));
  for (int step = 0; step < steps; ++step) {
    const int op = rnd(0, 9);
    if (op <= 3) {                                  // a new request
      Req r;
      const auto& pr = prompts[rnd(0, 3)];
      const int keep = rnd(0, (int)pr.size());
      r.tokens.assign(pr.begin(), pr.begin() + keep);
      const int extra = rnd(0, 3 * bs);
      for (int i = 0; i < extra; ++i) r.tokens.push_back(rnd(0, 50));
      const int64_t req = next_req++;
      const int64_t hit = pkv_pool_allocate(p, req, (int64_t)r.tokens.size(),
                                            r.tokens.empty() ? nullptr : r.tokens.data());
      REQUIRE(hit >= -1);
      if (hit >= 0) {
        REQUIRE(hit <= std::max<int64_t>(0, (int64_t)r.tokens.size() - 1));
        REQUIRE(hit % bs == 0);
        if (!caching) REQUIRE(hit == 0);
        live[req] = r;
      } else {
        REQUIRE(pkv_pool_num_blocks_of(p, req) == -1);   // a refused request owns nothing
      }
    } else if (op == 4 && !live.empty()) {          // grow a request
      auto it = live.begin();
      std::advance(it, rnd(0, (int)live.size() - 1));
      const int add = rnd(0, 2 * bs);
      std::vector<int32_t> grown = it->second.tokens;
      for (int i = 0; i < add; ++i) grown.push_back(rnd(0, 50));
      const int64_t before = pkv_pool_num_blocks_of(p, it->first);
      const int64_t r = pkv_pool_allocate(p, it->first, (int64_t)grown.size(), nullptr);
      REQUIRE(r == 0 || r == -1);
      if (r == 0) it->second.tokens = grown;
      else REQUIRE(pkv_pool_num_blocks_of(p, it->first) == before);
    } else if (op == 5 && !live.empty()) {          // enter full blocks into the cache
      auto it = live.begin();
      std::advance(it, rnd(0, (int)live.size() - 1));
      const auto& t = it->second.tokens;
      const int64_t n = rnd(0, (int)t.size());
      const pkv_status st = pkv_pool_cache_full_blocks(p, it->first, t.empty() ? nullptr : t.data(), n);
      REQUIRE(st == PKV_OK || (t.empty() && st == PKV_ERR_NULL));
    } else if (op <= 7 && !live.empty()) {          // release a request
      auto it = live.begin();
      std::advance(it, rnd(0, (int)live.size() - 1));
      REQUIRE(pkv_pool_free(p, it->first) == PKV_OK);
      REQUIRE(pkv_pool_num_blocks_of(p, it->first) == -1);
      REQUIRE(pkv_pool_free(p, it->first) != PKV_OK);   // a second release is refused
      live.erase(it);
    } else if (op == 8) {                           // bad arguments change nothing
      const int64_t nf = pkv_pool_num_free(p);
      REQUIRE(pkv_pool_allocate(p, next_req + 1000, -3, nullptr) == -2);
      REQUIRE(pkv_pool_allocate(nullptr, 1, 3, nullptr) == -2);
      int64_t slots[4];
      REQUIRE(pkv_pool_slot_mapping(p, next_req + 1000, 0, 1, slots) != PKV_OK);
      if (!live.empty()) {
        const auto& [req, r] = *live.begin();
        const int64_t cap = blocks_for((int64_t)r.tokens.size(), bs) * bs;
        REQUIRE(pkv_pool_slot_mapping(p, req, cap, 1, slots) != PKV_OK);
        REQUIRE(pkv_pool_slot_mapping(p, req, -1, 1, slots) != PKV_OK);
        REQUIRE(pkv_pool_slot_mapping(p, req, 0, 1, nullptr) != PKV_OK);
      }
      const int64_t unknown = next_req + 1000;
      int32_t row[4];
      REQUIRE(pkv_pool_block_table(p, &unknown, 1, 4, row) == PKV_ERR_SHAPE);
      REQUIRE(pkv_pool_block_table(p, nullptr, 1, 4, row) != PKV_OK);
      REQUIRE(pkv_pool_num_free(p) == nf);
    } else {                                        // the free queue with a small cap
      int32_t few[3] = {-1, -1, -1};
      const int64_t n = pkv_pool_free_queue(p, few, 2);
      REQUIRE(n == pkv_pool_num_free(p));
      REQUIRE(few[2] == -1);                        // never past the cap
    }
    check(p, live, num_blocks, bs);
  }
  for (const auto& kv : live) REQUIRE(pkv_pool_free(p, kv.first) == PKV_OK);
  REQUIRE(pkv_pool_num_free(p) == num_blocks - 1);
  pkv_pool_destroy(p);
  return 0;
}

}  // namespace

int main() {
  REQUIRE(pkv_pool_create(1, 16, 0) == nullptr);    // bad arguments
  REQUIRE(pkv_pool_create(8, 0, 0) == nullptr);
  pkv_pool_destroy(nullptr);
  uint32_t seed = 1;
  for (int64_t nb : {2, 3, 17, 200})
    for (int32_t bs : {1, 3, 16})
      for (int32_t caching : {0, 1})
        run(nb, bs, caching, seed++, nb <= 3 ? 400 : 1500);
  std::printf("pool stress: ok\n");
  return 0;
}
