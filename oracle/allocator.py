"""Reference model of the KV block allocator (the step that produces block
tables and slot mappings).

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the product
path; shares no code with the C++ allocator in the library.

It follows the block pool of the vLLM book, ch. 4.1 "Structures de données
du planificateur" and 4.4 "Détermination des touches du cache de préfixe et
cycle de vie des blocs", and the allocate_slots steps of «Khám phá vLLM»,
"Scheduler":
  * the pool's free blocks form a queue in eviction order; at start it holds
    every block in id order, and the first block taken from its head becomes
    the null block (id 0), a placeholder that is never handed out or freed;
  * taking n new blocks pops them from the head of the queue; a taken block
    that still carries a prefix-cache hash loses it (evicted from the cache)
    and gets reference count 1;
  * freeing a request releases its blocks last to first; a block whose count
    drops to 0 goes back to the HEAD of the queue when it has no hash (LIFO
    reuse) and to the TAIL when it has one (FIFO, so cached blocks are evicted
    least recently used first);
  * a prefix-cache hit "touches" a block: out of the free queue if it was in
    it, count + 1;
  * a request of n tokens owns ceil(n / block_size) blocks;
  * at most num_tokens - 1 tokens of a new request may come from the cache
    (the last token is always computed);
  * full blocks are entered into the cache by a hash chained over the
    previous block's hash and the block's token ids; when a hash is already
    present the existing entry is kept.
Readings where the pages are silent: the hash is 64-bit FNV-1a over the
parent hash (8 bytes, little endian; 0 for the first block) followed by the
block's token ids (int32, little endian); a request that cannot get all its
blocks changes nothing; capacity counts free blocks minus the cache hits that
sit in the free queue.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(parent: int, tokens: Sequence[int]) -> int:
    data = int(parent).to_bytes(8, "little")
    for t in tokens:
        data += int(t).to_bytes(4, "little", signed=True)
    return fnv1a64(data)


class BlockPoolModel:
    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True):
        if num_blocks < 2 or block_size <= 0:
            raise ValueError("need at least two blocks and a positive block size")
        self.bs = block_size
        self.caching = prefix_caching
        self.free: List[int] = list(range(num_blocks))        # head = index 0
        self.ref = [0] * num_blocks
        self.hash: List[Optional[int]] = [None] * num_blocks
        self.cache: Dict[int, int] = {}                        # hash -> block
        self.null_block = self.free.pop(0)
        self.req_blocks: Dict[int, List[int]] = {}
        self.req_cached: Dict[int, int] = {}                   # full blocks already hashed
        self.req_hashes: Dict[int, List[int]] = {}

    # -- pool primitives
    def num_free(self) -> int:
        return len(self.free)

    def _take(self, n: int) -> List[int]:
        out = []
        for _ in range(n):
            b = self.free.pop(0)
            if self.hash[b] is not None:
                if self.cache.get(self.hash[b]) == b:
                    del self.cache[self.hash[b]]
                self.hash[b] = None
            self.ref[b] = 1
            out.append(b)
        return out

    def _touch(self, blocks: Sequence[int]) -> None:
        for b in blocks:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1

    def _release(self, blocks: Sequence[int]) -> None:
        for b in reversed(list(blocks)):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if self.hash[b] is None:
                    self.free.insert(0, b)
                else:
                    self.free.append(b)

    def _cache_hits(self, token_ids: Sequence[int], num_tokens: int) -> List[int]:
        hits, parent = [], 0
        max_blocks = (num_tokens - 1) // self.bs
        for i in range(max_blocks):
            h = block_hash(parent, token_ids[i * self.bs:(i + 1) * self.bs])
            b = self.cache.get(h)
            if b is None:
                break
            hits.append(b)
            parent = h
        return hits

    # -- requests
    def allocate(self, req: int, num_tokens: int, token_ids: Optional[Sequence[int]] = None) -> int:
        """Make request `req` own blocks for num_tokens tokens.  Returns the
        number of leading tokens found in the prefix cache (new requests
        only), or -1 when the pool cannot provide the blocks."""
        blocks = self.req_blocks.get(req)
        hits: List[int] = []
        if blocks is None and self.caching and token_ids is not None and num_tokens > 0:
            hits = self._cache_hits(token_ids, num_tokens)
        have = len(blocks) if blocks is not None else len(hits)
        need = max(0, -(-num_tokens // self.bs) - have)
        evictable_hits = sum(1 for b in hits if self.ref[b] == 0)
        if need > self.num_free() - evictable_hits:
            return -1
        if blocks is None:
            self._touch(hits)
            blocks = list(hits)
            self.req_blocks[req] = blocks
            self.req_cached[req] = len(hits)
            self.req_hashes[req] = []
            parent = 0
            for i in range(len(hits)):
                parent = block_hash(parent, token_ids[i * self.bs:(i + 1) * self.bs])
                self.req_hashes[req].append(parent)
        blocks.extend(self._take(need))
        return len(hits) * self.bs

    def cache_full_blocks(self, req: int, token_ids: Sequence[int], num_tokens: int) -> None:
        if not self.caching:
            return
        blocks = self.req_blocks[req]
        hashes = self.req_hashes[req]
        full = min(num_tokens // self.bs, len(blocks))
        for i in range(self.req_cached[req], full):
            parent = hashes[i - 1] if i > 0 else 0
            h = block_hash(parent, token_ids[i * self.bs:(i + 1) * self.bs])
            hashes.append(h)
            b = blocks[i]
            if self.hash[b] is None:
                self.hash[b] = h
                self.cache.setdefault(h, b)
        self.req_cached[req] = max(self.req_cached[req], full)

    def free_request(self, req: int) -> None:
        blocks = self.req_blocks.pop(req)
        self.req_cached.pop(req)
        self.req_hashes.pop(req)
        self._release(blocks)

    def block_table(self, reqs: Sequence[int], max_blocks: int) -> List[List[int]]:
        rows = []
        for r in reqs:
            b = self.req_blocks[r]
            if len(b) > max_blocks:
                raise ValueError("max_blocks too small")
            rows.append(b + [self.null_block] * (max_blocks - len(b)))
        return rows

    def slot_mapping(self, req: int, first_pos: int, count: int) -> List[int]:
        b = self.req_blocks[req]
        return [b[p // self.bs] * self.bs + p % self.bs for p in range(first_pos, first_pos + count)]
