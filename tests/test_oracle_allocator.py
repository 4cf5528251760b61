"""Pins of the allocator reference model: hand-worked sequences that follow
the pages' rules (null block first, ceil(n / block_size) blocks, LIFO reuse of
unhashed blocks, FIFO eviction of hashed ones, prefix-cache hits capped at
n - 1 tokens, all-or-nothing allocation) and invariants under random use."""
import random

import pytest

from oracle.allocator import BlockPoolModel, block_hash, fnv1a64


def test_fnv1a_reference_values():
    # published FNV-1a 64-bit test vectors
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_null_block_and_ceil_blocks():
    p = BlockPoolModel(10, 16, prefix_caching=False)
    assert p.null_block == 0 and p.num_free() == 9
    assert p.allocate(7, 17) == 0                 # 17 tokens -> ceil(17/16) = 2 blocks
    assert p.req_blocks[7] == [1, 2]
    assert p.allocate(7, 32) == 0                 # still 2 blocks
    assert p.req_blocks[7] == [1, 2]
    assert p.allocate(7, 33) == 0
    assert p.req_blocks[7] == [1, 2, 3]
    assert p.block_table([7], 5) == [[1, 2, 3, 0, 0]]
    assert p.slot_mapping(7, 15, 3) == [1 * 16 + 15, 2 * 16 + 0, 2 * 16 + 1]


def test_unhashed_blocks_are_reused_lifo():
    p = BlockPoolModel(10, 16, prefix_caching=False)
    p.allocate(1, 48)                             # blocks 1, 2, 3
    p.allocate(2, 16)                             # block 4
    p.free_request(1)
    assert p.free[:4] == [1, 2, 3, 5]
    p.allocate(3, 20)
    assert p.req_blocks[3] == [1, 2]


def test_hashed_blocks_go_to_the_tail_and_are_evicted_last_block_first():
    p = BlockPoolModel(8, 4)
    toks = list(range(10))                        # 2 full blocks + 2 tokens
    p.allocate(1, 10, toks)                       # blocks 1, 2, 3
    p.cache_full_blocks(1, toks, 10)
    p.free_request(1)
    # 3 (no hash) at the head; then 2, 1 appended to the tail in release order
    assert p.free[0] == 3 and p.free[-2:] == [2, 1]
    assert len(p.cache) == 2
    # new request with other tokens: takes from the head: 3, 4, ...
    p.allocate(2, 8, [100 + i for i in range(8)])
    assert p.req_blocks[2] == [3, 4]
    # exhaust the free list until the hashed blocks are reused: 2 is evicted first
    p.allocate(3, 4 * 3, [200 + i for i in range(12)])   # 5, 6, 7
    p.allocate(4, 4, [300 + i for i in range(4)])        # 2 (evicted from the cache)
    assert p.req_blocks[4] == [2]
    assert p.hash[2] is None and len(p.cache) == 1


def test_prefix_hit_reuses_blocks_and_caps_at_n_minus_1():
    p = BlockPoolModel(16, 4)
    toks = list(range(12))
    p.allocate(1, 12, toks)
    p.cache_full_blocks(1, toks, 12)              # 3 full blocks cached
    # a second request with the same 12 tokens: at most 11 may be cached -> 2 blocks
    assert p.allocate(2, 12, toks) == 8
    assert p.req_blocks[2][:2] == p.req_blocks[1][:2]
    assert p.ref[p.req_blocks[1][0]] == 2
    # a longer request sharing the first 2 blocks: 8 tokens cached
    assert p.allocate(3, 20, toks[:8] + [999] * 12) == 8
    assert p.req_blocks[3][:2] == p.req_blocks[1][:2]
    # a hit on freed (queued) blocks takes them out of the free queue
    p.free_request(1)
    p.free_request(2)
    p.free_request(3)
    b0 = p.cache[block_hash(0, toks[:4])]
    assert b0 in p.free
    assert p.allocate(4, 9, toks[:9]) == 8
    assert b0 not in p.free and p.ref[b0] == 1


def test_allocation_is_all_or_nothing():
    p = BlockPoolModel(6, 8, prefix_caching=False)   # 5 usable blocks
    p.allocate(1, 24)
    snap = (list(p.free), list(p.ref), dict(p.req_blocks))
    assert p.allocate(2, 24) == -1                    # needs 3, 2 left
    assert (list(p.free), list(p.ref), dict(p.req_blocks)) == snap
    assert p.allocate(1, 40) == 0                     # grows by exactly the 2 left
    assert p.num_free() == 0 and p.allocate(9, 1) == -1


def _check_invariants(p: BlockPoolModel):
    owned = {}
    for blocks in p.req_blocks.values():
        for b in blocks:
            owned[b] = owned.get(b, 0) + 1
    assert len(p.free) == len(set(p.free))
    assert p.null_block not in p.free and p.null_block not in owned
    for b in range(len(p.ref)):
        if b == p.null_block:
            continue
        assert p.ref[b] == owned.get(b, 0)
        assert (b in p.free) == (p.ref[b] == 0)
    for h, b in p.cache.items():
        assert p.hash[b] == h


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants_under_random_use(seed):
    rng = random.Random(seed)
    p = BlockPoolModel(40, 4)
    live = {}
    prompts = [[rng.randrange(50) for _ in range(rng.randrange(1, 30))] for _ in range(6)]
    for step in range(400):
        op = rng.random()
        if op < 0.45:
            r = step
            toks = list(rng.choice(prompts)) + [rng.randrange(50) for _ in range(rng.randrange(0, 6))]
            if p.allocate(r, len(toks), toks) >= 0:
                live[r] = toks
        elif op < 0.75 and live:
            r = rng.choice(sorted(live))
            live[r].append(rng.randrange(50))
            if p.allocate(r, len(live[r])) >= 0:
                p.cache_full_blocks(r, live[r], len(live[r]))
        elif live:
            r = rng.choice(sorted(live))
            p.free_request(r)
            del live[r]
        _check_invariants(p)
