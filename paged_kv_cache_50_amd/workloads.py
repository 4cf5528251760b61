"""Seeded synthetic inputs for paged attention.

This module only builds inputs: sequence lengths, a shuffled pool of KV
blocks, block tables, slot mappings and normally distributed q/K/V values.
It performs none of the attention arithmetic, so both the CPU oracle and the
GPU path can consume the same arrays.

Conventions (taken from the vLLM pages):
  * KV cache per layer: separate K and V tensors shaped
    [num_blocks, block_size, num_kv_heads, head_size]
    (vLLM book, ch. 6, "Transformation de la disposition mémoire du KV cache").
  * A block table row lists a sequence's physical block ids; padding entries
    hold the null block id 0, and block 0 is reserved and never holds data
    (vLLM book, ch. 5.2, "slot_mapping et la block table"; ch. 4.1).
  * A sequence of L tokens owns ceil(L / block_size) blocks
    ("Khám phá vLLM", "Scheduler", the allocate_slots example).
  * slot_mapping[t] = physical_block * block_size + offset, int64, -1 marks a
    padded token that must not be written (vLLM book, ch. 5.2).

Random recipe (all integer draws inclusive):
  root = SeedSequence(seed); one metadata stream drawn from root draws the
  lengths and then the block permutation; spawned child streams draw q and,
  per sequence, that sequence's K then V values; the mixed chunked-prefill
  workloads use one more child for the new tokens' K, V and q. Values are standard_normal(float32) * sigma,
  rounded to bfloat16 (bf16 workloads) or IEEE binary16 (f16 workloads) by
  round-to-nearest-even.
Every cache slot that holds no valid token (block 0, spare pool blocks, the
tail of each sequence's last block) is filled with a quiet NaN.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)
F16_QNAN = np.uint16(0x7E00)
E4M3_NAN = np.uint8(0x7F)
F32_QNAN_BITS = np.uint32(0x7FC00000)

# Threads used to draw the per-sequence K/V streams.  The result does not
# depend on this number: every sequence has its own stream.
_GEN_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16 high bits as uint16.  NaN inputs map to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_QNAN
    return r


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (round to nearest, ties to even;
    overflow to infinity, gradual underflow).  Returns the bit patterns as
    uint16.  NaN inputs map to the quiet NaN 0x7E00."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        r = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = F16_QNAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One attention-layer step: cache contents, metadata and queries.

    Floating-point arrays are float32 for dtype 'f32', raw bfloat16 bits
    (uint16) for dtype 'bf16' and raw binary16 bits (uint16) for dtype
    'f16'.  dtype 'fp8': the caches hold e4m3 codes
    (uint8) with per-kv-head float32 scales k_scale / v_scale; q and the new
    key/value rows are bfloat16 bits.
    """
    name: str
    dtype: str                       # 'f32' | 'bf16' | 'f16' | 'fp8'
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    scale: float
    causal: bool
    q: np.ndarray                    # [num_q_rows, num_heads, head_size]
    k_cache: np.ndarray              # [num_blocks, block_size, num_kv_heads, head_size]
    v_cache: np.ndarray
    block_tables: np.ndarray         # int32 [num_seqs, max_blocks]
    seq_lens: np.ndarray             # int32 [num_seqs], context + query tokens
    cu_seqlens_q: Optional[np.ndarray] = None   # int32 [num_seqs + 1]; None = decode (one row per seq)
    key_new: Optional[np.ndarray] = None        # [num_new, num_kv_heads, head_size]
    value_new: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None   # int64 [num_new]
    partition_size: int = 0          # 0 = library default
    sigma: float = 1.0
    k_scale: Optional[np.ndarray] = None        # fp8: float32 [num_kv_heads]
    v_scale: Optional[np.ndarray] = None
    window_left: int = -1            # sliding window (keys pos - window_left .. pos), -1 none
    common_prefix_len: int = 0       # tokens of a prefix shared by every non-empty sequence
                                     # (its blocks start every table)

    @property
    def prefix_blocks(self) -> np.ndarray:
        """int32 [common_prefix_len / block_size]: the shared prefix's blocks."""
        owner = int(np.argmax(self.seq_lens > 0)) if self.seq_lens.size else 0
        return self.block_tables[owner, :self.common_prefix_len // self.block_size].copy()

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def query_lens(self) -> np.ndarray:
        if self.cu_seqlens_q is None:
            return np.ones(self.num_seqs, dtype=np.int32)
        return np.diff(self.cu_seqlens_q).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        ql = self.query_lens
        return int(ql.max()) if ql.size else 0

    @property
    def num_q_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def elem_bytes(self) -> int:
        """Bytes of one cached element."""
        return {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1}[self.dtype]

    @property
    def io_dtype(self) -> str:
        """dtype of q / out / new key and value rows."""
        return "bf16" if self.dtype == "fp8" else self.dtype

    @property
    def io_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def kv_block_bytes(self) -> int:
        """Bytes of one block of one layer, K and V together (2 * bs * Hkv * D * e)."""
        return 2 * self.block_size * self.num_kv_heads * self.head_size * self.elem_bytes

    def valid_slot_mask(self) -> np.ndarray:
        """bool [num_blocks, block_size]: True where the cache holds a token that
        attention may read after the new tokens (if any) have been written."""
        m = np.zeros((self.num_blocks, self.block_size), dtype=bool)
        bs = self.block_size
        for s in range(self.num_seqs):
            L = int(self.seq_lens[s])
            pos = np.arange(L)
            m[self.block_tables[s, pos // bs], pos % bs] = True
        return m


def _poison(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, F32_QNAN_BITS, dtype=np.uint32).view(np.float32)
    if dtype == "fp8":
        return np.full(shape, E4M3_NAN, dtype=np.uint8)
    if dtype == "f16":
        return np.full(shape, F16_QNAN, dtype=np.uint16)
    return np.full(shape, BF16_QNAN, dtype=np.uint16)


def _draw_e4m3_codes(rng: np.random.Generator, n: int) -> np.ndarray:
    """e4m3 codes drawn directly (no rounding of real values): sign U{0,1},
    exponent field clip(rint(N(10, 2)), 1, 15), mantissa U{0..7}; the NaN
    code becomes 0x7E / 0xFE (448)."""
    e = np.clip(np.rint(rng.normal(10.0, 2.0, n)), 1, 15).astype(np.uint8)
    m = rng.integers(0, 8, size=n, dtype=np.uint8)
    sgn = rng.integers(0, 2, size=n, dtype=np.uint8)
    c = (sgn << 7) | (e << 3) | m
    nan = (c & 0x7F) == 0x7F
    c[nan] = (c[nan] & 0x80) | 0x7E
    return c.astype(np.uint8)


def _draw(rng: np.random.Generator, n: int, sigma: float, dtype: str) -> np.ndarray:
    if dtype == "fp8":
        return _draw_e4m3_codes(rng, n)
    x = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _draw_scales(rng: np.random.Generator, num_kv_heads: int, dtype: str):
    """fp8 caches: per-kv-head scales U[0.5, 1) / 32 (float32), K then V."""
    if dtype != "fp8":
        return None, None
    k = (rng.uniform(0.5, 1.0, num_kv_heads) / 32).astype(np.float32)
    v = (rng.uniform(0.5, 1.0, num_kv_heads) / 32).astype(np.float32)
    return k, v


def blocks_needed(seq_len: int, block_size: int) -> int:
    return -(-int(seq_len) // int(block_size))


def build_pool(seq_lens, block_size: int, rng: np.random.Generator,
               num_blocks: Optional[int] = None, extra_frac: float = 0.10,
               shared_blocks: int = 0):
    """Shuffle physical block ids 1..num_blocks-1 and hand them out in order:
    first `shared_blocks` blocks that start every sequence's table (a shared
    prefix), then each sequence's own blocks.  Returns (num_blocks,
    block_tables int32)."""
    nb = [blocks_needed(L, block_size) for L in seq_lens]
    own = [max(0, n - shared_blocks) for n in nb]
    total = int(shared_blocks + sum(own))
    if num_blocks is None:
        num_blocks = 1 + int(math.ceil((1.0 + extra_frac) * total))
    if num_blocks - 1 < total:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {total} blocks")
    perm = rng.permutation(np.arange(1, num_blocks, dtype=np.int64))
    max_blocks = max(nb) if nb else 0
    bt = np.zeros((len(seq_lens), max(max_blocks, 1)), dtype=np.int32)
    pos = shared_blocks
    for s, n in enumerate(nb):
        if n == 0:
            continue
        bt[s, :shared_blocks] = perm[:shared_blocks]
        bt[s, shared_blocks:n] = perm[pos:pos + own[s]]
        pos += own[s]
    return num_blocks, bt


def slots_of(block_table_row: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Flat slot ids (block * block_size + offset) of token positions."""
    positions = np.asarray(positions, dtype=np.int64)
    return block_table_row[positions // block_size].astype(np.int64) * block_size + positions % block_size


def _fill_cache(k_cache, v_cache, block_tables, fill_lens, block_size, child_seeds, sigma, dtype,
                fill_from=None):
    """Write tokens fill_from[s] .. fill_lens[s]-1 (fill_from defaults to 0)
    of every sequence into the pool, K then V, each sequence from its own
    stream."""
    Hkv, D = k_cache.shape[2], k_cache.shape[3]
    kf = k_cache.reshape(-1, Hkv, D)
    vf = v_cache.reshape(-1, Hkv, D)
    chunk_tokens = max(1, (1 << 22) // (Hkv * D))

    def one(s):
        L = int(fill_lens[s])
        lo = 0 if fill_from is None else int(fill_from[s])
        if L <= lo:
            return
        rng = np.random.Generator(np.random.PCG64(child_seeds[s]))
        for cache in (kf, vf):
            for t0 in range(lo, L, chunk_tokens):
                t1 = min(L, t0 + chunk_tokens)
                vals = _draw(rng, (t1 - t0) * Hkv * D, sigma, dtype).reshape(t1 - t0, Hkv, D)
                cache[slots_of(block_tables[s], np.arange(t0, t1), block_size)] = vals

    if len(fill_lens) > 1 and _GEN_THREADS > 1:
        with _cf.ThreadPoolExecutor(_GEN_THREADS) as ex:
            list(ex.map(one, range(len(fill_lens))))
    else:
        for s in range(len(fill_lens)):
            one(s)


def make_decode(name, seq_lens, num_heads, num_kv_heads, head_size, block_size, dtype,
                seed, sigma=1.0, num_blocks=None, partition_size=0, meta_rng=None,
                root=None) -> Workload:
    """Decode step: one query row per sequence; the cache already holds all
    seq_lens[s] tokens (the current token included)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if root is None:
        root = np.random.SeedSequence(seed)
    if meta_rng is None:
        meta_rng = np.random.Generator(np.random.PCG64(root))
    num_blocks, bt = build_pool(seq_lens, block_size, meta_rng, num_blocks)
    children = root.spawn(1 + len(seq_lens))
    q_rng = np.random.Generator(np.random.PCG64(children[0]))
    io = "bf16" if dtype == "fp8" else dtype
    q = _draw(q_rng, len(seq_lens) * num_heads * head_size, sigma, io).reshape(
        len(seq_lens), num_heads, head_size)
    k_scale, v_scale = _draw_scales(q_rng, num_kv_heads, dtype)
    shape = (num_blocks, block_size, num_kv_heads, head_size)
    k_cache = _poison(shape, dtype)
    v_cache = _poison(shape, dtype)
    _fill_cache(k_cache, v_cache, bt, seq_lens, block_size, children[1:], sigma, dtype)
    return Workload(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                    head_size=head_size, block_size=block_size, scale=1.0 / math.sqrt(head_size),
                    causal=False, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=bt,
                    seq_lens=seq_lens, partition_size=partition_size, sigma=sigma,
                    k_scale=k_scale, v_scale=v_scale)


def make_varlen(name, context_lens, query_lens, num_heads, num_kv_heads, head_size, block_size,
                dtype, seed, sigma=1.0, causal=True, num_blocks=None, partition_size=0,
                meta_rng=None, root=None, common_prefix_len: int = 0) -> Workload:
    """Mixed step: sequence s has context_lens[s] tokens already cached and
    query_lens[s] new tokens whose K/V must first be scattered through
    slot_mapping; seq_lens = context + query.

    common_prefix_len > 0 (a whole number of blocks, at most every non-empty
    sequence's context): the first common_prefix_len tokens of every
    non-empty sequence are one shared prefix, held once in blocks that start
    every table and drawn from a stream of their own (spawned child 2 + S)."""
    context_lens = np.asarray(context_lens, dtype=np.int64)
    query_lens = np.asarray(query_lens, dtype=np.int64)
    seq_lens = (context_lens + query_lens).astype(np.int32)
    if root is None:
        root = np.random.SeedSequence(seed)
    if meta_rng is None:
        meta_rng = np.random.Generator(np.random.PCG64(root))
    cpl = int(common_prefix_len)
    if cpl % block_size or cpl < 0:
        raise ValueError("common_prefix_len must be a non-negative multiple of block_size")
    if cpl and np.any((seq_lens > 0) & (context_lens < cpl)):
        raise ValueError("the shared prefix must lie in every sequence's context")
    num_blocks, bt = build_pool(seq_lens, block_size, meta_rng, num_blocks,
                                shared_blocks=cpl // block_size)
    S = len(seq_lens)
    children = root.spawn(2 + S + (1 if cpl else 0))
    shape = (num_blocks, block_size, num_kv_heads, head_size)
    k_cache = _poison(shape, dtype)
    v_cache = _poison(shape, dtype)
    if cpl:
        owner = int(np.argmax(seq_lens > 0))           # any sequence holding the prefix
        _fill_cache(k_cache, v_cache, bt[owner:owner + 1], [cpl], block_size, children[2 + S:],
                    sigma, dtype)
    _fill_cache(k_cache, v_cache, bt, context_lens, block_size, children[2:2 + S], sigma, dtype,
                fill_from=np.where(seq_lens > 0, cpl, 0))
    T = int(query_lens.sum())
    new_rng = np.random.Generator(np.random.PCG64(children[1]))
    io = "bf16" if dtype == "fp8" else dtype
    key_new = _draw(new_rng, T * num_kv_heads * head_size, sigma, io).reshape(T, num_kv_heads, head_size)
    value_new = _draw(new_rng, T * num_kv_heads * head_size, sigma, io).reshape(T, num_kv_heads, head_size)
    q = _draw(new_rng, T * num_heads * head_size, sigma, io).reshape(T, num_heads, head_size)
    k_scale, v_scale = _draw_scales(new_rng, num_kv_heads, dtype)
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(query_lens)
    slot = np.empty(T, dtype=np.int64)
    for s in range(S):
        pos = np.arange(context_lens[s], seq_lens[s])
        slot[cu[s]:cu[s + 1]] = slots_of(bt[s], pos, block_size)
    return Workload(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                    head_size=head_size, block_size=block_size, scale=1.0 / math.sqrt(head_size),
                    causal=causal, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=bt,
                    seq_lens=seq_lens, cu_seqlens_q=cu, key_new=key_new, value_new=value_new,
                    slot_mapping=slot, partition_size=partition_size, sigma=sigma,
                    k_scale=k_scale, v_scale=v_scale, common_prefix_len=cpl)


# --------------------------------------------------------------------------
# The five workloads.  `scale_down` shrinks batch and lengths for parity runs
# while keeping head shapes, block size, dtype and length distribution shape.
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny_mha_decode_f32",
    2: "llama7b_mha_decode_bf16",
    3: "gqa_decode_bf16",
    4: "long_context_splitkv_decode_bf16",
    5: "mixed_chunked_prefill_decode_bf16",
    6: "llama7b_mha_decode_fp8",
    7: "gqa_decode_fp8",
    8: "long_context_sliding_window_decode_bf16",
    9: "shared_prefix_cascade_decode_bf16",
    10: "mixed_chunked_prefill_decode_fp8",
    11: "gqa_decode_f16",
    12: "mixed_chunked_prefill_decode_f16",
}

# 6, 7, 11: the lengths and pools of 2, 3, 3; 10, 12: those of 5
DEFAULT_SEEDS = {1: 0, 2: 1, 3: 2, 4: 3, 5: 4, 6: 1, 7: 2, 8: 3, 9: 5, 10: 4, 11: 2, 12: 4}


def config_lengths(cfg: int, rng: np.random.Generator, num_seqs=None, max_len=None):
    """Sequence lengths of a workload, drawn from the metadata stream."""
    if cfg == 1:
        n = num_seqs or 4
        return rng.integers(1, min(256, max_len or 256), size=n, endpoint=True)
    if cfg == 2:
        n = num_seqs or 64
        hi = min(4096, max_len or 4096)
        return rng.integers(min(200, hi), hi, size=n, endpoint=True)
    if cfg == 3:
        n = num_seqs or 256
        z = rng.standard_normal(n)
        L = np.rint(np.exp(math.log(1024.0) + 0.8 * z))
        return np.clip(L, 16, min(8192, max_len or 8192)).astype(np.int64)
    if cfg == 4:
        n = num_seqs or 8
        hi = min(131072, max_len or 131072)
        return rng.integers(min(32768, hi // 4), hi, size=n, endpoint=True)
    raise ValueError(cfg)


def make_config(cfg: int, seed: Optional[int] = None, num_seqs: Optional[int] = None,
                max_len: Optional[int] = None, num_chunks: Optional[int] = None,
                chunk_len: Optional[int] = None) -> Workload:
    """Build workload `cfg` (1..12).  num_seqs / max_len / num_chunks /
    chunk_len shrink it for quick parity runs; None keeps the full size."""
    if seed is None:
        seed = DEFAULT_SEEDS[cfg]
    root = np.random.SeedSequence(seed)
    meta = np.random.Generator(np.random.PCG64(root))
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        L = config_lengths(1, meta, num_seqs, max_len)
        return make_decode(name, L, 8, 8, 64, 16, "f32", seed, num_blocks=128,
                           meta_rng=meta, root=root)
    if cfg == 2:
        L = config_lengths(2, meta, num_seqs, max_len)
        return make_decode(name, L, 32, 32, 128, 16, "bf16", seed, meta_rng=meta, root=root)
    if cfg == 3:
        L = config_lengths(3, meta, num_seqs, max_len)
        return make_decode(name, L, 32, 8, 128, 16, "bf16", seed, meta_rng=meta, root=root)
    if cfg == 4:
        L = config_lengths(4, meta, num_seqs, max_len)
        return make_decode(name, L, 64, 8, 128, 16, "bf16", seed, sigma=0.5,
                           partition_size=512, meta_rng=meta, root=root)
    if cfg in (5, 10, 12):
        # 10, 12: the same step over an fp8 or a binary16 cache (same lengths
        # and pool)
        nc = 4 if num_chunks is None else num_chunks
        cl = 512 if chunk_len is None else chunk_len
        nd = 128 if num_seqs is None else num_seqs
        ctx_hi = 4096 if max_len is None else min(4096, max_len)
        dec_hi = 4096 if max_len is None else min(4096, max_len)
        ctx = meta.integers(0, ctx_hi, size=nc, endpoint=True)
        dec_L = meta.integers(min(64, dec_hi), dec_hi, size=nd, endpoint=True)
        context = np.concatenate([ctx, dec_L - 1]).astype(np.int64)
        qlens = np.concatenate([np.full(nc, cl), np.ones(nd)]).astype(np.int64)
        return make_varlen(name, context, qlens, 32, 8, 128, 32, {5: "bf16", 10: "fp8", 12: "f16"}[cfg],
                           seed, causal=True, meta_rng=meta, root=root)
    if cfg == 8:
        # the shapes, lengths and pool of workload 4 with a 4096-key window
        L = config_lengths(4, meta, num_seqs, max_len)
        w = make_decode(name, L, 64, 8, 128, 16, "bf16", seed, sigma=0.5,
                        partition_size=512, meta_rng=meta, root=root)
        w.window_left = 4095
        return w
    if cfg == 9:
        # decode rows of requests that share one prefix (a long system
        # prompt): the GQA shapes of workload 3, a 4096-token prefix, then
        # U{0..1023} tokens of each request's own context and its new token
        n = 256 if num_seqs is None else num_seqs
        cpl = 4096 if max_len is None else max(16, min(4096, (max_len // 2) // 16 * 16))
        own_hi = 1023 if max_len is None else max(0, min(1023, max_len - cpl - 1))
        own = meta.integers(0, own_hi, size=n, endpoint=True)
        context = (cpl + own).astype(np.int64)
        return make_varlen(name, context, np.ones(n, dtype=np.int64), 32, 8, 128, 16, "bf16",
                           seed, causal=True, meta_rng=meta, root=root, common_prefix_len=cpl)
    if cfg in (6, 7):
        # the MHA and GQA decode shapes of workloads 2 and 3 over an fp8 cache
        L = config_lengths(cfg - 4, meta, num_seqs, max_len)
        hq, hkv = (32, 32) if cfg == 6 else (32, 8)
        return make_decode(name, L, hq, hkv, 128, 16, "fp8", seed, meta_rng=meta, root=root)
    if cfg == 11:
        # the GQA decode step of workload 3 over a binary16 cache
        L = config_lengths(3, meta, num_seqs, max_len)
        return make_decode(name, L, 32, 8, 128, 16, "f16", seed, meta_rng=meta, root=root)
    raise ValueError(cfg)


# --------------------------------------------------------------------------
# Algorithmic byte and flop counts (what the method must move / compute).
# --------------------------------------------------------------------------

def algorithmic_bytes(w: Workload, include_write: bool = True, shared_prefix: bool = True) -> int:
    """KV bytes of every valid token read once, plus q, out, block-table
    entries and seq_lens; for a mixed step also the new K/V read and written
    and the slot_mapping read.  A shared prefix (common_prefix_len > 0) is
    counted once, as the cascade form reads it; shared_prefix=False counts it
    once per sequence, as the plain form does."""
    e = w.elem_bytes
    L = w.seq_lens.astype(np.int64)
    if w.window_left >= 0 and w.cu_seqlens_q is None:
        # a decode row reads only the keys of its window, and the table
        # entries of the blocks they lie in
        first = np.maximum(L - 1 - w.window_left, 0)
        keys = L - first
        blocks = (L + w.block_size - 1) // w.block_size - first // w.block_size
    else:
        keys = L
        blocks = np.array([blocks_needed(x, w.block_size) for x in L], dtype=np.int64)
    if shared_prefix and w.common_prefix_len > 0:
        cpl = w.common_prefix_len
        holders = int((L > 0).sum())
        keys = np.append(keys - np.where(L > 0, cpl, 0), cpl if holders else 0)
        blocks = np.append(blocks - np.where(L > 0, cpl // w.block_size, 0),
                           cpl // w.block_size if holders else 0)
    kv = int(keys.sum()) * 2 * w.num_kv_heads * w.head_size * e
    qo = 2 * w.num_q_rows * w.num_heads * w.head_size * w.io_bytes
    meta = 4 * int(blocks.sum()) + 4 * w.num_seqs
    if w.cu_seqlens_q is not None:
        meta += 4 * (w.num_seqs + 1)
    if w.k_scale is not None:
        meta += 2 * 4 * w.num_kv_heads
    total = kv + qo + meta
    if include_write and w.slot_mapping is not None:
        T = int(w.slot_mapping.shape[0])
        total += 2 * T * w.num_kv_heads * w.head_size * (w.io_bytes + e) + 8 * T
    return total


def prefix_flops(w: Workload) -> int:
    """Flops of the cascade prefix pass: every query row against the shared
    prefix (2 flops per multiply-add over QK^T and PV)."""
    return 4 * w.num_q_rows * w.num_heads * w.head_size * int(w.common_prefix_len)


def attention_flops(w: Workload) -> int:
    """2 flops per multiply-add over QK^T and PV for the scores each query
    row actually uses (causal rows stop at their own position)."""
    ql = w.query_lens.astype(np.int64)
    L = w.seq_lens.astype(np.int64)
    total = 0
    for s in range(w.num_seqs):
        if w.causal and w.cu_seqlens_q is not None:
            ctx = L[s] - ql[s]
            keys = int(ql[s] * ctx + ql[s] * (ql[s] + 1) // 2)
        else:
            keys = int(ql[s] * L[s])
        total += 4 * w.num_heads * w.head_size * keys
    return total


# --------------------------------------------------------------------------
# Device copies of a workload (for the GPU tests, the smoke check and the
# benchmark): the same arrays, moved as raw bits.
# --------------------------------------------------------------------------

def np_to_dev(x: np.ndarray, dtype: str, device="cuda"):
    """A device tensor holding the bits of x: bfloat16 bits (uint16) as
    torch.bfloat16, binary16 bits as torch.float16, e4m3 codes (uint8) as
    torch.float8_e4m3fn, else as is."""
    import torch as t
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(t.bfloat16).to(device)
    if dtype == "f16":
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(t.float16).to(device)
    if dtype == "fp8":
        return t.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(device).view(t.float8_e4m3fn)
    return t.from_numpy(np.ascontiguousarray(x)).to(device)


class DevWorkload:
    """Device copies of a Workload's tensors."""

    def __init__(self, w: Workload, device="cuda"):
        import torch as t
        self.w = w
        self.q = np_to_dev(w.q, w.io_dtype, device)
        self.k_cache = np_to_dev(w.k_cache, w.dtype, device)
        self.v_cache = np_to_dev(w.v_cache, w.dtype, device)
        self.block_tables = t.from_numpy(w.block_tables).to(device)
        self.seq_lens = t.from_numpy(w.seq_lens).to(device)
        self.cu_seqlens_q = None if w.cu_seqlens_q is None else t.from_numpy(w.cu_seqlens_q).to(device)
        self.key_new = None if w.key_new is None else np_to_dev(w.key_new, w.io_dtype, device)
        self.value_new = None if w.value_new is None else np_to_dev(w.value_new, w.io_dtype, device)
        self.k_scale = None if w.k_scale is None else t.from_numpy(w.k_scale).to(device)
        self.v_scale = None if w.v_scale is None else t.from_numpy(w.v_scale).to(device)
        self.slot_mapping = None if w.slot_mapping is None else t.from_numpy(w.slot_mapping).to(device)
        self.prefix_blocks = (t.from_numpy(w.prefix_blocks).to(device)
                              if w.common_prefix_len > 0 else None)
        self.out = t.empty_like(self.q)
        self.lse = t.empty(self.q.shape[0], self.q.shape[1], dtype=t.float32, device=device)
