"""CPU oracle for paged attention and the KV-cache slot write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module; only the test suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library.

It is the plain definition of what the paged kernels compute, in float64:
gather each sequence's KV blocks through its block table into contiguous K and
V, then evaluate softmax(scale * q K^T) V row by row.  Paging moves the data
around; it does not change the mathematics, so the oracle never blocks, fuses
or reorders beyond that definition.

Sources (the vLLM pages):
  * cache layout [num_blocks, block_size, num_kv_heads, head_size], K and V
    separate: vLLM book, ch. 6, "Transformation de la disposition mémoire du
    KV cache";
  * block table rows padded with the null block 0: ch. 5.2, "slot_mapping et
    la block table";
  * slot scatter, token count taken from slot_mapping, slot -1 skipped:
    ch. 6, "Écriture du KV cache : do_kv_cache_update", and ch. 5.2;
  * seq_len = context_len + query_len, query_start_loc prefix sums: ch. 6,
    "Structure des métadonnées";
  * causal alignment: query index i of a chunk of q_len rows sits at absolute
    position i + seq_len - q_len: ch. 6, "Branche de masque";
  * partial results of a split key range are merged: ch. 6, "forward()"
    (merge_attn_states) and "build() étape par étape" (the split buffer);
  * sliding window: a causal window (w, 0) becomes (w, w) when the
    attention is not causal: ch. 6, "forward()" (the window symmetrisation);
    the cache still holds every token, only the computation is windowed
    (ch. 2, "Le système de spécifications du KV Cache": conservative
    allocation, exact computation).

  * element formats: the flash-attention backend takes fp16 and bf16
    models, and its caches may also be fp8: ch. 6, "Sélection du backend",
    "Matrice de capacités : les champs comme contrat"; stored values are
    widened exactly (IEEE binary16 here from its own definition).

Readings where the pages are silent (each is pinned by a test):
  * slot = physical_block * block_size + offset;
  * query head h uses kv head h // (num_heads // num_kv_heads);
  * a row that sees no key (seq_len 0) has output 0 and lse -inf;
  * the merge of partial results is the max-shifted log-sum-exp combination.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from .fp8 import e4m3_decode


def binary16_decode(bits: np.ndarray) -> np.ndarray:
    """Value of IEEE 754 binary16 bit patterns (uint16), in float64, from
    the format's definition: 1 sign bit, 5 exponent bits with bias 15, 10
    fraction bits; exponent field 0 holds zero and the subnormals
    (fraction * 2^-24), field 31 the infinities (fraction 0) and NaNs."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, f * 2.0 ** -24, (1.0 + f / 1024.0) * np.exp2(e - 15.0))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements: float32 arrays, bfloat16 bit
    patterns (uint16) whose value is the float32 with those high bits,
    binary16 bit patterns (uint16), or e4m3 codes (uint8; the value before
    the per-head scale)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return binary16_decode(x)
    if dtype == "fp8":
        return e4m3_decode(x)
    raise ValueError(dtype)


def kv_cache_write(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray,
                   value: np.ndarray, slot_mapping: np.ndarray, block_size: int) -> None:
    """Scatter new K/V rows into the caches in place.

    The number of tokens is len(slot_mapping); key/value may hold extra
    padded rows, which are ignored.  A negative slot means "padding, write
    nothing".  Elements are copied bit for bit.
    """
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        k_cache[blk, off] = key[t]
        v_cache[blk, off] = value[t]


def gather_kv(cache: np.ndarray, block_table_row: np.ndarray, seq_len: int,
              block_size: int, kv_head: Optional[int] = None) -> np.ndarray:
    """Logical tokens 0..seq_len-1 of one sequence, in order, as stored.

    Token j lives in physical block block_table_row[j // block_size] at
    offset j % block_size.  Only the first ceil(seq_len / block_size) table
    entries are used.
    """
    nb = -(-seq_len // block_size)
    ids = np.asarray(block_table_row[:nb], dtype=np.int64)
    if kv_head is None:
        blocks = cache[ids]                                # [nb, bs, Hkv, D]
    else:
        blocks = cache[ids, :, kv_head, :]                 # [nb, bs, D]
    return blocks.reshape((nb * block_size,) + blocks.shape[2:])[:seq_len]


def _softmax_rows(S: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Textbook row softmax of logits S [R, L] (entries -inf are masked out)
    applied to V [L, D].  Returns (out [R, D], lse [R]); rows with no finite
    logit give out 0 and lse -inf."""
    R = S.shape[0]
    out = np.zeros((R, V.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if S.shape[1] == 0:
        return out, lse
    m = S.max(axis=1)
    ok = np.isfinite(m)
    if not ok.any():
        return out, lse
    P = np.exp(S[ok] - m[ok, None])
    l = P.sum(axis=1)
    out[ok] = (P @ V) / l[:, None]
    lse[ok] = m[ok] + np.log(l)
    return out, lse


def _seq_rows(s: int, cu_seqlens_q: Optional[np.ndarray]) -> Tuple[int, int]:
    if cu_seqlens_q is None:
        return s, s + 1
    return int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])


def attention_seq_kvhead(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                         block_table_row: np.ndarray, seq_len: int, row0: int, row1: int,
                         kv_head: int, num_heads: int, scale: float, block_size: int,
                         dtype: str, causal: bool,
                         key_range: Optional[Tuple[int, int]] = None,
                         k_scale=None, v_scale=None, window_left: int = -1):
    """Attention of query rows row0..row1-1 of one sequence for the query
    heads of one kv head.  key_range=(a, b) restricts the keys to logical
    positions a..b-1 (used to express a split).  window_left >= 0 is a
    sliding window: a row at position p sees keys p - w .. p when causal and
    p - w .. p + w otherwise (the causal window made symmetric).  dtype is
    the cache's; with
    an fp8 cache the queries are bfloat16 and cached values are
    decode(code) * k_scale[kv_head] (v_scale for V).  Returns out
    [q_len, g, D] and lse [q_len, g] in float64."""
    Hkv = k_cache.shape[2]
    g = num_heads // Hkv
    q_len = row1 - row0
    D = q.shape[2]
    L = int(seq_len)
    K = widen(gather_kv(k_cache, block_table_row, L, block_size, kv_head), dtype)  # [L, D]
    V = widen(gather_kv(v_cache, block_table_row, L, block_size, kv_head), dtype)
    if dtype == "fp8":
        K = K * float(np.float32(k_scale[kv_head]))
        V = V * float(np.float32(v_scale[kv_head]))
    qdtype = "bf16" if dtype == "fp8" else dtype
    Q = widen(q[row0:row1, kv_head * g:(kv_head + 1) * g], qdtype)                # [q_len, g, D]
    S = scale * (Q.reshape(q_len * g, D) @ K.T)                                   # [q_len*g, L]
    S = S.reshape(q_len, g, L)
    j = np.arange(L)
    allowed = np.ones((q_len, L), dtype=bool)
    qpos = np.arange(q_len) + L - q_len              # absolute position of each query row
    if causal:
        allowed &= j[None, :] <= qpos[:, None]
    if window_left is not None and window_left >= 0:
        allowed &= j[None, :] >= qpos[:, None] - window_left
        if not causal:
            allowed &= j[None, :] <= qpos[:, None] + window_left
    if key_range is not None:
        allowed &= (j >= key_range[0]) & (j < key_range[1])
    S = np.where(allowed[:, None, :], S, -np.inf)
    out, lse = _softmax_rows(S.reshape(q_len * g, L), V)
    return out.reshape(q_len, g, D), lse.reshape(q_len, g)


def paged_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    block_tables: np.ndarray, seq_lens: np.ndarray, scale: float,
                    block_size: int, dtype: str, cu_seqlens_q: Optional[np.ndarray] = None,
                    causal: bool = False,
                    pairs: Optional[Sequence[Tuple[int, int]]] = None,
                    k_scale=None, v_scale=None, window_left: int = -1):
    """Attention over a paged KV cache, as defined above.

    q: [num_rows, num_heads, D]; decode when cu_seqlens_q is None (row s is
    sequence s), else sequence s owns rows cu_seqlens_q[s]..cu_seqlens_q[s+1]-1.
    pairs: optional list of (seq, kv_head) to evaluate; other rows stay NaN.
    dtype "fp8": e4m3 caches with per-kv-head scales k_scale / v_scale.
    Returns out [num_rows, num_heads, D] and lse [num_rows, num_heads], float64
    (lse in natural log).
    """
    num_rows, num_heads, D = q.shape
    Hkv = k_cache.shape[2]
    if num_heads % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    g = num_heads // Hkv
    out = np.full((num_rows, num_heads, D), np.nan, dtype=np.float64)
    lse = np.full((num_rows, num_heads), np.nan, dtype=np.float64)
    if pairs is None:
        pairs = [(s, h) for s in range(len(seq_lens)) for h in range(Hkv)]
    for s, kvh in pairs:
        r0, r1 = _seq_rows(s, cu_seqlens_q)
        if r1 <= r0:
            continue
        o, l = attention_seq_kvhead(q, k_cache, v_cache, block_tables[s], int(seq_lens[s]),
                                    r0, r1, kvh, num_heads, scale, block_size, dtype, causal,
                                    k_scale=k_scale, v_scale=v_scale, window_left=window_left)
        out[r0:r1, kvh * g:(kvh + 1) * g] = o
        lse[r0:r1, kvh * g:(kvh + 1) * g] = l
    return out, lse


def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Combine attention results computed over disjoint key ranges.

    With lse_p the log-sum-exp of partition p's logits and o_p its normalised
    output: LSE = log(sum_p exp(lse_p)), o = sum_p exp(lse_p - LSE) * o_p,
    evaluated with the maximum subtracted.  Partitions with lse -inf carry
    no weight; if all are -inf the result is 0 with LSE -inf.
    """
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])       # [P, ...]
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])       # [P, ..., D]
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Msafe), 0.0)
    tot = w.sum(axis=0)
    o = np.where(finite[..., None],
                 (w[..., None] * np.nan_to_num(outs)).sum(axis=0) / np.where(tot > 0, tot, 1.0)[..., None],
                 0.0)
    LSE = np.where(finite, Msafe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return o, LSE


def split_attention(q, k_cache, v_cache, block_tables, seq_lens, scale, block_size, dtype,
                    partition_size: int, cu_seqlens_q=None, causal=False):
    """The same attention evaluated as a split over key partitions
    [p*P, (p+1)*P) and merged with merge_partials.  Used to test that a split
    followed by the merge is exact, not to produce reference outputs."""
    num_rows, num_heads, D = q.shape
    Hkv = k_cache.shape[2]
    g = num_heads // Hkv
    out = np.zeros((num_rows, num_heads, D))
    lse = np.full((num_rows, num_heads), -np.inf)
    for s in range(len(seq_lens)):
        r0, r1 = _seq_rows(s, cu_seqlens_q)
        L = int(seq_lens[s])
        nparts = max(1, -(-L // partition_size))
        for kvh in range(Hkv):
            parts = [attention_seq_kvhead(q, k_cache, v_cache, block_tables[s], L, r0, r1, kvh,
                                          num_heads, scale, block_size, dtype, causal,
                                          key_range=(p * partition_size, (p + 1) * partition_size))
                     for p in range(nparts)]
            o, l = merge_partials([p[0] for p in parts], [p[1] for p in parts])
            out[r0:r1, kvh * g:(kvh + 1) * g] = o
            lse[r0:r1, kvh * g:(kvh + 1) * g] = l
    return out, lse


def block_bytes(block_size: int, num_kv_heads: int, head_size: int, dtype_bytes: int) -> int:
    """Bytes of one KV block of one standard attention layer, K and V
    together ("Khám phá vLLM", LLM Engine & Engine Core, §1 note)."""
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Blocks a request of num_tokens needs: ceil(num_tokens / block_size)
    ("Khám phá vLLM", Scheduler, allocate_slots)."""
    return -(-int(num_tokens) // int(block_size))
