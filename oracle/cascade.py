"""Cascade (shared-prefix) attention in the oracle.

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the product
path; shares no code with the HIP library.

Sources (the vLLM book, ch. 6): "Structure des métadonnées" names the cascade
fields of the attention metadata (use_cascade, common_prefix_len,
cu_prefix_query_lens); "forward()" shows the cascade branch as two attention
calls, one over the shared prefix and one over the rest, whose results are
combined by merge_attn_states; "Réflexion de conception" gives the thresholds
of the decision to use it (a prefix of at least 256 tokens, at least 8
requests, no sliding window, no context parallelism).

Cascade attention computes exactly what plain paged attention computes over
the whole sequences; only the work is regrouped.  The steps, in float64:
  1. prefix: every query row of the batch attends, with no mask, to keys
     0 .. common_prefix_len - 1, read through the shared prefix blocks;
  2. suffix: each row attends to its own sequence's keys common_prefix_len ..
     seq_len - 1 under the usual mask (bottom-right causal);
  3. merge: the two partial results are combined by log-sum-exp
     (merge_partials).

Readings where the pages are silent:
  * common_prefix_len is a whole number of blocks, and every sequence's block
    table starts with the same prefix blocks;
  * the prefix lies in every sequence's context (common_prefix_len <=
    seq_len - query_len), so the causal mask never cuts into it and the
    prefix pass needs none;
  * sequences with seq_len 0 (batch padding) take no part: output 0, lse -inf,
    as in the plain call.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import _seq_rows, attention_seq_kvhead, merge_partials


def check_cascade_metadata(block_tables, seq_lens, cu_seqlens_q, common_prefix_len: int,
                           prefix_blocks, block_size: int) -> None:
    """Raise ValueError when the batch does not meet the cascade readings."""
    cpl = int(common_prefix_len)
    if cpl < 0 or cpl % block_size:
        raise ValueError("common_prefix_len must be a non-negative multiple of block_size")
    nb = cpl // block_size
    prefix_blocks = np.asarray(prefix_blocks)
    if len(prefix_blocks) < nb:
        raise ValueError("prefix block table shorter than the prefix")
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        if L == 0:
            continue
        r0, r1 = _seq_rows(s, cu_seqlens_q)
        if cpl > L - (r1 - r0):
            raise ValueError(f"sequence {s}: prefix longer than its context")
        if not np.array_equal(block_tables[s, :nb], prefix_blocks[:nb]):
            raise ValueError(f"sequence {s}: block table does not start with the prefix blocks")


def cascade_attention(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q,
                      common_prefix_len: int, prefix_blocks, scale: float, block_size: int,
                      dtype: str, causal: bool = True):
    """Cascade attention by the three steps above.  Arguments as for
    paged_attention (cu_seqlens_q None = one row per sequence); prefix_blocks
    lists the physical blocks of the shared prefix.  Returns out
    [num_rows, num_heads, D] and lse [num_rows, num_heads] (natural log)."""
    check_cascade_metadata(block_tables, seq_lens, cu_seqlens_q, common_prefix_len,
                           prefix_blocks, block_size)
    cpl = int(common_prefix_len)
    num_rows, num_heads, D = q.shape
    Hkv = k_cache.shape[2]
    g = num_heads // Hkv
    out = np.zeros((num_rows, num_heads, D))
    lse = np.full((num_rows, num_heads), -np.inf)
    pre_table = np.asarray(prefix_blocks)
    for s in range(len(seq_lens)):
        r0, r1 = _seq_rows(s, cu_seqlens_q)
        L = int(seq_lens[s])
        if r1 <= r0 or L == 0:
            continue
        for kvh in range(Hkv):
            # 1. prefix: no mask (the keys precede every row of the sequence)
            o_pre, l_pre = attention_seq_kvhead(q, k_cache, v_cache, pre_table, cpl, r0, r1, kvh,
                                                num_heads, scale, block_size, dtype, causal=False)
            # 2. suffix: the sequence's own keys under its mask
            o_suf, l_suf = attention_seq_kvhead(q, k_cache, v_cache, block_tables[s], L, r0, r1,
                                                kvh, num_heads, scale, block_size, dtype, causal,
                                                key_range=(cpl, L))
            # 3. merge
            o, l = merge_partials([o_pre, o_suf], [l_pre, l_suf])
            out[r0:r1, kvh * g:(kvh + 1) * g] = o
            lse[r0:r1, kvh * g:(kvh + 1) * g] = l
    return out, lse


def cascade_traffic_bytes(seq_lens, common_prefix_len: int, num_kv_heads: int, head_size: int,
                          elem_bytes: int) -> int:
    """KV bytes the cascade form must read: the prefix once plus every
    sequence's own keys (sequences of length 0 read nothing)."""
    L = np.asarray(seq_lens, dtype=np.int64)
    own = int(np.where(L > 0, L - int(common_prefix_len), 0).sum())
    return (int(common_prefix_len) + own) * 2 * num_kv_heads * head_size * elem_bytes
