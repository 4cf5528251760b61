"""What one GPU can show of the multi-GPU layouts of the long-context decode
(8 sequences of 32k-131k tokens, 64 query / 8 kv heads, head 128, bf16,
512-token partitions).

* Tensor parallelism over heads: with 8 ranks each GPU holds one kv head and
  its 8 query heads of the same block ids, so a rank's cache rows are a
  single head wide (vLLM book, ch. 6 "Transformation de la disposition
  mémoire du KV cache": the per-head stride degenerates).  The rank's
  kernel runs here at that shape, on the matrix cores.
* Context parallelism (the DCP fields of ch. 6 "Structure des métadonnées"):
  each of 8 ranks holds a block-aligned key range of every sequence and
  computes a partial result with its log-sum-exp; the partials are combined
  by the log-sum-exp merge (ch. 6 "forward()", merge_attn_states).  Here the
  8 ranks' decode calls run one after the other on one GPU, each over its own
  block-table slice, and the oracle's merge combines their outputs; the
  collective that would move the partials between GPUs is not part of it.
"""
import numpy as np
import pytest

import oracle
from paged_kv_cache_50_amd import pagedkv
from paged_kv_cache_50_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pagedkv.lib()
    yield
    torch.cuda.synchronize()


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _long_context_lengths():
    """The long-context decode's own sequence lengths (its seed and draw)."""
    meta = np.random.Generator(np.random.PCG64(np.random.SeedSequence(W.DEFAULT_SEEDS[4])))
    return W.config_lengths(4, meta)


def test_tensor_parallel_rank_shard():
    """One TP = 8 rank of the long-context decode: 8 query heads over 1 kv
    head, every (sequence, kv head) pair against the oracle."""
    L = _long_context_lengths()
    w = W.make_decode("tp8_rank_of_long_context", L, 8, 1, 128, 16, "bf16", seed=33, sigma=0.5,
                      partition_size=512)
    _announce(f"TP=8 rank shard: {w.num_seqs} seqs, 8/1 heads, max_seq_len {w.max_seq_len}")
    dw = G.DevWorkload(w)
    o = pagedkv.CallOptions()
    G.run(dw, options=o)
    assert o.launched & pagedkv.RAN_DECODE_MFMA, o.ran()
    ref, ref_lse = G.reference_full(w)
    G.assert_all_rows(G.dev_to_f64(dw.out), G.dev_to_f64(dw.lse), ref, ref_lse, "bf16",
                      "TP=8 rank shard")


@pytest.mark.parametrize("ranks", [8, 3])
def test_context_parallel_ranks_merged(ranks):
    """Each rank decodes against a block-aligned slice of every sequence's
    keys (its own block-table columns and length) and writes out + lse; the
    oracle's log-sum-exp merge of the ranks' outputs equals the oracle's
    attention over the whole sequence."""
    torch = G.torch()
    w = W.make_config(4)
    bs = w.block_size
    _announce(f"context split over {ranks} ranks: {w.num_seqs} seqs, max_seq_len {w.max_seq_len}")
    dw = G.DevWorkload(w)
    S, Hq, D = w.q.shape
    outs, lses = [], []
    for r in range(ranks):
        # rank r holds blocks [b0, b1) of each sequence (a contiguous share)
        nb = -(-w.seq_lens.astype(np.int64) // bs)
        b0 = nb * r // ranks
        b1 = nb * (r + 1) // ranks
        lo = b0 * bs
        hi = np.minimum(b1 * bs, w.seq_lens)
        lens = np.maximum(hi - lo, 0).astype(np.int32)
        width = int((b1 - b0).max())
        bt = np.zeros((S, max(width, 1)), dtype=np.int32)
        for s in range(S):
            bt[s, :b1[s] - b0[s]] = w.block_tables[s, b0[s]:b1[s]]
        out = torch.empty_like(dw.q)
        lse = torch.empty(S, Hq, dtype=torch.float32, device=dw.q.device)
        pagedkv.paged_attention_decode(out, dw.q, dw.k_cache, dw.v_cache,
                                       torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                       w.scale, int(lens.max()), partition_size=512, lse_out=lse)
        outs.append(G.dev_to_f64(out))
        lses.append(G.dev_to_f64(lse))
    merged, merged_lse = oracle.merge_partials(outs, lses)
    ref, ref_lse = G.reference_full(w)
    G.assert_all_rows(merged, merged_lse, ref, ref_lse, "bf16", f"context split x{ranks}")
