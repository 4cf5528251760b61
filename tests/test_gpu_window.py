"""GPU parity of sliding-window attention: decode (VALU, matrix-core and fp8
kernels, split or not), chunked prefill (causal and symmetric), the mixed
one-launch step, exact window edges (a dominant key just inside counts, one
just outside does not) and wide windows, up to the largest int32 width,
equal to none."""
import numpy as np
import pytest

from paged_kv_cache_50_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_50_amd import pagedkv
    pagedkv.lib()
    yield
    torch.cuda.synchronize()


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _run(dw, ps, win):
    from paged_kv_cache_50_amd import pagedkv
    w = dw.w
    if w.slot_mapping is not None:
        pagedkv.kv_cache_write(dw.k_cache, dw.v_cache, dw.key_new, dw.value_new, dw.slot_mapping,
                               k_scale=dw.k_scale, v_scale=dw.v_scale)
    if w.cu_seqlens_q is None:
        pagedkv.paged_attention_decode(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables,
                                       dw.seq_lens, w.scale, w.max_seq_len, partition_size=ps,
                                       lse_out=dw.lse, k_scale=dw.k_scale, v_scale=dw.v_scale,
                                       window_left=win)
    else:
        pagedkv.paged_attention_varlen(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.cu_seqlens_q,
                                       dw.seq_lens, dw.block_tables, w.scale, w.max_query_len,
                                       w.max_seq_len, causal=w.causal, partition_size=ps,
                                       lse_out=dw.lse, k_scale=dw.k_scale, v_scale=dw.v_scale,
                                       window_left=win)


def _reference(w, win):
    import oracle
    kc, vc = G.oracle_inputs(w)
    return oracle.paged_attention(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale, w.block_size,
                                  w.dtype, cu_seqlens_q=w.cu_seqlens_q, causal=w.causal,
                                  k_scale=w.k_scale, v_scale=w.v_scale, window_left=win)


@pytest.mark.parametrize("cfg", [2, 3, 7])
@pytest.mark.parametrize("win", [0, 5, 37, 300])
@pytest.mark.parametrize("ps", [0, -1, 128])
def test_window_decode(cfg, win, ps):
    w = W.make_config(cfg, num_seqs=6, max_len=1500)
    _announce(f"window decode config{cfg} win={win} ps={ps}")
    dw = G.DevWorkload(w)
    _run(dw, ps, win)
    ref, ref_lse = _reference(w, win)
    G.assert_close(G.dev_to_f64(dw.out), ref, w.io_dtype, f"config{cfg} win={win} ps={ps}")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, f"config{cfg} win={win} ps={ps}")


@pytest.mark.parametrize("win", [0, 17, 100, 600])
@pytest.mark.parametrize("ps", [0, -1])
def test_window_mixed_step(win, ps):
    """Chunked prefill + decode rows (the one-launch path when split)."""
    w = W.make_config(5, num_seqs=10, max_len=900, num_chunks=3, chunk_len=77)
    _announce(f"window mixed win={win} ps={ps}")
    dw = G.DevWorkload(w)
    _run(dw, ps, win)
    ref, ref_lse = _reference(w, win)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", f"mixed win={win} ps={ps}")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, f"mixed win={win} ps={ps}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("win", [0, 40, 200])
def test_window_prefill_shapes(causal, win):
    ctx = np.array([0, 130, 700])
    ql = np.array([150, 33, 260])
    w = W.make_varlen("win_prefill", ctx, ql, 16, 4, 128, 16, "bf16", seed=41, causal=causal)
    _announce(f"window prefill causal={causal} win={win}")
    dw = G.DevWorkload(w)
    _run(dw, -1, win)
    ref, ref_lse = _reference(w, win)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", f"prefill causal={causal} win={win}")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, f"prefill causal={causal} win={win}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8)])
@pytest.mark.parametrize("ps", [-1, 128])
def test_window_edges_exact(hq, hkv, ps):
    """A dominant key exactly at the window start is the whole output; the
    same key one position further out is ignored."""
    torch = G.torch()
    win = 50
    L = np.array([400, 130, 64], dtype=np.int32)
    w = W.make_decode("win_edge", L, hq, hkv, 128, 16, "bf16", seed=43)
    w.q[:] = 0
    w.q[:, :, 0] = W.f32_to_bf16_bits(np.float32(64.0))
    bs = 16
    for s, n in enumerate(L):
        blk = w.block_tables[s, np.arange(n) // bs]
        w.k_cache[blk, np.arange(n) % bs, :, 0] = 0
    inside = [int(n) - 1 - win for n in L]
    for s, j in enumerate(inside):
        w.k_cache[w.block_tables[s, j // bs], j % bs, :, 0] = W.f32_to_bf16_bits(np.float32(64.0))
    _announce(f"window edge inside hq={hq} ps={ps}")
    dw = G.DevWorkload(w)
    _run(dw, ps, win)
    torch.cuda.synchronize()
    out = G.dev_to_bits(dw.out)
    g = hq // hkv
    for s, j in enumerate(inside):
        for h in range(hq):
            assert np.array_equal(out[s, h], w.v_cache[w.block_tables[s, j // bs], j % bs, h // g])
    # move each needle one position out of the window: it must not dominate
    for s, j in enumerate(inside):
        w.k_cache[w.block_tables[s, j // bs], j % bs, :, 0] = 0
        jo = j - 1
        w.k_cache[w.block_tables[s, jo // bs], jo % bs, :, 0] = W.f32_to_bf16_bits(np.float32(64.0))
    dw = G.DevWorkload(w)
    _run(dw, ps, win)
    ref, _ = _reference(w, win)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", "needle outside")
    outside_v = np.stack([[G.W.bf16_bits_to_f32(w.v_cache[w.block_tables[s, (j - 1) // bs], (j - 1) % bs,
                                                         h // g]) for h in range(hq)]
                          for s, j in enumerate(inside)]).astype(np.float64)
    assert not np.allclose(G.dev_to_f64(dw.out), outside_v, atol=1e-3)


@pytest.mark.parametrize("cfg", [2, 3, 5, "5nc"])
@pytest.mark.parametrize("wide", ["max_seq_len-1", "max_seq_len+5", "int32_max"])
def test_wide_window_equals_none(cfg, wide):
    """A window of max_seq_len - 1 keys or more excludes no key: the output
    equals the call without a window bit for bit, up to the largest int32
    width (where a position + window sum would leave int32 unless clamped),
    for decode, causal chunked prefill and symmetric (non-causal) rows."""
    torch = G.torch()
    if cfg in (5, "5nc"):
        w = W.make_config(5, num_seqs=8, max_len=900, num_chunks=2, chunk_len=70)
        w.causal = cfg == 5
    else:
        w = W.make_config(cfg, num_seqs=8, max_len=2000)
    win = {"max_seq_len-1": int(w.max_seq_len) - 1, "max_seq_len+5": int(w.max_seq_len) + 5,
           "int32_max": 2**31 - 1}[wide]
    _announce(f"wide window cfg={cfg} window={win}")
    dw = G.DevWorkload(w)
    _run(dw, 0, -1)
    torch.cuda.synchronize()
    a = G.dev_to_bits(dw.out).copy()
    ref, _ = _reference(w, -1)
    G.assert_close(G.dev_to_f64(dw.out), ref, w.dtype, f"no window cfg={cfg}")
    _run(dw, 0, win)
    torch.cuda.synchronize()
    G.assert_close(G.dev_to_f64(dw.out), _reference(w, win)[0], w.dtype, f"window {win} cfg={cfg}")
    assert np.array_equal(G.dev_to_bits(dw.out), a)
