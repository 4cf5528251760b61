"""Every launch variant a call's options can force, against the oracle, and
the report of the kernels each call launched (pkv_call_options).

The library picks one variant per call; the others stay available for A/B
measurements.  Each forced variant must meet the same tolerances, and its
report must name the kernels that ran, so that a benchmark's label and byte
count follow what actually ran.
"""
import numpy as np
import pytest

from paged_kv_cache_50_amd import pagedkv
from paged_kv_cache_50_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
P = pagedkv


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


def _check(w, dw, opts, want, ps, what, key_span=None):
    """Parity with the oracle, and the report: exactly the kernels in `want`,
    plus the split merge only when the key range is split.  (Whether a split
    batch needs the merge launch depends on the launch geometry: a row whose
    partitions all fall to one workgroup is finished by it.)"""
    ref, ref_lse = G.reference(w)
    tol = w.dtype if w.dtype in ("f32", "f16") else "bf16"
    G.assert_close(G.dev_to_f64(dw.out), ref, tol, what, w=w)
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, what)
    assert opts.launched & ~P.RAN_SPLIT_MERGE == want, (what, opts.ran())
    span = w.max_seq_len if key_span is None else key_span
    split = pagedkv.choose_partition_size(w.num_seqs, w.num_heads, w.num_kv_heads, span, ps)
    if split <= 0 or span <= split:
        assert not opts.launched & P.RAN_SPLIT_MERGE, (what, opts.ran())


CASES = [
    # (workload, shrink kwargs, partition_size, options, expected kernels other
    # than the split merge)
    (2, dict(num_seqs=6, max_len=1500), 0, {}, P.RAN_DECODE_MFMA),
    (2, dict(num_seqs=6, max_len=1500), 0, dict(decode_kernel=1),
     P.RAN_DECODE_VALU),
    (2, dict(num_seqs=6, max_len=1500), -1, dict(decode_kernel=2), P.RAN_DECODE_MFMA),
    (3, dict(num_seqs=70, max_len=1200), 0, {},
     P.RAN_PLANNER | P.RAN_DECODE_MFMA),
    (3, dict(num_seqs=70, max_len=1200), 0, dict(decode_kernel=1),
     P.RAN_DECODE_VALU),
    (3, dict(num_seqs=10, max_len=1200), 128, {}, P.RAN_DECODE_MFMA),
    (6, dict(num_seqs=6, max_len=1500), 0, {},
     P.RAN_DECODE_MFMA | P.RAN_DECODE_PAIRS),
    (6, dict(num_seqs=6, max_len=1500), 0, dict(fp8_head_pairs=1),
     P.RAN_DECODE_MFMA),
    (6, dict(num_seqs=6, max_len=1500), 0, dict(decode_kernel=1),       # no VALU fp8 kernel
     P.RAN_DECODE_MFMA | P.RAN_DECODE_PAIRS),
    (5, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, {},
     P.RAN_PLANNER | P.RAN_MIXED),
    (5, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, dict(mixed_launch=1),
     P.RAN_PREFILL_MFMA | P.RAN_DECODE_MFMA),
    (5, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, dict(prefill_kernel=1),
     P.RAN_PREFILL_VALU | P.RAN_DECODE_MFMA),
    (5, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), -1, {},
     P.RAN_PREFILL_MFMA | P.RAN_DECODE_MFMA),
    (10, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, {},
     P.RAN_PLANNER | P.RAN_MIXED),
    (10, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, dict(mixed_launch=1),
     P.RAN_PREFILL_MFMA | P.RAN_DECODE_MFMA | P.RAN_DECODE_PAIRS),
    # binary16 caches: the same choices as bfloat16
    (11, dict(num_seqs=70, max_len=1200), 0, {},
     P.RAN_PLANNER | P.RAN_DECODE_MFMA),
    (11, dict(num_seqs=70, max_len=1200), 0, dict(decode_kernel=1),
     P.RAN_DECODE_VALU),
    (11, dict(num_seqs=10, max_len=1200), 128, {}, P.RAN_DECODE_MFMA),
    (12, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, {},
     P.RAN_PLANNER | P.RAN_MIXED),
    (12, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, dict(mixed_launch=1),
     P.RAN_PREFILL_MFMA | P.RAN_DECODE_MFMA),
    (12, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0, dict(prefill_kernel=1),
     P.RAN_PREFILL_VALU | P.RAN_DECODE_MFMA),
    (12, dict(num_seqs=9, max_len=900, num_chunks=2, chunk_len=70), 0,
     dict(prefill_kernel=1, decode_kernel=1), P.RAN_PREFILL_VALU | P.RAN_DECODE_VALU),
]


@pytest.mark.parametrize("cfg,kw,ps,opts,want", CASES,
                         ids=[f"w{c[0]}-ps{c[2]}-{'-'.join(f'{k}{v}' for k, v in c[3].items()) or 'default'}"
                              for c in CASES])
def test_forced_variant_matches_oracle_and_is_reported(cfg, kw, ps, opts, want):
    w = W.make_config(cfg, **kw)
    _announce(f"variant workload {cfg} {kw} ps={ps} {opts}")
    dw = G.DevWorkload(w)
    o = P.CallOptions(**opts)
    G.run(dw, partition_size=ps, options=o)
    _check(w, dw, o, want, ps, f"workload {cfg} {opts} ps={ps}")


@pytest.mark.parametrize("cascade_launch", [0, 1])
def test_cascade_launch_forms(cascade_launch):
    w = W.make_config(9, num_seqs=20, max_len=1400)
    _announce(f"cascade launch form {cascade_launch}")
    dw = G.DevWorkload(w)
    o = P.CallOptions(cascade_launch=cascade_launch)
    G.run_cascade(dw, options=o)
    want = (P.RAN_PLANNER | P.RAN_CASCADE_ONE | P.RAN_CASCADE_MERGE if cascade_launch == 0
            else P.RAN_PREFIX | P.RAN_DECODE_MFMA | P.RAN_CASCADE_MERGE)
    _check(w, dw, o, want, 0, f"cascade launch {cascade_launch}",
           key_span=w.max_seq_len - (w.common_prefix_len // 32 * 32))


def test_report_is_per_call():
    """The report describes the call it was passed to, nothing earlier."""
    w = W.make_config(3, num_seqs=5, max_len=700)
    dw = G.DevWorkload(w)
    o = P.CallOptions()
    G.run(dw, partition_size=-1, options=o)
    assert o.launched == P.RAN_DECODE_MFMA
    o.decode_kernel = 1
    G.run(dw, partition_size=-1, options=o)
    assert o.launched == P.RAN_DECODE_VALU
    o.decode_kernel = 0
    with pytest.raises(pagedkv.PagedKVError):
        G.run(dw, partition_size=-1, options=P.CallOptions(decode_kernel=3))


def test_binding_refuses_bad_buffers():
    """The binding refuses, before any launch, buffers the kernels would
    write or read past: an overlapping (expanded) workspace that claims more
    bytes than it spans, a workspace too small for the split, an lse_out in
    another dtype, and prefix_blocks shorter than the shared prefix; the
    call with proper buffers still matches the oracle afterwards."""
    torch = G.torch()
    w = W.make_config(3, num_seqs=6, max_len=1500)
    dw = G.DevWorkload(w)
    need = P.workspace_bytes(6, 32, 8, 128, int(w.max_seq_len), 512)
    assert need > 0
    args = (dw.out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.seq_lens, w.scale,
            int(w.max_seq_len))
    over = torch.empty(1, dtype=torch.uint8, device="cuda").expand(need)
    with pytest.raises(ValueError, match="workspace"):
        P.paged_attention_decode(*args, partition_size=512, workspace=over)
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PagedKVError):
        P.paged_attention_decode(*args, partition_size=512, workspace=small)
    bad_lse = torch.empty(6, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="lse_out"):
        P.paged_attention_decode(*args, partition_size=512, lse_out=bad_lse)
    c = W.make_config(9, num_seqs=8, max_len=600)
    dc = G.DevWorkload(c)
    nb = c.common_prefix_len // c.block_size
    short = torch.from_numpy(c.prefix_blocks[:nb - 1].copy()).cuda()
    with pytest.raises(ValueError, match="prefix_blocks"):
        P.cascade_attention(dc.out, dc.q, dc.k_cache, dc.v_cache, dc.cu_seqlens_q, dc.seq_lens,
                            dc.block_tables, short, c.common_prefix_len, c.scale,
                            c.max_query_len, int(c.max_seq_len))
    torch.cuda.synchronize()
    G.run(dw, partition_size=512)
    ref, ref_lse = G.reference(w)
    G.assert_all_rows(G.dev_to_f64(dw.out), G.dev_to_f64(dw.lse), ref, ref_lse, "bf16",
                      "after refusals", w=w)
