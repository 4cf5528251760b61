"""GPU parity of cascade attention whose prefix pass runs on the VALU kernel:
float32 caches, head sizes 64 and 256, and bfloat16 with the VALU row
kernel forced.  Decode rows and batches mixing prefill chunks, each launch
form requested, padding sequences, an exact needle in the shared prefix
across its partitions, against the oracle's plain definition."""
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


def _batch(dtype, head, rows, bs, seed, hq=16, hkv=4, cpl_blocks=40):
    rng = np.random.default_rng(seed)
    cpl = cpl_blocks * bs
    if rows == "decode":
        ql = np.ones(10, dtype=np.int64)
    else:
        ql = np.array([1, 1, 1, 45, 1, 130, 7, 1])
    own = rng.integers(0, 400, size=len(ql))
    ctx = cpl + own
    ctx[2] = 0                                      # a padding sequence: no keys, no rows
    ql[2] = 0
    return W.make_varlen(f"cascade_valu_{dtype}_{head}", ctx, ql, hq, hkv, head, bs, dtype, seed,
                         causal=True, common_prefix_len=cpl)


def _check(w, dw, what):
    ref, ref_lse = G.reference(w)
    tol = w.dtype if w.dtype in ("f32", "f16") else "bf16"
    G.assert_all_rows(G.dev_to_f64(dw.out), G.dev_to_f64(dw.lse), ref, ref_lse, tol, what, w=w)


@pytest.mark.parametrize("dtype,head", [("f32", 128), ("f32", 64), ("f32", 256), ("bf16", 64),
                                        ("bf16", 256), ("f16", 64), ("f16", 256)])
@pytest.mark.parametrize("rows", ["decode", "mixed"])
@pytest.mark.parametrize("cascade_launch", [0, 1])
def test_cascade_valu_prefix(dtype, head, rows, cascade_launch):
    """The prefix pass on the VALU kernel (no one-launch form exists for it,
    so either request runs separate launches), then the suffix pass and the
    merge, for float32, bfloat16 and binary16 caches at head sizes 64, 128
    (float32) and 256."""
    w = _batch(dtype, head, rows, 16, seed=head + 3 * cascade_launch + (rows == "mixed"))
    _announce(f"cascade VALU prefix {dtype} D={head} {rows} launch={cascade_launch}")
    dw = G.DevWorkload(w)
    o = P.CallOptions(cascade_launch=cascade_launch)
    G.run_cascade(dw, options=o)
    assert o.launched & P.RAN_PREFIX and o.launched & P.RAN_CASCADE_MERGE, o.ran()
    assert not o.launched & P.RAN_CASCADE_ONE, o.ran()
    _check(w, dw, f"cascade VALU prefix {dtype} D={head} {rows}")


@pytest.mark.parametrize("rows", ["decode", "mixed"])
def test_cascade_forced_valu_prefix_bf16(rows):
    """bfloat16 at head size 128 with the VALU row kernel requested: the
    prefix pass runs on the VALU kernel instead of the matrix cores."""
    w = _batch("bf16", 128, rows, 32, seed=77 + (rows == "mixed"), hq=32, hkv=8, cpl_blocks=20)
    _announce(f"cascade forced VALU prefix bf16 {rows}")
    dw = G.DevWorkload(w)
    o = P.CallOptions(prefill_kernel=1)
    G.run_cascade(dw, options=o)
    assert o.launched & P.RAN_PREFIX and not o.launched & P.RAN_CASCADE_ONE, o.ran()
    _check(w, dw, f"cascade forced VALU prefix bf16 {rows}")


@pytest.mark.parametrize("head", [64, 256])
def test_cascade_valu_prefix_needle_exact(head):
    """float32: q = 16 e0 for every row and one prefix key = 16 e0, every
    other key 0 in dimension 0 (and q is 0 elsewhere), with a scale that puts
    the needle's logit 2^10 above the rest: the prefix pass finds it in
    whichever partition holds it, and the merged output is its V row bit for
    bit."""
    torch = G.torch()
    bs = 16
    w = _batch("f32", head, "decode", bs, seed=5 + head, cpl_blocks=48)
    cpl = w.common_prefix_len
    w.q[:] = 0
    w.q[:, :, 0] = 16.0
    needle = 500                                      # a key inside the prefix
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        for j in range(L):
            slot = W.slots_of(w.block_tables[s], np.array([j]), bs)[0]
            b, off = divmod(int(slot), bs)
            w.k_cache[b, off][:, 0] = 16.0 if j == needle else 0.0
    w.scale = 4.0                                     # 16 * 16 * 4 = 1024
    _announce(f"cascade VALU prefix needle D={head} cpl={cpl}")
    dw = G.DevWorkload(w)
    G.run_cascade(dw)
    torch.cuda.synchronize()
    got = G.dev_to_bits(dw.out).view(np.uint32)
    g = w.num_heads // w.num_kv_heads
    slot = W.slots_of(w.block_tables[0], np.array([needle]), bs)[0]
    b, off = divmod(int(slot), bs)
    want = np.repeat(w.v_cache[b, off], g, axis=0).view(np.uint32)
    rows = np.flatnonzero(np.diff(w.cu_seqlens_q) > 0)
    for s in rows:
        r = int(w.cu_seqlens_q[s])
        assert np.array_equal(got[r], want), f"sequence {s}"
