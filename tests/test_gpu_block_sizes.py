"""Blocks of 64 and 128 tokens, larger than the kernels' 32-token key tile,
on every kernel: decode (VALU, matrix cores, fp8 one or two kv heads per
wave), chunked prefill on both kernels, the mixed one-launch step, the
cascade in both launch forms, sliding windows and the slot write.

Two checks for each case: parity with the oracle, and bit-identity with the
same logical batch stored in blocks of 16 (or 32) tokens.  The generator
draws the same values for the same logical positions whatever the block
size (only the placement in the pool differs), and the kernels' arithmetic
order depends on logical positions only, so the outputs and log-sum-exps
must agree bit for bit."""
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


def _tol(w):
    return w.dtype if w.dtype in ("f32", "f16") else "bf16"


def _run_both(make, bs_small, bs_large, what, ps=None, opts=None, cascade=False):
    """Run the batch make(bs) at both block sizes; check the large one
    against the oracle and bit for bit against the small one."""
    outs = []
    for bs in (bs_small, bs_large):
        w = make(bs)
        dw = G.DevWorkload(w)
        o = P.CallOptions(**(opts or {}))
        if cascade:
            G.run_cascade(dw, partition_size=ps, options=o)
        else:
            G.run(dw, partition_size=ps, options=o)
        outs.append((w, G.dev_to_bits(dw.out), G.dev_to_f64(dw.out), G.dev_to_f64(dw.lse), o.launched))
    (ws, bits_s, _, lse_s, ran_s), (wl, bits_l, out_l, lse_l, ran_l) = outs
    ref, ref_lse = G.reference(wl)
    G.assert_all_rows(out_l, lse_l, ref, ref_lse, _tol(wl), f"{what} bs={bs_large}", w=wl)
    assert ran_s == ran_l, (what, P.CallOptions(launched=ran_s).ran(), P.CallOptions(launched=ran_l).ran())
    owned = ~np.isnan(ref_lse)
    assert np.array_equal(bits_s[owned], bits_l[owned]), f"{what}: bs {bs_small} and {bs_large} differ"
    assert np.array_equal(lse_s[owned], lse_l[owned]), f"{what}: lse differs across block sizes"


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f16", "f32"])
def test_large_block_kv_write_bit_exact(bs, dtype):
    torch = G.torch()
    w = W.make_varlen("bs_write", [5, 200, 0, 130], [3, 1, 70, 2], 8, 2, 128 if dtype != "f32" else 64,
                      bs, dtype, seed=bs)
    kc, vc = G.oracle_inputs(w)
    _announce(f"kv write bs={bs} {dtype}")
    dk, dv = G.np_to_dev(w.k_cache, dtype), G.np_to_dev(w.v_cache, dtype)
    ks = None if w.k_scale is None else torch.from_numpy(w.k_scale).cuda()
    vs = None if w.v_scale is None else torch.from_numpy(w.v_scale).cuda()
    pagedkv.kv_cache_write(dk, dv, G.np_to_dev(w.key_new, w.io_dtype), G.np_to_dev(w.value_new, w.io_dtype),
                           torch.from_numpy(w.slot_mapping).cuda(), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert np.array_equal(G.dev_to_bits(dk).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(G.dev_to_bits(dv).view(np.uint8), vc.view(np.uint8))


DECODE = [
    # (dtype, num_heads, num_kv_heads, head_size, options): the kernels these take
    ("bf16", 8, 8, 128, {}),                         # VALU MHA
    ("bf16", 32, 8, 128, {}),                        # matrix-core GQA
    ("bf16", 32, 8, 128, {"decode_kernel": 1}),      # VALU GQA
    ("f16", 32, 8, 128, {}),
    ("f16", 16, 16, 64, {}),                         # head 64 (VALU)
    ("f32", 8, 2, 64, {}),
    ("f32", 4, 4, 128, {}),
    ("fp8", 32, 8, 128, {}),                         # two kv heads per wave
    ("fp8", 32, 8, 128, {"fp8_head_pairs": 1}),      # one kv head per wave
    ("fp8", 24, 3, 128, {}),                         # odd kv heads: one per wave
]


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("case", DECODE, ids=[f"{c[0]}-{c[1]}x{c[2]}-D{c[3]}-{c[4]}" for c in DECODE])
@pytest.mark.parametrize("ps", [0, -1, 96])
def test_large_block_decode(bs, case, ps):
    """Lengths below, at and past block boundaries, and an empty row;
    partitions of 96 tokens do not divide the blocks."""
    dtype, hq, hkv, D, opts = case
    lens = [1, 31, 32, 63, 64, 65, 127, 128, 129, 700, 1500, 0]
    _announce(f"large-block decode bs={bs} {case} ps={ps}")
    _run_both(lambda b: W.make_decode("bs_dec", lens, hq, hkv, D, b, dtype, seed=hq + hkv + D),
              16, bs, f"decode {case} ps={ps}", ps=ps, opts=opts)


PREFILL = [("bf16", {}), ("bf16", {"prefill_kernel": 1}), ("fp8", {}), ("f16", {}),
           ("f16", {"prefill_kernel": 1})]


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("case", PREFILL, ids=[f"{c[0]}-{c[1]}" for c in PREFILL])
@pytest.mark.parametrize("causal", [True, False])
def test_large_block_prefill(bs, case, causal):
    """Chunks with contexts that start mid-block, a ragged last tile, and
    decode rows and an empty sequence beside them (split rows, so the mixed
    one-launch form for the default options)."""
    dtype, opts = case
    ctx = [0, 100, 1000, 5, 700, 0, 2000]
    ql = [130, 77, 1, 200, 1, 0, 1]
    _announce(f"large-block prefill bs={bs} {case} causal={causal}")
    _run_both(lambda b: W.make_varlen("bs_pre", ctx, ql, 32, 8, 128, b, dtype, seed=11,
                                      causal=causal),
              32, bs, f"prefill {case} causal={causal}", opts=opts)


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f16"])
@pytest.mark.parametrize("mixed_launch", [0, 1])
def test_large_block_mixed_step(bs, dtype, mixed_launch):
    """The mixed chunked-prefill step's shapes, shrunk, at large blocks."""
    def make(b):
        rng = np.random.default_rng(5)
        ctx = np.concatenate([rng.integers(0, 1500, 3), rng.integers(64, 1500, 30) - 1])
        ql = np.concatenate([np.full(3, 150), np.ones(30, dtype=np.int64)])
        return W.make_varlen("bs_mixed", ctx, ql, 32, 8, 128, b, dtype, seed=4, causal=True)
    _announce(f"large-block mixed step bs={bs} {dtype} launch={mixed_launch}")
    _run_both(make, 32, bs, f"mixed {dtype} launch={mixed_launch}",
              opts={"mixed_launch": mixed_launch})


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f16"])
@pytest.mark.parametrize("cascade_launch", [0, 1])
@pytest.mark.parametrize("rows", ["decode", "mixed"])
def test_large_block_cascade(bs, dtype, cascade_launch, rows):
    """Cascades whose shared prefix is a whole number of 128-token blocks."""
    cpl = 512
    if rows == "decode":
        ctx = cpl + np.random.default_rng(3).integers(0, 600, 12)
        ql = np.ones(12, dtype=np.int64)
    else:
        ctx = np.array([cpl + 40, cpl + 7, cpl, cpl + 300])
        ql = np.array([1, 60, 1, 130])
    _announce(f"large-block cascade bs={bs} {dtype} {rows} launch={cascade_launch}")
    _run_both(lambda b: W.make_varlen("bs_cascade", ctx, ql, 32, 8, 128, b, dtype, seed=19,
                                      common_prefix_len=cpl),
              16, bs, f"cascade {dtype} {rows} launch={cascade_launch}",
              opts={"cascade_launch": cascade_launch}, cascade=True)


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("win", [0, 37, 300])
def test_large_block_window(bs, win):
    """Sliding windows whose start falls anywhere in a large block: decode
    rows on both decode kernels and prefill rows."""
    for hq, hkv, causal in ((32, 8, True), (8, 8, True), (16, 4, False)):
        def make(b):
            w = W.make_varlen("bs_win", [0, 1200, 500, 64], [90, 1, 1, 33], hq, hkv, 128, b, "bf16",
                              seed=win + hq, causal=causal)
            w.window_left = win
            return w
        _announce(f"large-block window bs={bs} win={win} {hq}/{hkv} causal={causal}")
        _run_both(make, 16, bs, f"window {win} {hq}/{hkv} causal={causal}")


@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("hq,hkv,ps", [(8, 8, -1), (32, 8, -1), (32, 8, 128), (32, 8, 0)])
def test_large_block_needle_exact(bs, hq, hkv, ps):
    """A key that dominates its row at positions on both sides of block and
    tile boundaries: the output is that token's V row, bit for bit."""
    lens = [130, 300, 1024, 257]
    positions = [[0, 31, 32, 63, 64, 127, 128, 129], [95, 96, 255, 256, 299],
                 [511, 512, 1023], [192, 193, 256]]
    torch = G.torch()
    for s_pick in range(max(len(p) for p in positions)):
        w = W.make_decode("bs_needle", lens, hq, hkv, 128, bs, "bf16", seed=bs + hq + ps)
        one = np.uint16(0x4280)                      # 64.0 in bfloat16
        w.q[:] = 0
        w.q[:, :, 0] = one
        needles = [p[min(s_pick, len(p) - 1)] for p in positions]
        for s, L in enumerate(lens):
            for j in range(L):
                slot = W.slots_of(w.block_tables[s], np.array([j]), w.block_size)[0]
                b, o = divmod(int(slot), w.block_size)
                w.k_cache[b, o][:, 0] = one if j == needles[s] else 0
        _announce(f"large-block needle bs={bs} {hq}/{hkv} ps={ps} at {needles}")
        dw = G.DevWorkload(w)
        G.run(dw, partition_size=ps)
        got = G.dev_to_bits(dw.out)
        g = hq // hkv
        for s in range(len(lens)):
            slot = W.slots_of(w.block_tables[s], np.array([needles[s]]), w.block_size)[0]
            b, o = divmod(int(slot), w.block_size)
            assert np.array_equal(got[s], np.repeat(w.v_cache[b, o], g, axis=0)), (s, needles[s])
        del dw
        torch.cuda.synchronize()


N_RANDOM = 48


def draw_large_block_case(i: int):
    """A random small batch at block size 64 or 128: dtype, head size, heads,
    decode or varlen rows, causality, window, partition size, one forced
    variant."""
    rng = np.random.default_rng(90_000 + i)
    bs = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f32", "bf16", "f16", "fp8"]))
    head = 128 if dtype == "fp8" else int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    S = int(rng.integers(1, 11))
    decode = bool(rng.random() < 0.4)
    causal = bool(rng.random() < 0.75)
    if decode:
        L = rng.integers(0, 1600, S)
        w = W.make_decode(f"bs_random{i}", L, hkv * group, hkv, head, bs, dtype, seed=91_000 + i)
    else:
        ctx = rng.integers(0, 1500, S)
        ql = np.where(rng.random(S) < 0.5, 1, rng.integers(2, 130, S))
        w = W.make_varlen(f"bs_random{i}", ctx, ql, hkv * group, hkv, head, bs, dtype,
                          seed=91_000 + i, causal=causal)
    if rng.random() < 0.3:
        w.window_left = int(rng.integers(0, 700))
    ps = int(rng.choice([0, -1, 32, 96, 256]))
    opts = [{}, {"decode_kernel": 1}, {"decode_kernel": 2}, {"prefill_kernel": 1},
            {"mixed_launch": 1}][int(rng.integers(0, 5))]
    desc = (f"large-block case {i}: bs{bs} {dtype} D{head} {hkv * group}/{hkv} heads, {S} seqs, "
            f"{'decode' if decode else 'varlen'}, causal {causal}, window {w.window_left}, "
            f"ps {ps}, options {opts}")
    return w, ps, opts, desc


@pytest.mark.parametrize("i", range(N_RANDOM))
def test_large_block_random(i):
    w, ps, opts, desc = draw_large_block_case(i)
    print(f"[gpu-test] {desc}", flush=True)
    dw = G.DevWorkload(w)
    G.run(dw, partition_size=ps, options=P.CallOptions(**opts))
    ref, ref_lse = G.reference(w)
    G.assert_all_rows(G.dev_to_f64(dw.out), G.dev_to_f64(dw.lse), ref, ref_lse, _tol(w), desc, w=w)
