"""GPU parity of the fp8 (e4m3) KV cache: the quantising slot write against
the oracle bit for bit, decode attention against the oracle within the
bfloat16 tolerances, exact needle indexing, and identity with the bfloat16
path when the scales are powers of two."""
import numpy as np
import pytest

import oracle
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


def _decode_rows_varlen(seed=21, n=40, max_len=900):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, max_len, size=n)
    return W.make_varlen("fp8_rows", ctx, np.ones(n, dtype=np.int64), 32, 8, 128, 16, "fp8", seed)


def test_fp8_kv_write_bit_exact():
    torch = G.torch()
    w = _decode_rows_varlen()
    key, val = w.key_new.copy(), w.value_new.copy()
    # special inputs: saturation, NaN, signed zero, tiny values, plus 3 padded rows
    key[0, 0, :4] = [0x4700, 0xC700, 0x7FC0, 0x8000]        # 32768, -32768, NaN, -0.0
    key[1, 1, :3] = [0x0001, 0x8001, 0x3A80]                # tiny +-, 9.8e-4
    val[2, 3, :2] = [0x7F7F, 0xFF7F]                        # +-max bfloat16
    slots = w.slot_mapping.copy()
    slots[[5, 17]] = -1
    pad = np.full((3,) + key.shape[1:], 0x4000, dtype=np.uint16)
    key = np.concatenate([key, pad])
    val = np.concatenate([val, pad])
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_cache_write_fp8(kc, vc, key, val, slots, w.block_size, w.k_scale, w.v_scale)
    _announce(f"fp8 kv_write T={len(slots)}")
    from paged_kv_cache_50_amd import pagedkv
    dk = G.np_to_dev(w.k_cache, "fp8")
    dv = G.np_to_dev(w.v_cache, "fp8")
    pagedkv.kv_cache_write(dk, dv, G.np_to_dev(key, "bf16"), G.np_to_dev(val, "bf16"),
                           torch.from_numpy(slots).cuda(), k_scale=torch.from_numpy(w.k_scale).cuda(),
                           v_scale=torch.from_numpy(w.v_scale).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(G.dev_to_bits(dk), kc)
    assert np.array_equal(G.dev_to_bits(dv), vc)


@pytest.mark.parametrize("cfg", [6, 7])
@pytest.mark.parametrize("ps", [0, -1, 128])
def test_fp8_decode_small(cfg, ps):
    w = W.make_config(cfg, num_seqs=6, max_len=1500)
    _announce(f"fp8 config{cfg} small ps={ps} seq_lens={list(w.seq_lens)}")
    dw = G.DevWorkload(w)
    G.run(dw, partition_size=ps)
    ref, ref_lse = G.reference(w)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", f"fp8 config{cfg} ps={ps}")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, f"fp8 config{cfg} ps={ps}")


@pytest.mark.parametrize("hq,hkv,bs", [(8, 2, 16), (16, 4, 8), (32, 8, 32), (12, 3, 16),
                                       (40, 2, 16), (5, 5, 16), (32, 32, 16)])
@pytest.mark.parametrize("ps", [0, 128])
def test_fp8_decode_head_layouts(hq, hkv, bs, ps):
    """Every kv-head layout of the fp8 decode kernel: pairs of adjacent kv
    heads read by one wave (an even count with at most 16 query heads per kv
    head), one kv head per wave otherwise (an odd count, or query-head chunks
    of 16), with per-head scales that differ, and block sizes 8, 16 and 32."""
    lens = [1, 37, 300, 513, 1024, 777]
    w = W.make_decode("fp8_heads", lens, hq, hkv, 128, bs, "fp8", seed=hq * 7 + hkv + bs)
    assert len(set(w.k_scale.tolist())) == hkv or hkv == 1
    _announce(f"fp8 decode heads {hq}/{hkv} bs={bs} ps={ps}")
    dw = G.DevWorkload(w)
    G.run(dw, partition_size=ps)
    ref, ref_lse = G.reference(w)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", f"fp8 heads {hq}/{hkv} bs={bs} ps={ps}")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, f"fp8 heads {hq}/{hkv} bs={bs} ps={ps}")


@pytest.mark.parametrize("ps", [-1, 128])
def test_fp8_needle_bit_exact(ps):
    """q = 64 e0 and one key = 64 e0 (code 0x68, scale 1): the needle's
    logit dominates by far, every other probability underflows to 0, and
    the output is that token's V row times a power-of-two scale, exactly."""
    w = W.make_decode("fp8_needle", [300, 77, 513], 8, 2, 128, 16, "fp8", seed=31)
    w.k_scale = np.ones(2, dtype=np.float32)
    w.v_scale = np.full(2, 2.0 ** -5, dtype=np.float32)
    w.q[:] = 0
    w.q[:, :, 0] = W.f32_to_bf16_bits(np.float32(64.0))
    needles = [257, 16, 512]
    # the needles' V rows hold every finite code (2 kv heads x 128 dims), so
    # the kernels' e4m3 -> bfloat16 conversion is checked code by code; -0
    # (0x80) is left out: an output summed from a +0 start reads +0
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0x80, 0xFF]] = 0
    for s, L in enumerate(w.seq_lens):
        blk = w.block_tables[s, np.arange(L) // 16]
        off = np.arange(L) % 16
        w.k_cache[blk, off, :, 0] = 0                          # every key orthogonal to e0
        j = needles[s]
        w.k_cache[w.block_tables[s, j // 16], j % 16, :, 0] = 0x68   # 64.0
        w.v_cache[w.block_tables[s, j // 16], j % 16] = np.roll(codes, 37 * s).reshape(2, 128)
    _announce(f"fp8 needle ps={ps}")
    dw = G.DevWorkload(w)
    G.run(dw, partition_size=ps)
    out = G.dev_to_bits(dw.out)
    for s, j in enumerate(needles):
        blk, off = w.block_tables[s, j // 16], j % 16
        for h in range(8):
            v = oracle.e4m3_decode(w.v_cache[blk, off, h // 4]) * 2.0 ** -5
            assert np.array_equal(out[s, h], W.f32_to_bf16_bits(v.astype(np.float32))), (s, h)


@pytest.mark.parametrize("ps", [-1, 256])
def test_fp8_equals_bf16_path_with_power_of_two_scales(ps):
    """The same values held as e4m3 codes with power-of-two scales or as
    bfloat16: with one partition per row (the same split of the keys over the
    waves) the two kernels' outputs are bit-identical.  Split rows may group
    their partitions into different workgroup ranges (the fp8 launch reads
    two kv heads per wave and has its own workgroup count), so there the
    merge order may differ and the outputs agree within the tolerance."""
    torch = G.torch()
    w8 = W.make_config(7, num_seqs=10, max_len=2500)
    w8.k_scale = np.full(w8.num_kv_heads, 2.0 ** -6, dtype=np.float32)
    w8.v_scale = np.full(w8.num_kv_heads, 2.0 ** -4, dtype=np.float32)
    kb = W.f32_to_bf16_bits((oracle.e4m3_decode(w8.k_cache) * 2.0 ** -6).astype(np.float32))
    vb = W.f32_to_bf16_bits((oracle.e4m3_decode(w8.v_cache) * 2.0 ** -4).astype(np.float32))
    kb[w8.k_cache == 0x7F] = W.BF16_QNAN                       # poison stays poison
    vb[w8.v_cache == 0x7F] = W.BF16_QNAN
    import dataclasses
    wb = dataclasses.replace(w8, dtype="bf16", k_cache=kb, v_cache=vb, k_scale=None, v_scale=None)
    _announce(f"fp8 vs bf16 identity ps={ps}")
    d8, db = G.DevWorkload(w8), G.DevWorkload(wb)
    G.run(d8, partition_size=ps)
    G.run(db, partition_size=ps, options=dict(decode_kernel=2))
    torch.cuda.synchronize()
    if ps == -1:
        assert np.array_equal(G.dev_to_bits(d8.out), G.dev_to_bits(db.out))
    G.assert_close(G.dev_to_f64(d8.out), G.dev_to_f64(db.out), "bf16", "fp8 vs bf16")


def test_fp8_varlen_decode_rows_with_write():
    w = _decode_rows_varlen(seed=22, n=30, max_len=2000)
    _announce(f"fp8 varlen rows + write, {w.num_seqs} seqs")
    dw = G.DevWorkload(w)
    G.run(dw, partition_size=256)
    ref, ref_lse = G.reference(w)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", "fp8 varlen rows")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, "fp8 varlen rows")


def _fp8_mixed(hq, hkv, bs, causal, seed, cpl=0):
    rng = np.random.default_rng(seed)
    ql = np.array([1] * 6 + [37, 150, 64, 3])
    ctx = cpl + rng.integers(0, 400, size=len(ql))
    return W.make_varlen("fp8_mixed", ctx, ql, hq, hkv, 128, bs, "fp8", seed, causal=causal,
                         common_prefix_len=cpl)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8)])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("ps", [256, -1])
def test_fp8_prefill_chunks(hq, hkv, bs, causal, ps):
    """Chunked prefill rows and decode rows over an fp8 cache, with the
    quantising write of the new tokens first.  With split rows (ps 256) both
    kinds run in one persistent launch; unsplit (ps -1), in two launches."""
    w = _fp8_mixed(hq, hkv, bs, causal, 90 + hq + bs)
    _announce(f"fp8 prefill hq={hq} hkv={hkv} bs={bs} causal={causal} ps={ps}")
    dw = G.DevWorkload(w)
    G.run(dw, partition_size=ps)
    ref, ref_lse = G.reference(w)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", f"fp8 prefill {hq}/{hkv} bs={bs}")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, f"fp8 prefill {hq}/{hkv} bs={bs}")


def test_fp8_prefill_needle_bit_exact():
    """q = 64 e0 and key 0 = 64 e0 (code 0x68, scale 1), every other key
    orthogonal to e0: every prefill row sees key 0, whose probability is 1
    while every other one underflows to 0, so each output row is that key's
    value row times a power-of-two scale, exactly."""
    w = W.make_varlen("fp8_pf_needle", [100, 260], [70, 130], 32, 8, 128, 16, "fp8", seed=33)
    kc, vc = G.oracle_inputs(w)
    import dataclasses
    w = dataclasses.replace(w, k_cache=kc, v_cache=vc, slot_mapping=None, key_new=None,
                            value_new=None)
    w.k_scale = np.ones(8, dtype=np.float32)
    w.v_scale = np.full(8, 2.0 ** -5, dtype=np.float32)
    valid = w.valid_slot_mask()
    w.k_cache[valid, :, 0] = 0
    w.q[:] = 0
    w.q[:, :, 0] = W.f32_to_bf16_bits(np.float32(64.0))
    # key 0's V rows hold every finite code except -0 (each 4 times over 8
    # kv heads)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0x80, 0xFF]] = 0
    for s in range(2):
        w.k_cache[w.block_tables[s, 0], 0, :, 0] = 0x68
        w.v_cache[w.block_tables[s, 0], 0] = np.resize(np.roll(codes, 11 * s), (8, 128))
    _announce("fp8 prefill needle")
    dw = G.DevWorkload(w)
    G.run(dw, write=False)
    out = G.dev_to_bits(dw.out)
    for s in range(2):
        blk = w.block_tables[s, 0]
        for r in range(w.cu_seqlens_q[s], w.cu_seqlens_q[s + 1]):
            for h in range(32):
                v = oracle.e4m3_decode(w.v_cache[blk, 0, h // 4]) * 2.0 ** -5
                assert np.array_equal(out[r, h], W.f32_to_bf16_bits(v.astype(np.float32))), (s, r, h)


def test_fp8_prefill_equals_bf16_path_with_power_of_two_scales():
    """Prefill chunks over the same values held as e4m3 codes with
    power-of-two scales or as bfloat16: bit-identical outputs."""
    import dataclasses
    torch = G.torch()
    w8 = _fp8_mixed(32, 8, 16, True, 95)
    kc, vc = G.oracle_inputs(w8)
    w8 = dataclasses.replace(w8, k_cache=kc, v_cache=vc, slot_mapping=None, key_new=None,
                             value_new=None)
    w8.k_scale = np.full(8, 2.0 ** -6, dtype=np.float32)
    w8.v_scale = np.full(8, 2.0 ** -4, dtype=np.float32)
    kb = W.f32_to_bf16_bits((oracle.e4m3_decode(w8.k_cache) * 2.0 ** -6).astype(np.float32))
    vb = W.f32_to_bf16_bits((oracle.e4m3_decode(w8.v_cache) * 2.0 ** -4).astype(np.float32))
    kb[w8.k_cache == 0x7F] = W.BF16_QNAN
    vb[w8.v_cache == 0x7F] = W.BF16_QNAN
    wb = dataclasses.replace(w8, dtype="bf16", k_cache=kb, v_cache=vb, k_scale=None, v_scale=None)
    _announce("fp8 prefill vs bf16 identity")
    d8, db = G.DevWorkload(w8), G.DevWorkload(wb)
    G.run(d8, partition_size=256, write=False)
    G.run(db, partition_size=256, write=False)
    torch.cuda.synchronize()
    # the decode rows take the grouped decode kernel in both cases; the
    # prefill rows the matrix-core prefill kernel (fp8 and bf16 forms)
    assert np.array_equal(G.dev_to_bits(d8.out), G.dev_to_bits(db.out))


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8)])
def test_fp8_cascade(hq, hkv):
    """Cascade attention over an fp8 cache (prefix pass on the fp8 form of
    the prefill body, suffix pass on the fp8 kernels) against the oracle."""
    w = _fp8_mixed(hq, hkv, 16, True, 97, cpl=256)
    _announce(f"fp8 cascade hq={hq} hkv={hkv}")
    dw = G.DevWorkload(w)
    G.run_cascade(dw)
    ref, ref_lse = G.reference(w)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", f"fp8 cascade {hq}/{hkv}")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, f"fp8 cascade {hq}/{hkv}")


def test_fp8_cascade_decode_rows_one_launch():
    """Decode rows only: the prefix pass and the suffix's decode rows share
    one persistent launch over the fp8 cache."""
    rng = np.random.default_rng(98)
    n = 24
    ctx = 512 + rng.integers(0, 300, size=n)
    w = W.make_varlen("fp8_casc_dec", ctx, np.ones(n, dtype=np.int64), 32, 8, 128, 16, "fp8", 98,
                      causal=True, common_prefix_len=512)
    _announce("fp8 cascade decode rows")
    dw = G.DevWorkload(w)
    G.run_cascade(dw, partition_size=128)
    ref, ref_lse = G.reference(w)
    G.assert_close(G.dev_to_f64(dw.out), ref, "bf16", "fp8 cascade decode rows")
    G.lse_close(G.dev_to_f64(dw.lse), ref_lse, "fp8 cascade decode rows")
