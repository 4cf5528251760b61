"""Pins of the oracle's fp8 (e4m3) KV-cache arithmetic.

The e4m3 decode and the round-to-nearest-even encode are checked against
PyTorch's float8_e4m3fn conversion (a library routine of the same format);
the quantising write against hand-worked codes and its error bound; attention
on fp8 caches against the already pinned bfloat16 path on the same values.
"""
import numpy as np
import pytest

import oracle
from oracle import fp8 as F

torch = pytest.importorskip("torch")


def _torch_codes(x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    a = F.e4m3_decode(codes)
    b = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok])
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))
    assert F.e4m3_decode(np.uint8(0x7E)) == 448.0 and np.isnan(F.e4m3_decode(np.uint8(0xFF)))
    assert F.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9          # smallest subnormal
    assert F.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6          # smallest normal


def test_encode_matches_torch_on_all_bf16_patterns_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    x = bits.view(np.float32)
    keep = np.isfinite(x) & (np.abs(x) <= F.E4M3_MAX)
    x = x[keep]
    assert np.array_equal(F.e4m3_encode(x), _torch_codes(x))


def test_encode_ties_and_neighbours_match_torch():
    v = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))          # 0 .. 448, increasing
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)              # exact in float32
    assert np.array_equal(mid.astype(np.float64), (v[:-1] + v[1:]) / 2)
    near = np.concatenate([mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))])
    near = near[near <= F.E4M3_MAX]
    xs = np.concatenate([near, -near]).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(xs), _torch_codes(xs))
    # ties go to the even code: 2^-10 lies halfway between 0 and 2^-9
    assert F.e4m3_encode(np.float32(2.0 ** -10)) == 0x00
    assert F.e4m3_encode(np.float32(3 * 2.0 ** -10)) == 0x02    # halfway between codes 1 and 2
    rng = np.random.default_rng(0)
    r = (rng.standard_normal(200_000) * rng.choice([1e-3, 1, 30, 200], 200_000)).astype(np.float32)
    r = np.clip(r, -F.E4M3_MAX, F.E4M3_MAX)
    assert np.array_equal(F.e4m3_encode(r), _torch_codes(r))


def test_quantize_worked_codes():
    assert F.quantize(np.float32(1.0), np.float32(0.5)) == 0x40           # 2.0 = 2^(8-7)
    assert F.quantize(np.float32(-3.25), np.float32(1.0)) == 0xC5         # -(1 + 5/8) * 2
    assert F.quantize(np.float32(1000.0), np.float32(1.0)) == 0x7E        # saturates to 448
    assert F.quantize(np.float32(-1e9), np.float32(2.0)) == 0xFE          # -448
    assert F.quantize(np.float32(-1e-5), np.float32(1.0)) == 0x80         # rounds to -0
    assert F.quantize(np.float32(np.nan), np.float32(1.0)) == 0x7F
    # the division is float32: 0.1f / 0.3f is 0.33333334f, between codes
    # 0x2A (0.3125) and 0x2B (0.34375), nearer the latter
    assert F.quantize(np.float32(0.1), np.float32(0.3)) == 0x2B


def test_write_fp8_round_trip_error_bound():
    rng = np.random.default_rng(1)
    nb, bs, Hkv, D, T = 6, 8, 3, 16, 30
    kc = np.full((nb, bs, Hkv, D), 0x7F, dtype=np.uint8)                  # NaN poison
    vc = kc.copy()
    key = rng.standard_normal((T + 2, Hkv, D)).astype(np.float32)
    val = rng.standard_normal((T + 2, Hkv, D)).astype(np.float32)
    kb = (key.view(np.uint32) >> np.uint32(16)).astype(np.uint16)       # truncated to bf16
    vb = (val.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[3] = -1
    ks = np.array([0.01, 0.02, 0.005], dtype=np.float32)      # 0.005: some elements saturate
    vs = np.array([0.03, 0.01, 0.02], dtype=np.float32)
    oracle.kv_cache_write_fp8(kc, vc, kb, vb, slots, bs, ks, vs)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), bs)
        for h in range(Hkv):
            x = F.bf16_bits_to_f32(kb[t, h]).astype(np.float64)
            y = F.e4m3_decode(kc[b, o, h]) * float(ks[h])
            sat = np.abs(x) > F.E4M3_MAX * float(ks[h])
            # beyond the range: exactly +-448 * scale
            assert np.array_equal(y[sat], np.sign(x[sat]) * F.E4M3_MAX * float(ks[h]))
            # inside: a relative half-ulp of a 3-bit mantissa, or half the subnormal step
            bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * float(ks[h])) * (1 + 1e-6)
            assert (np.abs(y - x)[~sat] <= bound[~sat]).all()
    written = {int(s) for s in slots if s >= 0}
    for s in range(nb * bs):
        if s not in written:
            b, o = divmod(s, bs)
            assert (kc[b, o] == 0x7F).all() and (vc[b, o] == 0x7F).all()


def _small_fp8_case(rng, pow2_scales):
    nb, bs, Hkv, Hq, D = 12, 8, 2, 4, 16
    kc = rng.integers(0, 0x7E, size=(nb, bs, Hkv, D), dtype=np.uint8)
    vc = rng.integers(0, 0x7E, size=(nb, bs, Hkv, D), dtype=np.uint8)
    kc |= (rng.integers(0, 2, size=kc.shape, dtype=np.uint8) << 7)
    vc |= (rng.integers(0, 2, size=vc.shape, dtype=np.uint8) << 7)
    bt = np.array([[3, 7, 1, 0], [5, 2, 9, 11]], dtype=np.int32)
    L = np.array([27, 30], dtype=np.int32)
    q = (rng.standard_normal((2, Hq, D)).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if pow2_scales:
        ks = np.array([2.0 ** -6, 2.0 ** -5], dtype=np.float32)
        vs = np.array([2.0 ** -4, 2.0 ** -7], dtype=np.float32)
    else:
        ks = np.array([0.013, 0.007], dtype=np.float32)
        vs = np.array([0.021, 0.003], dtype=np.float32)
    return kc, vc, bt, L, q, ks, vs


def _as_bf16_bits(x64):
    b = np.asarray(x64, dtype=np.float32).view(np.uint32) >> np.uint32(16)
    assert np.array_equal(F.bf16_bits_to_f32(b.astype(np.uint16)).astype(np.float64), x64)
    return b.astype(np.uint16)


def test_fp8_attention_equals_bf16_path_on_the_same_values():
    rng = np.random.default_rng(2)
    kc, vc, bt, L, q, ks, vs = _small_fp8_case(rng, pow2_scales=True)
    scale = 0.25
    out8, lse8 = oracle.paged_attention(q, kc, vc, bt, L, scale, 8, "fp8", k_scale=ks, v_scale=vs)
    # the same values stored as bfloat16 (every e4m3 value times a power of two is one)
    kv = F.e4m3_decode(kc) * ks[None, None, :, None].astype(np.float64)
    vv = F.e4m3_decode(vc) * vs[None, None, :, None].astype(np.float64)
    outb, lseb = oracle.paged_attention(q, _as_bf16_bits(kv), _as_bf16_bits(vv), bt, L, scale, 8, "bf16")
    assert np.array_equal(out8, outb) and np.array_equal(lse8, lseb)


def test_fp8_attention_scale_homogeneity():
    rng = np.random.default_rng(3)
    kc, vc, bt, L, q, ks, vs = _small_fp8_case(rng, pow2_scales=False)
    o1, l1 = oracle.paged_attention(q, kc, vc, bt, L, 0.5, 8, "fp8", k_scale=ks, v_scale=vs)
    # doubling v_scale doubles the output; doubling k_scale equals doubling the logit scale
    o2, l2 = oracle.paged_attention(q, kc, vc, bt, L, 0.5, 8, "fp8", k_scale=ks, v_scale=2 * vs)
    assert np.allclose(o2, 2 * o1, rtol=1e-13, atol=0) and np.array_equal(l1, l2)
    o3, l3 = oracle.paged_attention(q, kc, vc, bt, L, 0.5, 8, "fp8", k_scale=2 * ks, v_scale=vs)
    o4, l4 = oracle.paged_attention(q, kc, vc, bt, L, 1.0, 8, "fp8", k_scale=ks, v_scale=vs)
    assert np.allclose(o3, o4, rtol=1e-12, atol=1e-14) and np.allclose(l3, l4, rtol=1e-12)
