"""FP8 (e4m3) KV-cache arithmetic for the oracle.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path; shares no code with
the HIP library.

The pages admit an fp8 family of KV-cache dtypes next to fp16/bf16 (vLLM
book, ch. 6 "Sélection du backend": the backend's supported cache dtypes),
with a dequantisation scale of shape (num_sequences, num_kv_heads) that is a
broadcast view of the layer's scales ("Flux des paramètres du chemin
non-cascadé"), and the cache written by the slot scatter ("Écriture du KV
cache : do_kv_cache_update").  Readings taken here:
  * format: e4m3 in its OCP "fn" variant - 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals when the exponent field is 0, no
    infinities, codes 0x7F / 0xFF are NaN, largest finite value 448;
  * one scale per kv head (float32), shared by the write and the attention:
    stored code c of head h stands for decode(c) * scale[h];
  * the write quantises x (bfloat16) as: t = float32(x) / float32(scale),
    correctly rounded in float32; t clamped to [-448, 448]; then rounded to
    the nearest e4m3 value, ties to the even code (the code's last bit is
    the mantissa's last bit).  NaN stays NaN.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = np.uint8(0x7F)


def e4m3_decode(codes) -> np.ndarray:
    """Exact float64 value of e4m3 codes (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# the 127 non-negative finite values in code order (increasing)
_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(t) -> np.ndarray:
    """Nearest e4m3 code of values already inside [-448, 448], ties to the
    even code; the sign bit follows the input's sign bit (so -0.0 and small
    negatives that round to zero give 0x80).  NaN gives 0x7F."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    if np.any(a[np.isfinite(a)] > E4M3_MAX):
        raise ValueError("e4m3_encode expects values clamped to [-448, 448]")
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, 126)   # first value >= a
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(np.signbit(t), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(t), E4M3_NAN, code).astype(np.uint8)


def quantize(x_f32, scale_f32) -> np.ndarray:
    """Codes of float32 values x for a float32 scale (the write's rule)."""
    x = np.asarray(x_f32, dtype=np.float32)
    t = (x / np.float32(scale_f32)).astype(np.float32)      # IEEE float32 division
    t = np.where(np.isnan(t), t, np.clip(t, -E4M3_MAX, E4M3_MAX))
    return e4m3_encode(t)


def bf16_bits_to_f32(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def kv_cache_write_fp8(k_cache: np.ndarray, v_cache: np.ndarray, key_bits: np.ndarray,
                       value_bits: np.ndarray, slot_mapping: np.ndarray, block_size: int,
                       k_scale: np.ndarray, v_scale: np.ndarray) -> None:
    """Slot scatter into fp8 caches (uint8 codes [nb, bs, Hkv, D]) of
    bfloat16 key/value rows (uint16 bits [>=T, Hkv, D]), quantising each
    element with its kv head's scale.  Slot < 0 writes nothing."""
    Hkv = k_cache.shape[2]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        for h in range(Hkv):
            k_cache[blk, off, h] = quantize(bf16_bits_to_f32(key_bits[t, h]), k_scale[h])
            v_cache[blk, off, h] = quantize(bf16_bits_to_f32(value_bits[t, h]), v_scale[h])
