"""Thin ctypes binding of libpagedkv.so (declared in include/pagedkv.h).

Only argument marshalling happens here: torch tensors supply device pointers,
shapes and the current HIP stream; every step of the computation runs in the
library's kernels.  There is no fallback: if the library is missing, or a
tensor is not on the GPU, a call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK = 0
PKV_F32 = 0
PKV_BF16 = 1
PKV_FP8_E4M3 = 2
PKV_F16 = 3
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_SHAPE", 3: "PKV_ERR_UNSUPPORTED",
                4: "PKV_ERR_ALIGN", 5: "PKV_ERR_WORKSPACE", 6: "PKV_ERR_METADATA", 7: "PKV_ERR_HIP"}


class PkvKvCache(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("block_stride", ctypes.c_int64),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


# PKV_RAN_* bits of pkv_call_options.launched: the kernels a call enqueued
RAN_PLANNER = 0x001
RAN_DECODE_VALU = 0x002
RAN_DECODE_MFMA = 0x004
RAN_DECODE_PAIRS = 0x008
RAN_PREFILL_MFMA = 0x010
RAN_PREFILL_VALU = 0x020
RAN_MIXED = 0x040
RAN_PREFIX = 0x080
RAN_CASCADE_ONE = 0x100
RAN_SPLIT_MERGE = 0x200
RAN_CASCADE_MERGE = 0x400
RAN_NAMES = {RAN_PLANNER: "planner", RAN_DECODE_VALU: "decode_valu",
             RAN_DECODE_MFMA: "decode_mfma", RAN_DECODE_PAIRS: "decode_fp8_head_pairs",
             RAN_PREFILL_MFMA: "prefill_mfma", RAN_PREFILL_VALU: "prefill_valu",
             RAN_MIXED: "mixed_one_launch", RAN_PREFIX: "cascade_prefix_pass",
             RAN_CASCADE_ONE: "cascade_one_launch", RAN_SPLIT_MERGE: "split_merge",
             RAN_CASCADE_MERGE: "cascade_merge"}
NOALLOC_SCRATCH_BYTES = 128 << 20


class CallOptions(ctypes.Structure):
    """pkv_call_options: per-call launch choices (0 = the library's) and, after
    the call, `launched`, the RAN_* bits of the kernels it enqueued."""
    _fields_ = [
        ("decode_kernel", ctypes.c_int32),    # 1 VALU, 2 matrix cores
        ("prefill_kernel", ctypes.c_int32),   # 1 VALU rows
        ("fp8_head_pairs", ctypes.c_int32),   # 1 one kv head per wave
        ("mixed_launch", ctypes.c_int32),     # 1 separate launches
        ("cascade_launch", ctypes.c_int32),   # 1 separate launches
        ("launched", ctypes.c_uint32),
    ]

    def ran(self):
        """Names of the kernels the last call with these options enqueued."""
        return [n for b, n in sorted(RAN_NAMES.items()) if self.launched & b]


def _opts(options):
    """A CallOptions from None, a CallOptions, or a dict of its fields."""
    if options is None or isinstance(options, CallOptions):
        return options
    return CallOptions(**options)


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None

_vp, _i32, _i64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_size_t)
_SIGS = {
    "pkv_kv_cache_write": (_i32, [ctypes.POINTER(PkvKvCache), _vp, _vp, _vp, _i64, _vp]),
    "pkv_choose_partition_size": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_attention_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attention_decode": (_i32, [_vp, _vp, ctypes.POINTER(PkvKvCache), _vp, _i32, _vp,
                                          _i32, _i32, _i32, _f32, _i32, _i32, _vp, _vp, _sz,
                                          ctypes.POINTER(CallOptions), _vp]),
    "pkv_paged_attention_decode_noalloc": (_i32, [_vp, _vp, ctypes.POINTER(PkvKvCache), _vp, _i32,
                                                  _vp, _i32, _i32, _i32, _f32, _i32, _i32, _vp,
                                                  ctypes.POINTER(CallOptions), _vp]),
    "pkv_paged_attention_varlen": (_i32, [_vp, _vp, ctypes.POINTER(PkvKvCache), _vp, _vp, _vp,
                                          _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i32,
                                          _vp, _vp, _sz, ctypes.POINTER(CallOptions), _vp]),
    "pkv_cascade_attention": (_i32, [_vp, _vp, ctypes.POINTER(PkvKvCache), _vp, _vp, _vp, _i32,
                                     _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32,
                                     _vp, _vp, _sz, ctypes.POINTER(CallOptions), _vp]),
    "pkv_cascade_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_cascade_reason": (ctypes.c_char_p, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_validate_cascade": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, ctypes.c_char_p,
                                    _sz]),
    "pkv_unsupported_reason": (ctypes.c_char_p, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_status_string": (ctypes.c_char_p, [_i32]),
    "pkv_validate_metadata": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _vp, _i64, _i64,
                                     _i32, ctypes.c_char_p, _sz]),
    "pkv_timing_enable": (_i32, [_i32]),
    "pkv_timing_read": (_i32, [ctypes.POINTER(ctypes.c_float), _i32]),
    "pkv_xcd_probe": (_i32, [_vp, _i32, _vp]),
    "pkv_pool_create": (_vp, [_i64, _i32, _i32]),
    "pkv_pool_destroy": (None, [_vp]),
    "pkv_pool_num_free": (_i64, [_vp]),
    "pkv_pool_allocate": (_i64, [_vp, _i64, _i64, _vp]),
    "pkv_pool_cache_full_blocks": (_i32, [_vp, _i64, _vp, _i64]),
    "pkv_pool_free": (_i32, [_vp, _i64]),
    "pkv_pool_num_blocks_of": (_i64, [_vp, _i64]),
    "pkv_pool_block_table": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "pkv_pool_slot_mapping": (_i32, [_vp, _i64, _i64, _i64, _vp]),
    "pkv_pool_free_queue": (_i64, [_vp, _vp, _i64]),
}


def lib() -> ctypes.CDLL:
    """Load libpagedkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m paged_kv_cache_50_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def unsupported_reason(dtype: int, head_size: int, block_size: int, num_heads: int,
                       num_kv_heads: int) -> Optional[str]:
    r = lib().pkv_unsupported_reason(dtype, head_size, block_size, num_heads, num_kv_heads)
    return None if r is None else r.decode()


def choose_partition_size(num_seqs, num_heads, num_kv_heads, max_seq_len, partition_size=0) -> int:
    return int(lib().pkv_choose_partition_size(num_seqs, num_heads, num_kv_heads, max_seq_len,
                                               partition_size))


def workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len,
                    partition_size=0) -> int:
    n = lib().pkv_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size,
                                            max_seq_len, partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise PagedKVError(2, "workspace_bytes")
    return int(n)


# --------------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float16:
        return PKV_F16
    if t.dtype == torch.float8_e4m3fn:
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _io_dtype(k_cache):
    """dtype of q/out/key/value for a cache: bfloat16 for fp8 caches."""
    torch = _torch()
    return torch.bfloat16 if k_cache.dtype == torch.float8_e4m3fn else k_cache.dtype


def _require_gpu(*ts):
    """Every given tensor on the GPU, and all on the same one."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (no CPU fallback)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different GPUs ({dev} and {t.device})")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def cache_descriptor(k_cache, v_cache, k_scale=None, v_scale=None) -> PkvKvCache:
    """Describe [num_blocks, block_size, num_kv_heads, head_size] caches whose
    blocks may be strided (dense inside a block).  fp8 (float8_e4m3fn) caches
    need float32 [num_kv_heads] scales k_scale / v_scale."""
    torch = _torch()
    _require_gpu(k_cache, v_cache, k_scale, v_scale)
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have the same 4-D shape and dtype")
    nb, bs, hkv, d = k_cache.shape
    for t in (k_cache, v_cache):
        if t.stride(3) != 1 or t.stride(2) != d or t.stride(1) != hkv * d:
            raise ValueError("cache blocks must be dense [block_size, num_kv_heads, head_size]")
    if k_cache.stride(0) != v_cache.stride(0):
        raise ValueError("k_cache and v_cache must share the block stride")
    code = _dtype_code(k_cache)
    if code == PKV_FP8_E4M3:
        for t in (k_scale, v_scale):
            if t is None or t.dtype != torch.float32 or tuple(t.shape) != (hkv,) or not t.is_contiguous():
                raise ValueError("fp8 caches need contiguous float32 k_scale/v_scale [num_kv_heads]")
    return PkvKvCache(k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, hkv, d, code,
                      k_cache.stride(0) if nb > 1 else 0,
                      _ptr(k_scale) if code == PKV_FP8_E4M3 else None,
                      _ptr(v_scale) if code == PKV_FP8_E4M3 else None)


def _check(status: int, what: str):
    if status != PKV_OK:
        raise PagedKVError(status, what)


def kv_cache_write(k_cache, v_cache, key, value, slot_mapping, k_scale=None, v_scale=None) -> None:
    """Scatter key/value rows [>= T, Hkv, D] into the caches at slot_mapping
    (int64 [T], -1 = skip).  In place, asynchronous on the current stream.
    fp8 caches take bfloat16 rows and quantise them with k_scale / v_scale."""
    torch = _torch()
    _require_gpu(key, value, slot_mapping, k_cache)
    desc = cache_descriptor(k_cache, v_cache, k_scale, v_scale)
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be a contiguous int64 tensor")
    for t in (key, value):
        if not t.is_contiguous() or t.dtype != _io_dtype(k_cache) or tuple(t.shape[1:]) != tuple(k_cache.shape[2:]):
            raise ValueError("key/value must be contiguous [T, num_kv_heads, head_size] in the cache's "
                             "input dtype")
    T = slot_mapping.shape[0]
    if key.shape[0] < T or value.shape[0] < T:
        raise ValueError("key/value hold fewer rows than slot_mapping")
    _check(lib().pkv_kv_cache_write(ctypes.byref(desc), key.data_ptr(), value.data_ptr(),
                                    slot_mapping.data_ptr(), T, _stream(key)), "kv_cache_write")


def _workspace(ws, need: int, device):
    """The workspace and its size in bytes (allocated here when not given).
    A given one must be contiguous on the device of q: the library takes
    numel * element_size bytes from its first element on."""
    torch = _torch()
    if ws is not None and (not ws.is_contiguous() or ws.device != device):
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    if need == 0:
        return ws, 0 if ws is None else ws.numel() * ws.element_size()
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def _meta(t, name):
    torch = _torch()
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")


def _check_lse(lse_out, rows, heads, what):
    """lse_out is optional; the kernels write float32 [rows, heads] through it."""
    torch = _torch()
    if lse_out is None:
        return
    if (lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (rows, heads)
            or not lse_out.is_contiguous()):
        raise ValueError(f"lse_out must be a contiguous float32 [{what}, num_heads]")


def _byref(options):
    return None if options is None else ctypes.byref(options)


def _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, lse_out, k_scale, v_scale):
    _require_gpu(out, q, block_tables, seq_lens, lse_out, k_cache)
    desc = cache_descriptor(k_cache, v_cache, k_scale, v_scale)
    _meta(block_tables, "block_tables")
    _meta(seq_lens, "seq_lens")
    if not (q.is_contiguous() and out.is_contiguous()) or q.dtype != _io_dtype(k_cache) or out.dtype != q.dtype:
        raise ValueError("q/out must be contiguous and in the cache's input dtype")
    S, Hq, D = q.shape
    if out.shape != q.shape or D != k_cache.shape[3] or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("shape mismatch")
    _check_lse(lse_out, S, Hq, "num_seqs")
    return desc, S, Hq, D


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                           max_seq_len: int, partition_size: int = 0, workspace=None,
                           lse_out=None, k_scale=None, v_scale=None, window_left: int = -1,
                           options=None):
    """Decode attention, one query row per sequence.  out/q: [S, Hq, D].
    max_seq_len is a host-side upper bound of seq_lens (no device sync).
    window_left >= 0: sliding window (keys seq_len - 1 - window_left ..).
    options: a CallOptions (or dict of its fields); its `launched` holds the
    kernels the call enqueued."""
    _require_gpu(workspace)
    desc, S, Hq, D = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, lse_out,
                                  k_scale, v_scale)
    options = _opts(options)
    need = workspace_bytes(S, Hq, desc.num_kv_heads, D, max_seq_len, partition_size)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    _check(lib().pkv_paged_attention_decode(
        out.data_ptr(), q.data_ptr(), ctypes.byref(desc), block_tables.data_ptr(),
        block_tables.shape[1], seq_lens.data_ptr(), S, Hq, int(max_seq_len), float(scale),
        int(window_left), int(partition_size), _ptr(lse_out), _ptr(workspace), ws_bytes,
        _byref(options), _stream(q)),
        "paged_attention_decode")
    return out


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens,
                                   scale: float, max_seq_len: int, partition_size: int = 0,
                                   lse_out=None, k_scale=None, v_scale=None,
                                   window_left: int = -1, options=None):
    """paged_attention_decode without a workspace: the split partials live in
    the library's per-GPU scratch array (NOALLOC_SCRATCH_BYTES), so neither
    the library nor this wrapper allocates device memory.  Calls on one GPU
    that may overlap in time race; order them on one stream."""
    desc, S, Hq, D = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, lse_out,
                                  k_scale, v_scale)
    options = _opts(options)
    _check(lib().pkv_paged_attention_decode_noalloc(
        out.data_ptr(), q.data_ptr(), ctypes.byref(desc), block_tables.data_ptr(),
        block_tables.shape[1], seq_lens.data_ptr(), S, Hq, int(max_seq_len), float(scale),
        int(window_left), int(partition_size), _ptr(lse_out), _byref(options), _stream(q)),
        "paged_attention_decode_noalloc")
    return out


def paged_attention_varlen(out, q, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables,
                           scale: float, max_query_len: int, max_seq_len: int, causal: bool = True,
                           partition_size: int = 0, workspace=None, lse_out=None,
                           k_scale=None, v_scale=None, window_left: int = -1, options=None):
    """Variable-length attention over a flattened batch (q/out [T, Hq, D]).
    window_left >= 0: sliding window (symmetric when not causal).  options
    as for paged_attention_decode."""
    _require_gpu(out, q, cu_seqlens_q, seq_lens, block_tables, workspace, lse_out, k_cache)
    desc = cache_descriptor(k_cache, v_cache, k_scale, v_scale)
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        _meta(t, n)
    if not (q.is_contiguous() and out.is_contiguous()) or q.dtype != _io_dtype(k_cache) or out.dtype != q.dtype:
        raise ValueError("q/out must be contiguous and in the cache's input dtype")
    T, Hq, D = q.shape
    S = seq_lens.shape[0]
    if out.shape != q.shape or cu_seqlens_q.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("shape mismatch")
    _check_lse(lse_out, T, Hq, "num_tokens")
    options = _opts(options)
    need = workspace_bytes(S, Hq, desc.num_kv_heads, D, max_seq_len, partition_size)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    _check(lib().pkv_paged_attention_varlen(
        out.data_ptr(), q.data_ptr(), ctypes.byref(desc), cu_seqlens_q.data_ptr(),
        seq_lens.data_ptr(), block_tables.data_ptr(), block_tables.shape[1], S, T, Hq,
        int(max_query_len), int(max_seq_len), float(scale), 1 if causal else 0, int(window_left),
        int(partition_size), _ptr(lse_out), _ptr(workspace), ws_bytes, _byref(options),
        _stream(q)),
        "paged_attention_varlen")
    return out


def cascade_workspace_bytes(num_seqs, num_tokens, num_heads, num_kv_heads, head_size,
                            max_seq_len, common_prefix_len, partition_size=0) -> int:
    n = lib().pkv_cascade_workspace_bytes(num_seqs, num_tokens, num_heads, num_kv_heads,
                                          head_size, max_seq_len, common_prefix_len,
                                          partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise PagedKVError(2, "cascade_workspace_bytes")
    return int(n)


def cascade_reason(common_prefix_len, num_seqs, num_tokens, num_heads, num_kv_heads, head_size,
                   dtype=PKV_BF16, window_left=-1) -> Optional[str]:
    """None when cascade attention is advised for the batch, else why not."""
    r = lib().pkv_cascade_reason(common_prefix_len, num_seqs, num_tokens, num_heads, num_kv_heads,
                                 head_size, dtype, window_left)
    return None if r is None else r.decode()


def cascade_attention(out, q, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables,
                      prefix_blocks, common_prefix_len: int, scale: float, max_query_len: int,
                      max_seq_len: int, causal: bool = True, partition_size: int = 0,
                      workspace=None, lse_out=None, k_scale=None, v_scale=None, options=None):
    """Cascade (shared-prefix) attention over a flattened batch (q/out
    [T, Hq, D]): the result of paged_attention_varlen on the same arguments,
    with the prefix blocks (int32 [common_prefix_len / block_size], shared
    by every sequence's table) read once for the whole batch.  fp8 caches
    take k_scale / v_scale as in paged_attention_varlen."""
    _require_gpu(out, q, cu_seqlens_q, seq_lens, block_tables, prefix_blocks, workspace, lse_out,
                 k_cache)
    desc = cache_descriptor(k_cache, v_cache, k_scale, v_scale)
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (seq_lens, "seq_lens"),
                 (block_tables, "block_tables"), (prefix_blocks, "prefix_blocks")):
        _meta(t, n)
    if not (q.is_contiguous() and out.is_contiguous()) or q.dtype != _io_dtype(k_cache) or out.dtype != q.dtype:
        raise ValueError("q/out must be contiguous and in the cache's input dtype")
    T, Hq, D = q.shape
    S = seq_lens.shape[0]
    if out.shape != q.shape or cu_seqlens_q.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("shape mismatch")
    if prefix_blocks.shape[0] * k_cache.shape[1] < common_prefix_len:
        raise ValueError("prefix_blocks shorter than the prefix")
    _check_lse(lse_out, T, Hq, "num_tokens")
    options = _opts(options)
    need = cascade_workspace_bytes(S, T, Hq, desc.num_kv_heads, D, max_seq_len, common_prefix_len,
                                   partition_size)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    _check(lib().pkv_cascade_attention(
        out.data_ptr(), q.data_ptr(), ctypes.byref(desc), cu_seqlens_q.data_ptr(),
        seq_lens.data_ptr(), block_tables.data_ptr(), block_tables.shape[1],
        prefix_blocks.data_ptr(), S, T, Hq, int(max_query_len), int(max_seq_len),
        int(common_prefix_len), float(scale), 1 if causal else 0, int(partition_size),
        _ptr(lse_out), _ptr(workspace), ws_bytes, _byref(options), _stream(q)),
        "cascade_attention")
    return out


def validate_cascade(block_tables, seq_lens, cu_seqlens_q, prefix_blocks, common_prefix_len,
                     block_size):
    """Check host copies of a cascade batch's metadata.  Returns "" when
    valid, else the first problem found."""
    import numpy as np

    def arr(x):
        if hasattr(x, "detach"):
            x = x.detach().cpu().numpy()
        return np.ascontiguousarray(x, dtype=np.int32)

    bt, sl, cu, pb = arr(block_tables), arr(seq_lens), arr(cu_seqlens_q), arr(prefix_blocks)
    S = sl.shape[0]
    # the library reads these arrays to the extents the sizes imply: refuse
    # short ones here rather than let it read past them
    if bt.ndim != 2 or bt.shape[0] < S:
        raise ValueError(f"block_tables must be 2-D with at least {S} rows")
    if cu.ndim != 1 or cu.shape[0] < S + 1:
        raise ValueError(f"cu_seqlens_q must hold at least num_seqs + 1 = {S + 1} entries")
    bs, cpl = int(block_size), int(common_prefix_len)
    need = cpl // bs if bs > 0 and cpl >= 0 and cpl % bs == 0 else 0
    if pb.size < need:
        raise ValueError(f"prefix_blocks holds {pb.size} entries, the prefix needs {need}")
    msg = ctypes.create_string_buffer(256)
    st = lib().pkv_validate_cascade(bt.ctypes.data, bt.shape[1], sl.ctypes.data, sl.shape[0],
                                    cu.ctypes.data, pb.ctypes.data if pb.size else None,
                                    int(common_prefix_len), int(block_size), msg, 256)
    return "" if st == PKV_OK else (msg.value.decode() or "invalid metadata")


def validate_metadata(block_tables, seq_lens, max_seq_len, num_blocks, block_size,
                      cu_seqlens_q=None, num_tokens=0, max_query_len=0, slot_mapping=None):
    """Check host copies of the metadata (numpy arrays or CPU tensors).
    Returns "" when valid, else the first problem found."""
    import numpy as np

    def arr(x, dt):
        if x is None:
            return None
        if hasattr(x, "detach"):
            x = x.detach().cpu().numpy()
        return np.ascontiguousarray(x, dtype=dt)

    bt = arr(block_tables, np.int32)
    sl = arr(seq_lens, np.int32)
    cu = arr(cu_seqlens_q, np.int32)
    sm = arr(slot_mapping, np.int64)
    S = sl.shape[0]
    if bt.ndim != 2 or bt.shape[0] < S:
        raise ValueError(f"block_tables must be 2-D with at least {S} rows")
    if cu is not None and (cu.ndim != 1 or cu.shape[0] < S + 1):
        raise ValueError(f"cu_seqlens_q must hold at least num_seqs + 1 = {S + 1} entries")
    msg = ctypes.create_string_buffer(256)
    st = lib().pkv_validate_metadata(
        bt.ctypes.data, bt.shape[1], sl.ctypes.data, sl.shape[0],
        None if cu is None else cu.ctypes.data, int(num_tokens), int(max_query_len),
        int(max_seq_len), None if sm is None else sm.ctypes.data,
        0 if sm is None else sm.shape[0], int(num_blocks), int(block_size), msg, 256)
    return "" if st == PKV_OK else (msg.value.decode() or "invalid metadata")


def timing_enable(enable: bool = True, every_n: int = 1) -> None:
    """Record the main attention kernel's duration for one call in every_n
    (enable=False turns timing off)."""
    _check(lib().pkv_timing_enable(int(every_n) if enable else 0), "timing_enable")


def timing_read(cap: int = 4096):
    """Durations (ms) of the main attention kernel of each call since the
    last read; waits for them to finish."""
    buf = (ctypes.c_float * cap)()
    n = lib().pkv_timing_read(buf, cap)
    if n < 0:
        raise PagedKVError(7, "timing_read")
    return [buf[i] for i in range(n)]


def xcd_probe(n: int = 8):
    """The XCD (0-7) that each of n one-wave workgroups of one launch on the
    current stream ran on: where the dispatcher starts a launch."""
    torch = _torch()
    out = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    _check(lib().pkv_xcd_probe(_ptr(out), int(n), _stream(out)), "xcd_probe")
    return out.tolist()


def default_scale(head_size: int) -> float:
    return 1.0 / math.sqrt(head_size)


# ------------------------------------------------------------------ block pool

class BlockPool:
    """Host KV block pool of the library (pkv_pool_*): allocation of cache
    blocks to requests, prefix caching, block tables and slot mappings."""

    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True):
        self._p = lib().pkv_pool_create(int(num_blocks), int(block_size), 1 if prefix_caching else 0)
        if not self._p:
            raise PagedKVError(2, "pool_create")
        self.block_size = int(block_size)

    def close(self):
        if self._p:
            lib().pkv_pool_destroy(self._p)
            self._p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ids(token_ids):
        import numpy as np
        if token_ids is None:
            return None, None
        a = np.ascontiguousarray(token_ids, dtype=np.int32)
        return a, a.ctypes.data

    def num_free(self) -> int:
        return int(lib().pkv_pool_num_free(self._p))

    def allocate(self, req: int, num_tokens: int, token_ids=None) -> int:
        """Cached leading tokens (>= 0) or -1 when the pool is short of blocks."""
        keep, ptr = self._ids(token_ids)
        if keep is not None and len(keep) < num_tokens:
            raise ValueError("token_ids shorter than num_tokens")
        r = int(lib().pkv_pool_allocate(self._p, int(req), int(num_tokens), ptr))
        if r == -2:
            raise PagedKVError(2, "pool_allocate")
        return r

    def cache_full_blocks(self, req: int, token_ids, num_tokens: int) -> None:
        keep, ptr = self._ids(token_ids)
        if len(keep) < num_tokens:
            raise ValueError("token_ids shorter than num_tokens")
        _check(lib().pkv_pool_cache_full_blocks(self._p, int(req), ptr, int(num_tokens)),
               "pool_cache_full_blocks")

    def free(self, req: int) -> None:
        _check(lib().pkv_pool_free(self._p, int(req)), "pool_free")

    def num_blocks_of(self, req: int) -> int:
        return int(lib().pkv_pool_num_blocks_of(self._p, int(req)))

    def block_table(self, reqs, max_blocks: int):
        import numpy as np
        r = np.ascontiguousarray(reqs, dtype=np.int64)
        out = np.empty((len(r), int(max_blocks)), dtype=np.int32)
        _check(lib().pkv_pool_block_table(self._p, r.ctypes.data, len(r), int(max_blocks),
                                          out.ctypes.data), "pool_block_table")
        return out

    def slot_mapping(self, req: int, first_pos: int, count: int):
        import numpy as np
        out = np.empty(int(count), dtype=np.int64)
        _check(lib().pkv_pool_slot_mapping(self._p, int(req), int(first_pos), int(count),
                                           out.ctypes.data if count else None), "pool_slot_mapping")
        return out

    def free_queue(self):
        import numpy as np
        n = int(lib().pkv_pool_free_queue(self._p, None, 0))
        out = np.empty(n, dtype=np.int32)
        lib().pkv_pool_free_queue(self._p, out.ctypes.data, n)
        return out
