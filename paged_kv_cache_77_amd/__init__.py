"""paged_kv_cache_77_amd -- paged attention for MI355X (gfx950).

Thin Python binding of the C ABI in ``include/pa.h`` (``libpa.so``, built by
``paged_kv_cache_77_amd.build``).  Each function has the C entry point's
name; it marshals torch tensors (device memory) to pointers and launches on
torch's current HIP stream.  All arithmetic runs in the HIP kernels: when
the library is missing these functions raise, there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PA_CACHE_BF16", "PA_CACHE_FP8_E4M3", "PaError", "PaKvLayout", "lib", "make_layout",
    "pa_status_string", "pa_kv_cache_bytes", "pa_compute_slot_mapping",
    "pa_reshape_and_cache", "pa_reshape_and_cache_varlen", "pa_decode",
    "pa_decode_workspace_size", "pa_decode_balanced",
    "pa_decode_partitioned", "pa_merge_partitions", "pa_prefill_varlen",
    "pa_debug_gather_kv", "pa_debug_fp8_to_f32", "pa_debug_fp8_to_f16", "pa_validate_metadata",
    "PaDecodePlan", "pa_decode_plan_for", "pa_decode_auto", "pa_decode_partitioned_range",
    "pa_decode_shared_prefix", "pa_decode_append", "pa_measure_read_stream", "EXPORTED_SYMBOLS",
    "pa_decode_auto_static", "PA_STATIC_SCRATCH_BYTES",
]

HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY may point at another build of the same sources (e.g. a tuning variant).
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_HIP = -3
PA_ERR_METADATA = -4
PA_ERR_SCRATCH = -5
# size of pa_decode_auto_static's device array (include/pa.h)
PA_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024
PA_CACHE_BF16 = 0
PA_CACHE_FP8_E4M3 = 1

EXPORTED_SYMBOLS = (
    "pa_status_string", "pa_kv_cache_bytes", "pa_compute_slot_mapping",
    "pa_reshape_and_cache", "pa_reshape_and_cache_varlen", "pa_decode",
    "pa_decode_workspace_size", "pa_decode_balanced",
    "pa_decode_partitioned", "pa_merge_partitions", "pa_prefill_varlen",
    "pa_debug_gather_kv", "pa_debug_fp8_to_f32", "pa_debug_fp8_to_f16", "pa_validate_metadata",
    "pa_decode_plan_for", "pa_decode_auto", "pa_decode_partitioned_range",
    "pa_decode_shared_prefix", "pa_decode_append", "pa_measure_read_stream",
    "pa_decode_auto_static",
    # host block manager (include/pa_blocks.h; binding in blocks.py)
    "pa_block_hashes", "pa_pool_create", "pa_pool_destroy", "pa_pool_num_free", "pa_pool_usage",
    "pa_pool_ref_count", "pa_pool_lookup", "pa_pool_get_new_blocks", "pa_pool_touch",
    "pa_pool_free_blocks", "pa_pool_cache_block", "pa_pool_allocate_prompt", "pa_pool_commit",
    "pa_pool_free_request", "pa_map_to_kernel_blocks",
)


class PaKvLayout(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32)]


class PaDecodePlan(ctypes.Structure):
    _fields_ = [("split", ctypes.c_int32), ("partition_size", ctypes.c_int32),
                ("max_num_partitions", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {pa_status_string(status)} ({status})")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float


def lib() -> ctypes.CDLL:
    """The loaded libpa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_77_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        lp = ctypes.POINTER(PaKvLayout)
        sig = {
            "pa_status_string": ([_I], ctypes.c_char_p),
            "pa_kv_cache_bytes": ([lp, ctypes.POINTER(ctypes.c_size_t)], _I),
            "pa_compute_slot_mapping": ([_P, _P, _I, _P, _P, _I, _I, _I, _P], _I),
            "pa_reshape_and_cache": ([lp, _P, _P, _P, _P, _I, _P, _P, _P, _P], _I),
            "pa_reshape_and_cache_varlen": ([lp, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _P,
                                             _P, _P, _P], _I),
            "pa_decode": ([lp, _P, _P, _I, _I, _P, _P, _P, _I, _P, _I, _F, _P, _P, _P, _P],
                          _I),
            "pa_decode_workspace_size": ([lp, _I, _I], ctypes.c_size_t),
            "pa_decode_balanced": ([lp, _P, _P, _I, _I, _P, _P, _P, _I, _P, _I, _F, _P, _P, _P,
                                    _P, ctypes.c_size_t, _P], _I),
            "pa_decode_partitioned": ([lp, _P, _I, _I, _P, _P, _P, _I, _P, _I, _F, _P, _P, _P,
                                       _I, _I, _P, _P, _P, _P], _I),
            "pa_merge_partitions": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
            "pa_decode_partitioned_range": ([lp, _P, _I, _I, _P, _P, _P, _I, _P, _I, _F, _P, _P,
                                             _P, _I, _I, _I, _I, _P, _P, _P, _P], _I),
            "pa_decode_append": ([lp, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _I, _F,
                                  _P, _P, _P, _P], _I),
            "pa_measure_read_stream": ([_P, ctypes.c_size_t, _P, _I, _P], _I),
            "pa_decode_shared_prefix": ([lp, _P, _P, _I, _I, _P, _P, _P, _I, _P, _I, _F, _P,
                                         _P, _P, _I, _I, _I, _P, _P, _P, _P], _I),
            "pa_prefill_varlen": ([lp, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                   _F, _P, _P, _P, _P], _I),
            "pa_debug_gather_kv": ([lp, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _P], _I),
            "pa_debug_fp8_to_f32": ([_P, _P, _I, _P], _I),
            "pa_debug_fp8_to_f16": ([_P, _P, _I, _P], _I),
            "pa_decode_plan_for": ([lp, _I, _I, _I, ctypes.POINTER(PaDecodePlan)], _I),
            "pa_decode_auto": ([lp, _P, _P, _I, _I, _P, _P, _P, _I, _P, _I, _F, _P, _P, _P,
                                ctypes.POINTER(PaDecodePlan), _P, ctypes.c_size_t, _P], _I),
            "pa_validate_metadata": ([_P, _I, _P, _P, _I, _P, _I, _I, _I], _I),
            "pa_decode_auto_static": ([lp, _P, _P, _I, _I, _P, _P, _P, _I, _P, _I, _F, _P, _P,
                                       _P, ctypes.POINTER(PaDecodePlan), _P], _I),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def make_layout(num_blocks: int, num_kv_heads: int, head_dim: int,
                cache_dtype: int = PA_CACHE_BF16, block_size: int = 16) -> PaKvLayout:
    return PaKvLayout(num_blocks, num_kv_heads, head_dim, block_size, cache_dtype)


def _check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PaError(status, where)


def _dev(t: Optional[torch.Tensor], name: str):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------------------
# Argument checks made before any launch.  The kernels trust dtypes and
# sizes (a pool smaller than its layout, or an int64 table read as int32,
# would be read or written out of bounds on the device), so the binding
# rejects mismatches with ValueError first.  Checks that need no device
# (dtype, rank, sizes) come before the device check, so they hold on a host
# without a GPU too.

def _need(t, name: str, dtype, dims=None, min_numel: int = 0, optional: bool = False):
    """t must have `dtype`; `dims` (a tuple, None entries free) fixes its
    rank and sizes; at least `min_numel` elements."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if dims is not None:
        if t.dim() != len(dims):
            raise ValueError(f"{name}: {t.dim()} dimensions, expected {len(dims)}")
        for i, want in enumerate(dims):
            if want is not None and t.shape[i] != want:
                raise ValueError(f"{name}: shape {tuple(t.shape)}, dimension {i} must be {want}")
    if t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")


def _cache_elem_dtype(layout) -> torch.dtype:
    return torch.uint8 if layout.cache_dtype == PA_CACHE_FP8_E4M3 else torch.bfloat16


def _need_pools(layout, k_cache, v_cache) -> None:
    """K and V pools: the layout's element type and at least num_blocks
    (num_kv_heads, block_size, head_dim) tiles each."""
    n = (int(layout.num_blocks) * int(layout.num_kv_heads) * int(layout.block_size) *
         int(layout.head_dim))
    dt = _cache_elem_dtype(layout)
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, dt, min_numel=n)
        if t.dim() == 4 and (tuple(t.shape[1:]) != (layout.num_kv_heads, layout.block_size,
                                                     layout.head_dim)
                             or t.shape[0] < layout.num_blocks):
            raise ValueError(f"{name}: shape {tuple(t.shape)} does not hold the layout's "
                             f"[{layout.num_blocks}][{layout.num_kv_heads}]"
                             f"[{layout.block_size}][{layout.head_dim}] tiles")


def _need_scales(layout, k_scale, v_scale) -> None:
    fp8 = layout.cache_dtype == PA_CACHE_FP8_E4M3
    _need(k_scale, "k_scale", torch.float32, min_numel=1, optional=not fp8)
    _need(v_scale, "v_scale", torch.float32, min_numel=1, optional=not fp8)


def _need_rows(layout, q, out, rows, num_q_heads, what="q") -> None:
    """q and out: bf16 [rows][num_q_heads][head_dim]."""
    dims = (rows, num_q_heads, int(layout.head_dim))
    _need(q, what, torch.bfloat16, dims)
    if out is not None:
        _need(out, "out", torch.bfloat16, dims)


def _need_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes) -> None:
    _need(q, "q", torch.bfloat16, (None, None, int(layout.head_dim)))
    R, H = int(q.shape[0]), int(q.shape[1])
    _need_rows(layout, q, out, R, H)
    _need_pools(layout, k_cache, v_cache)
    _need(block_table, "block_table", torch.int32, (None, None))
    if block_table.shape[0] < R:
        raise ValueError(f"block_table: {block_table.shape[0]} rows for {R} requests")
    _need(seq_lens, "seq_lens", torch.int32, (R,))
    _need_scales(layout, k_scale, v_scale)
    _need(alibi_slopes, "alibi_slopes", torch.float32, (H,), optional=True)


def _need_partials(tmp_out, max_logits, exp_sums, R, H, D) -> None:
    _need(max_logits, "max_logits", torch.float32, (R, H, None))
    P = int(max_logits.shape[2])
    _need(exp_sums, "exp_sums", torch.float32, (R, H, P))
    _need(tmp_out, "tmp_out", torch.float32, (R, H, P, D))


def pa_kv_cache_bytes(layout: PaKvLayout) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().pa_kv_cache_bytes(ctypes.byref(layout), ctypes.byref(n)), "pa_kv_cache_bytes")
    return int(n.value)


def pa_compute_slot_mapping(slot_mapping, block_table, query_start_loc, seq_lens,
                            block_size: int = 16) -> None:
    _need(seq_lens, "seq_lens", torch.int32, (None,))
    R = int(seq_lens.shape[0])
    _need(query_start_loc, "query_start_loc", torch.int32, (R + 1,))
    _need(block_table, "block_table", torch.int32, (None, None))
    if block_table.shape[0] < R:
        raise ValueError(f"block_table: {block_table.shape[0]} rows for {R} requests")
    _need(slot_mapping, "slot_mapping", torch.int64, (None,))
    _check(lib().pa_compute_slot_mapping(
        _dev(slot_mapping, "slot_mapping"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(query_start_loc, "query_start_loc"),
        _dev(seq_lens, "seq_lens"), seq_lens.shape[0], slot_mapping.shape[0], block_size,
        _stream()), "pa_compute_slot_mapping")


def pa_reshape_and_cache(layout, k_cache, v_cache, key, value, slot_mapping, k_scale=None,
                         v_scale=None) -> None:
    kv = (None, int(layout.num_kv_heads), int(layout.head_dim))
    _need(key, "key", torch.bfloat16, kv)
    _need(value, "value", torch.bfloat16, (key.shape[0],) + kv[1:])
    _need_pools(layout, k_cache, v_cache)
    _need(slot_mapping, "slot_mapping", torch.int64, (None,), min_numel=int(key.shape[0]))
    _need_scales(layout, k_scale, v_scale)
    _check(lib().pa_reshape_and_cache(
        ctypes.byref(layout), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(key, "key"), _dev(value, "value"), key.shape[0],
        _dev(slot_mapping, "slot_mapping"), _dev(k_scale, "k_scale"),
        _dev(v_scale, "v_scale"), _stream()), "pa_reshape_and_cache")


def pa_reshape_and_cache_varlen(layout, k_cache, v_cache, key, value, block_table,
                                query_start_loc, seq_lens, slot_mapping=None, k_scale=None,
                                v_scale=None) -> None:
    kv = (None, int(layout.num_kv_heads), int(layout.head_dim))
    _need(key, "key", torch.bfloat16, kv)
    T = int(key.shape[0])
    _need(value, "value", torch.bfloat16, (T,) + kv[1:])
    _need_pools(layout, k_cache, v_cache)
    _need(seq_lens, "seq_lens", torch.int32, (None,))
    R = int(seq_lens.shape[0])
    _need(query_start_loc, "query_start_loc", torch.int32, (R + 1,))
    _need(block_table, "block_table", torch.int32, (None, None))
    if block_table.shape[0] < R:
        raise ValueError(f"block_table: {block_table.shape[0]} rows for {R} requests")
    _need(slot_mapping, "slot_mapping", torch.int64, (None,), min_numel=T, optional=True)
    _need_scales(layout, k_scale, v_scale)
    _check(lib().pa_reshape_and_cache_varlen(
        ctypes.byref(layout), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(key, "key"), _dev(value, "value"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(query_start_loc, "query_start_loc"),
        _dev(seq_lens, "seq_lens"), seq_lens.shape[0], key.shape[0],
        _dev(slot_mapping, "slot_mapping"), _dev(k_scale, "k_scale"),
        _dev(v_scale, "v_scale"), _stream()), "pa_reshape_and_cache_varlen")


def pa_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int,
              scale: float, k_scale=None, v_scale=None, alibi_slopes=None) -> None:
    _need(out, "out", torch.bfloat16)
    _need_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    _check(lib().pa_decode(
        ctypes.byref(layout), _dev(out, "out"), _dev(q, "q"), q.shape[0], q.shape[1],
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
        _dev(alibi_slopes, "alibi_slopes"), _stream()), "pa_decode")


def pa_decode_plan_for(layout, num_reqs: int, num_q_heads: int, max_seq_len: int) -> PaDecodePlan:
    plan = PaDecodePlan()
    _check(lib().pa_decode_plan_for(ctypes.byref(layout), int(num_reqs), int(num_q_heads),
                                    int(max_seq_len), ctypes.byref(plan)), "pa_decode_plan_for")
    return plan


def pa_decode_auto(layout, out, q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int,
                   scale: float, plan: PaDecodePlan, workspace=None, k_scale=None,
                   v_scale=None, alibi_slopes=None) -> None:
    _need(out, "out", torch.bfloat16)
    _need_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    _need(workspace, "workspace", torch.uint8, optional=True)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_auto(
        ctypes.byref(layout), _dev(out, "out"), _dev(q, "q"), q.shape[0], q.shape[1],
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _dev(alibi_slopes, "alibi_slopes"),
        ctypes.byref(plan), _dev(workspace, "workspace"), nbytes, _stream()), "pa_decode_auto")


def pa_decode_auto_static(layout, out, q, k_cache, v_cache, block_table, seq_lens,
                          max_seq_len: int, scale: float, plan: PaDecodePlan, k_scale=None,
                          v_scale=None, alibi_slopes=None) -> None:
    """pa_decode_auto with the split path's partials in the library's static
    device array (no workspace, nothing allocated)."""
    _need(out, "out", torch.bfloat16)
    _need_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    _check(lib().pa_decode_auto_static(
        ctypes.byref(layout), _dev(out, "out"), _dev(q, "q"), q.shape[0], q.shape[1],
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _dev(alibi_slopes, "alibi_slopes"),
        ctypes.byref(plan), _stream()), "pa_decode_auto_static")


def pa_decode_workspace_size(layout, num_reqs: int, num_q_heads: int) -> int:
    return int(lib().pa_decode_workspace_size(ctypes.byref(layout), int(num_reqs),
                                              int(num_q_heads)))


def pa_decode_balanced(layout, out, q, k_cache, v_cache, block_table, seq_lens,
                       max_seq_len: int, scale: float, workspace, k_scale=None,
                       v_scale=None, alibi_slopes=None) -> None:
    _need(out, "out", torch.bfloat16)
    _need_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    _need(workspace, "workspace", torch.uint8)
    _check(lib().pa_decode_balanced(
        ctypes.byref(layout), _dev(out, "out"), _dev(q, "q"), q.shape[0], q.shape[1],
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
        _dev(alibi_slopes, "alibi_slopes"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream()), "pa_decode_balanced")


def pa_decode_partitioned(layout, q, k_cache, v_cache, block_table, seq_lens,
                          max_seq_len: int, scale: float, partition_size: int, tmp_out,
                          max_logits, exp_sums, k_scale=None, v_scale=None,
                          alibi_slopes=None) -> None:
    _need_decode(layout, None, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    _need_partials(tmp_out, max_logits, exp_sums, q.shape[0], q.shape[1], layout.head_dim)
    _check(lib().pa_decode_partitioned(
        ctypes.byref(layout), _dev(q, "q"), q.shape[0], q.shape[1], _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_table, "block_table"), block_table.shape[1],
        _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale), _dev(k_scale, "k_scale"),
        _dev(v_scale, "v_scale"), _dev(alibi_slopes, "alibi_slopes"), int(partition_size),
        max_logits.shape[2],
        _dev(tmp_out, "tmp_out"), _dev(max_logits, "max_logits"), _dev(exp_sums, "exp_sums"),
        _stream()), "pa_decode_partitioned")


def pa_decode_partitioned_range(layout, q, k_cache, v_cache, block_table, seq_lens,
                                max_seq_len: int, scale: float, partition_size: int,
                                part_begin: int, part_end: int, tmp_out, max_logits, exp_sums,
                                k_scale=None, v_scale=None, alibi_slopes=None) -> None:
    _need_decode(layout, None, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    _need_partials(tmp_out, max_logits, exp_sums, q.shape[0], q.shape[1], layout.head_dim)
    _check(lib().pa_decode_partitioned_range(
        ctypes.byref(layout), _dev(q, "q"), q.shape[0], q.shape[1], _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_table, "block_table"), block_table.shape[1],
        _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale), _dev(k_scale, "k_scale"),
        _dev(v_scale, "v_scale"), _dev(alibi_slopes, "alibi_slopes"), int(partition_size),
        max_logits.shape[2], int(part_begin), int(part_end), _dev(tmp_out, "tmp_out"),
        _dev(max_logits, "max_logits"), _dev(exp_sums, "exp_sums"), _stream()),
        "pa_decode_partitioned_range")


def pa_merge_partitions(out, tmp_out, max_logits, exp_sums, seq_lens,
                        partition_size: int) -> None:
    _need(out, "out", torch.bfloat16, (None, None, None))
    R, H, D = (int(x) for x in out.shape)
    _need(seq_lens, "seq_lens", torch.int32, (R,))
    _need_partials(tmp_out, max_logits, exp_sums, R, H, D)
    _check(lib().pa_merge_partitions(
        _dev(out, "out"), _dev(tmp_out, "tmp_out"), _dev(max_logits, "max_logits"),
        _dev(exp_sums, "exp_sums"), _dev(seq_lens, "seq_lens"), seq_lens.shape[0],
        out.shape[1], out.shape[2], int(partition_size), max_logits.shape[2], _stream()),
        "pa_merge_partitions")


def pa_decode_append(layout, out, q, k_cache, v_cache, key, value, slot_mapping, block_table,
                     seq_lens, max_seq_len: int, scale: float, k_scale=None, v_scale=None,
                     alibi_slopes=None) -> None:
    _need(out, "out", torch.bfloat16)
    _need_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    kv = (int(q.shape[0]), int(layout.num_kv_heads), int(layout.head_dim))
    _need(key, "key", torch.bfloat16, kv)
    _need(value, "value", torch.bfloat16, kv)
    _need(slot_mapping, "slot_mapping", torch.int64, (None,), min_numel=kv[0], optional=True)
    _check(lib().pa_decode_append(
        ctypes.byref(layout), _dev(out, "out"), _dev(q, "q"), q.shape[0], q.shape[1],
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(key, "key"),
        _dev(value, "value"), _dev(slot_mapping, "slot_mapping"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _dev(alibi_slopes, "alibi_slopes"),
        _stream()), "pa_decode_append")


def pa_measure_read_stream(src, sink, work_groups: int = 0) -> None:
    """One streaming read of the whole of `src` (device tensor) on the
    current stream; `sink`: a device tensor with at least one int32."""
    _check(lib().pa_measure_read_stream(_dev(src, "src"), src.numel() * src.element_size(),
                                        _dev(sink, "sink"), int(work_groups), _stream()),
           "pa_measure_read_stream")


def pa_decode_shared_prefix(layout, out, q, k_cache, v_cache, block_table, seq_lens,
                            max_seq_len: int, scale: float, shared_blocks: int,
                            partition_size: int, tmp_out, max_logits, exp_sums,
                            k_scale=None, v_scale=None, alibi_slopes=None) -> None:
    _need(out, "out", torch.bfloat16)
    _need_decode(layout, out, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 alibi_slopes)
    _need_partials(tmp_out, max_logits, exp_sums, q.shape[0], q.shape[1], layout.head_dim)
    _check(lib().pa_decode_shared_prefix(
        ctypes.byref(layout), _dev(out, "out"), _dev(q, "q"), q.shape[0], q.shape[1],
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _dev(alibi_slopes, "alibi_slopes"),
        int(shared_blocks), int(partition_size), max_logits.shape[2], _dev(tmp_out, "tmp_out"),
        _dev(max_logits, "max_logits"), _dev(exp_sums, "exp_sums"), _stream()),
        "pa_decode_shared_prefix")


def pa_prefill_varlen(layout, out, q, k_cache, v_cache, query_start_loc, seq_lens,
                      block_table, max_query_len: int, max_seq_len: int, scale: float,
                      k_scale=None, v_scale=None, alibi_slopes=None) -> None:
    _need(q, "q", torch.bfloat16, (None, None, int(layout.head_dim)))
    T, H = int(q.shape[0]), int(q.shape[1])
    _need_rows(layout, q, out, T, H)
    _need(out, "out", torch.bfloat16)
    _need_pools(layout, k_cache, v_cache)
    _need(seq_lens, "seq_lens", torch.int32, (None,))
    R = int(seq_lens.shape[0])
    _need(query_start_loc, "query_start_loc", torch.int32, (R + 1,))
    _need(block_table, "block_table", torch.int32, (None, None))
    if block_table.shape[0] < R:
        raise ValueError(f"block_table: {block_table.shape[0]} rows for {R} requests")
    _need_scales(layout, k_scale, v_scale)
    _need(alibi_slopes, "alibi_slopes", torch.float32, (H,), optional=True)
    _check(lib().pa_prefill_varlen(
        ctypes.byref(layout), _dev(out, "out"), _dev(q, "q"), q.shape[0], q.shape[1],
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(query_start_loc, "query_start_loc"), _dev(seq_lens, "seq_lens"),
        _dev(block_table, "block_table"), block_table.shape[1], seq_lens.shape[0],
        int(max_query_len), int(max_seq_len), float(scale), _dev(k_scale, "k_scale"),
        _dev(v_scale, "v_scale"), _dev(alibi_slopes, "alibi_slopes"), _stream()),
        "pa_prefill_varlen")


def pa_debug_gather_kv(layout, k_out, v_out, k_cache, v_cache, block_table, seq_lens,
                       cu_seq_lens, max_seq_len: int) -> None:
    _need_pools(layout, k_cache, v_cache)
    _need(seq_lens, "seq_lens", torch.int32, (None,))
    R = int(seq_lens.shape[0])
    _need(cu_seq_lens, "cu_seq_lens", torch.int32, (R + 1,))
    _need(block_table, "block_table", torch.int32, (None, None))
    if block_table.shape[0] < R:
        raise ValueError(f"block_table: {block_table.shape[0]} rows for {R} requests")
    dt = _cache_elem_dtype(layout)
    _need(k_out, "k_out", dt, (None, int(layout.num_kv_heads), int(layout.head_dim)))
    _need(v_out, "v_out", dt, tuple(k_out.shape))
    _check(lib().pa_debug_gather_kv(
        ctypes.byref(layout), _dev(k_out, "k_out"), _dev(v_out, "v_out"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), _dev(cu_seq_lens, "cu_seq_lens"),
        seq_lens.shape[0], int(max_seq_len), _stream()), "pa_debug_gather_kv")


def pa_debug_fp8_to_f32(codes, out) -> None:
    _need(codes, "codes", torch.uint8)
    _need(out, "out", torch.float32, min_numel=codes.numel())
    _check(lib().pa_debug_fp8_to_f32(_dev(codes, "codes"), _dev(out, "out"), codes.numel(),
                                     _stream()), "pa_debug_fp8_to_f32")


def pa_debug_fp8_to_f16(codes, out) -> None:
    _need(codes, "codes", torch.uint8)
    if out is None or out.dtype not in (torch.int16, torch.float16, torch.uint16):
        raise ValueError("out: a 16-bit tensor is required")
    _need(out, "out", out.dtype, min_numel=codes.numel())
    _check(lib().pa_debug_fp8_to_f16(_dev(codes, "codes"), _dev(out, "out"), codes.numel(),
                                     _stream()), "pa_debug_fp8_to_f16")


def pa_validate_metadata(block_table, query_start_loc, seq_lens, slot_mapping,
                         num_blocks: int, block_size: int = 16) -> int:
    """Host check of metadata (numpy arrays); returns the status code."""
    import numpy as np

    def host(a, dt):
        return None if a is None else np.ascontiguousarray(a, dtype=dt)
    bt = host(block_table, np.int32)
    qsl = host(query_start_loc, np.int32)
    sl = host(seq_lens, np.int32)
    sm = host(slot_mapping, np.int64)

    def p(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    return int(lib().pa_validate_metadata(
        p(bt), bt.shape[1], p(qsl), p(sl), sl.shape[0], p(sm),
        0 if sm is None else sm.shape[0], int(num_blocks), int(block_size)))
