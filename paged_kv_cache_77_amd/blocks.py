"""Python binding of the host block manager (include/pa_blocks.h, in libpa.so).

Marshalling only: the pool, its free queue, reference counts and prefix
index live in the C++ library.  ``BlockPool.allocate_prompt`` returns the
block-table row a request's attention kernels read.
"""
from __future__ import annotations

import ctypes
from typing import Sequence

import numpy as np

from . import PA_OK, PaError, lib

_P = ctypes.c_void_p
_I = ctypes.c_int32
_U64 = ctypes.c_uint64

_SIGS = {
    "pa_block_hashes": ([_P, _I, _I, _U64, _P], _I),
    "pa_pool_create": ([_I, _I, ctypes.POINTER(_P)], _I),
    "pa_pool_destroy": ([_P], None),
    "pa_pool_num_free": ([_P], _I),
    "pa_pool_usage": ([_P], ctypes.c_double),
    "pa_pool_ref_count": ([_P, _I], _I),
    "pa_pool_lookup": ([_P, _U64], _I),
    "pa_pool_get_new_blocks": ([_P, _I, _P], _I),
    "pa_pool_touch": ([_P, _P, _I], _I),
    "pa_pool_free_blocks": ([_P, _P, _I], _I),
    "pa_pool_cache_block": ([_P, _I, _U64], _I),
    "pa_pool_allocate_prompt": ([_P, _P, _I, _I, _I, _P, _I, _P], _I),
    "pa_pool_commit": ([_P, _P, _P, _I], _I),
    "pa_pool_free_request": ([_P, _P, _I], _I),
    "pa_map_to_kernel_blocks": ([_P, _I, _I, _P], _I),
}
_ready = False


def _lib():
    global _ready
    L = lib()
    if not _ready:
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _ready = True
    return L


def _check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PaError(status, where)


def _i32(a) -> np.ndarray:
    if isinstance(a, np.ndarray) and a.dtype == np.int32:
        return np.ascontiguousarray(a)
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).astype(np.int32))


def _u64(a) -> np.ndarray:
    if isinstance(a, np.ndarray) and a.dtype == np.uint64:
        return np.ascontiguousarray(a)
    return np.ascontiguousarray(np.asarray([int(x) for x in a], dtype=np.uint64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P) if a.size else None


def block_hashes(tokens: Sequence[int], block_size: int = 16, extra_key: int = 0) -> list:
    """Chained hashes of the full blocks of ``tokens`` (pa_block_hashes)."""
    t = _i32(tokens)
    out = np.zeros(max(1, len(t) // block_size), dtype=np.uint64)
    n = _lib().pa_block_hashes(_ptr(t), len(t), block_size, extra_key, _ptr(out))
    if n < 0:
        raise PaError(n, "pa_block_hashes")
    return [int(x) for x in out[:n]]


def map_to_kernel_blocks(ids: Sequence[int], blocks_per_kv_block: int) -> list:
    """Kernel block ids of manager blocks of blocks_per_kv_block kernel blocks."""
    a = _i32(ids)
    out = np.zeros(max(1, len(a) * blocks_per_kv_block), dtype=np.int32)
    _check(_lib().pa_map_to_kernel_blocks(_ptr(a), len(a), blocks_per_kv_block, _ptr(out)),
           "pa_map_to_kernel_blocks")
    return [int(x) for x in out[:len(a) * blocks_per_kv_block]]


class BlockPool:
    """One pool of physical KV blocks (ids 0 .. num_blocks-1, 0 = null block)."""

    def __init__(self, num_blocks: int, caching: bool = True):
        h = _P()
        _check(_lib().pa_pool_create(num_blocks, 1 if caching else 0, ctypes.byref(h)),
               "pa_pool_create")
        self._h = h
        self.num_blocks = num_blocks

    def close(self) -> None:
        if self._h:
            _lib().pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return int(_lib().pa_pool_num_free(self._h))

    def usage(self) -> float:
        return float(_lib().pa_pool_usage(self._h))

    def ref_count(self, block_id: int) -> int:
        return int(_lib().pa_pool_ref_count(self._h, block_id))

    def lookup(self, h: int) -> int:
        return int(_lib().pa_pool_lookup(self._h, h))

    def get_new_blocks(self, n: int) -> list:
        out = np.zeros(max(n, 1), dtype=np.int32)
        _check(_lib().pa_pool_get_new_blocks(self._h, n, _ptr(out)), "pa_pool_get_new_blocks")
        return [int(x) for x in out[:n]]

    def touch(self, blocks) -> None:
        b = _i32(blocks)
        _check(_lib().pa_pool_touch(self._h, _ptr(b), len(b)), "pa_pool_touch")

    def free_blocks(self, blocks) -> None:
        b = _i32(blocks)
        _check(_lib().pa_pool_free_blocks(self._h, _ptr(b), len(b)), "pa_pool_free_blocks")

    def cache_block(self, block_id: int, h: int) -> None:
        _check(_lib().pa_pool_cache_block(self._h, block_id, h), "pa_pool_cache_block")

    def allocate_prompt(self, hashes, num_tokens: int, block_size: int = 16):
        """(block-table row, number of tokens whose K/V are already cached)."""
        hs = _u64(hashes)
        nblk = -(-num_tokens // block_size)
        out = np.zeros(max(nblk, 1), dtype=np.int32)
        cached = ctypes.c_int32(0)
        _check(_lib().pa_pool_allocate_prompt(self._h, _ptr(hs), len(hs), num_tokens,
                                              block_size, _ptr(out), nblk,
                                              ctypes.byref(cached)),
               "pa_pool_allocate_prompt")
        return out[:nblk].tolist(), int(cached.value)

    def commit(self, blocks, hashes) -> None:
        b, hs = _i32(blocks), _u64(hashes)
        n = min(len(b), len(hs))
        _check(_lib().pa_pool_commit(self._h, _ptr(b), _ptr(hs), n), "pa_pool_commit")

    def free_request(self, blocks) -> None:
        b = _i32(blocks)
        _check(_lib().pa_pool_free_request(self._h, _ptr(b), len(b)), "pa_pool_free_request")
