"""Full-size configurations and their oracle results, computed once per
test session and shared by the GPU tests that run them (the oracle at full
size takes seconds, the generation of a configuration up to tens)."""
import functools

import numpy as np

import oracle
from paged_kv_cache_77_amd import workloads as wl


@functools.lru_cache(maxsize=None)
def config(cfg: int):
    return wl.config_workload(cfg)


@functools.lru_cache(maxsize=None)
def after_write(cfg: int):
    """(slot_mapping, k_pool, v_pool) of configuration cfg after this step's
    new tokens are written (the generated pools when it writes none)."""
    w = config(cfg)
    if not w.writes_new_kv:
        return None, w.k_pool, w.v_pool
    sm = oracle.slot_mapping(w.block_table, w.query_start_loc, w.seq_lens, 16)
    kp, vp = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.k_new, w.v_new, sm, 16,
                                      cache_dtype=w.cache_dtype, k_scale=w.k_scale,
                                      v_scale=w.v_scale)
    return sm, kp, vp


@functools.lru_cache(maxsize=None)
def decode_ref(cfg: int) -> np.ndarray:
    """The oracle's decode of every request and head of configuration cfg."""
    w = config(cfg)
    _, kp, vp = after_write(cfg)
    return oracle.decode(w, k_pool=kp, v_pool=vp)


@functools.lru_cache(maxsize=None)
def prefill_ref(cfg: int) -> np.ndarray:
    """The oracle's varlen prefill of every row and head of configuration cfg."""
    w = config(cfg)
    _, kp, vp = after_write(cfg)
    return oracle.prefill_varlen(w, k_pool=kp, v_pool=vp)
