"""Pools past 4 GiB: tiles whose byte offsets need more than 32 bits."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_77_amd as pa
from paged_kv_cache_77_amd import workloads as wl
from paged_kv_cache_77_amd import device as dv
from tests.parity import check_bf16

pytestmark = pytest.mark.gpu

BIG_BLOCKS = 140_000          # x 8 KV heads x 16 x 128 x bf16 = 4.59 GB per pool


def _to_big_pool(d, w):
    """The same logical data with every used block moved to id BIG_BLOCKS-1-id
    of a 4.59 GB pool.  Every other element of the pool holds bf16 NaN, as
    the unused slots of the small pools do, so a stray read past 2^32 shows
    up in the outputs instead of reading whatever the memory held."""
    shape = (BIG_BLOCKS,) + tuple(d.k_cache.shape[1:])
    kb = torch.full(shape, float("nan"), dtype=d.k_cache.dtype, device="cuda")
    vb = torch.full(shape, float("nan"), dtype=d.v_cache.dtype, device="cuda")
    used = np.unique(w.block_table[w.block_table >= 0])
    old = torch.from_numpy(used).long().cuda()
    new = BIG_BLOCKS - 1 - old
    kb[new] = d.k_cache[old]
    vb[new] = d.v_cache[old]
    bt = w.block_table.copy()
    bt[bt >= 0] = BIG_BLOCKS - 1 - bt[bt >= 0]
    big = dataclasses.replace(
        d, k_cache=kb, v_cache=vb, block_table=torch.from_numpy(bt).cuda(),
        layout=pa.make_layout(BIG_BLOCKS, w.num_kv_heads, w.head_dim, pa.PA_CACHE_BF16))
    return big, used


def test_decode_and_append_in_a_pool_past_4gib():
    """Decode step with its write (one launch), split-KV and the single pass
    over blocks at byte offsets up to 4.59 GB: pools bit-exact at the moved
    blocks, outputs against the oracle on the original small pool."""
    print("\n[case] decode + append, 4.59 GB pools", flush=True)
    ctx = [300, 1000, 17, 2049, 1, 4096, 513, 64]
    w = wl.make_workload(name="t", seq_lens=ctx, q_lens=[1] * len(ctx), num_q_heads=32,
                         num_kv_heads=8, head_dim=128, seed=61, writes_new_kv=True,
                         bt_extra_cols=2)
    d = dv.to_device(w)
    big, used = _to_big_pool(d, w)
    assert (BIG_BLOCKS - 1 - int(used.max())) * 8 * 16 * 128 * 2 > 2 ** 32   # every moved tile
    sm = torch.empty((w.num_reqs,), dtype=torch.int64, device="cuda")
    out = torch.full((w.num_reqs, 32, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    dv.run_decode_append(big, out, sm)
    out2 = torch.full_like(out, float("nan"))
    dv.run_decode_partitioned(big, out2, 512)
    torch.cuda.synchronize()
    ref_sm = oracle.slot_mapping(w.block_table, w.query_start_loc, w.seq_lens, 16)
    kp, vp = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.k_new, w.v_new, ref_sm, 16)
    moved = BIG_BLOCKS - 1 - used
    assert np.array_equal(sm.cpu().numpy(),
                          (BIG_BLOCKS - 1 - ref_sm // 16) * 16 + ref_sm % 16)
    assert np.array_equal(dv.bits_of(big.k_cache[torch.from_numpy(moved).cuda()]), kp[used])
    assert np.array_equal(dv.bits_of(big.v_cache[torch.from_numpy(moved).cuda()]), vp[used])
    ref = oracle.decode(w, k_pool=kp, v_pool=vp)
    check_bf16(dv.bits_of(out), ref, "append, big pool")
    check_bf16(dv.bits_of(out2), ref, "split-KV, big pool")


def test_prefill_in_a_pool_past_4gib():
    """Varlen chunked prefill (with decode rows) reading through the moved
    blocks of a 4.59 GB pool."""
    print("\n[case] prefill, 4.59 GB pools", flush=True)
    w = wl.make_workload(name="t", seq_lens=[1, 700, 300, 2100], q_lens=[1, 129, 300, 1],
                         num_q_heads=32, num_kv_heads=8, head_dim=128, seed=62,
                         writes_new_kv=False, bt_extra_cols=2)
    d = dv.to_device(w)
    big, _ = _to_big_pool(d, w)
    out = torch.full((w.num_tokens, 32, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    dv.run_prefill(big, out)
    torch.cuda.synchronize()
    check_bf16(dv.bits_of(out), oracle.prefill_varlen(w), "prefill, big pool")
