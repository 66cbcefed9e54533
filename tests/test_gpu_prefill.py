"""GPU parity of varlen chunked prefill (MFMA tiles) and its decode rows."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_77_amd import workloads as wl
from paged_kv_cache_77_amd import device as dv
from tests import full_size as full
from tests.parity import check_bf16

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _run(w, write=True):
    d = dv.to_device(w)
    kp, vp = w.k_pool, w.v_pool
    if write and w.writes_new_kv:
        sm = torch.empty((w.num_tokens,), dtype=torch.int64, device="cuda")
        dv.write_new_kv(d, sm)
        ref_sm = oracle.slot_mapping(w.block_table, w.query_start_loc, w.seq_lens, 16)
        kp, vp = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.k_new, w.v_new, ref_sm, 16,
                                          cache_dtype=w.cache_dtype, k_scale=w.k_scale,
                                          v_scale=w.v_scale)
        assert np.array_equal(dv.bits_of(d.k_cache) if w.cache_dtype == "bf16"
                              else d.k_cache.cpu().numpy(), kp), "K pool after the write"
    out = torch.full((w.num_tokens, w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    dv.run_prefill(d, out)
    torch.cuda.synchronize()
    return dv.bits_of(out), kp, vp


MIX = dict(seq_lens=[1, 40, 300, 129, 700, 64, 2, 5000],
           q_lens=[1, 17, 300, 2, 129, 0, 2, 1000])


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (4, 2, 64), (28, 4, 128), (8, 8, 128),
                                      (16, 1, 64)])
def test_prefill_mixed_batch(hq, hkv, d):
    _announce(f"prefill mix hq={hq} hkv={hkv} d={d}")
    w = wl.make_workload(name="t", num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                         seed=41 + hq + d, bt_extra_cols=2, **MIX)
    got, kp, vp = _run(w)
    ref = oracle.prefill_varlen(w, k_pool=kp, v_pool=vp)
    check_bf16(got, ref, f"prefill {hq}/{hkv}/{d}")


def test_prefill_fp8_cache():
    _announce("prefill fp8 cache")
    w = wl.make_workload(name="t", num_q_heads=28, num_kv_heads=4, head_dim=128, seed=47,
                         cache_dtype="fp8", writes_new_kv=False, **MIX)
    got, _, _ = _run(w)
    check_bf16(got, oracle.prefill_varlen(w), "prefill fp8")


def test_prefill_whole_prompt_and_orders():
    """q_len == seq_len (textbook causal) and the prefill row placed first or last."""
    _announce("prefill whole prompt / order")
    for order in ([0, 1, 2], [2, 0, 1]):
        sl = np.array([200, 1, 77])[order]
        ql = np.array([200, 1, 77])[order]
        w = wl.make_workload(name="t", seq_lens=sl, q_lens=ql, num_q_heads=8, num_kv_heads=2,
                             head_dim=128, seed=48)
        got, kp, vp = _run(w)
        check_bf16(got, oracle.prefill_varlen(w, k_pool=kp, v_pool=vp), f"order {order}")


@pytest.mark.parametrize("prefill_first,share", [(False, 0), (True, 0), (False, 16)])
def test_config4_scaled(prefill_first, share):
    """The mixed chunked-prefill configuration at 1/8 scale: 16 decode rows and
    a 256-token chunk on a 768-token prefix (optionally 16 decode rows share
    the chunk's first cached blocks)."""
    _announce(f"config 4 / 8, prefill_first={prefill_first}, share={share}")
    w = wl.config_workload(4, scale_down=8, prefill_first=prefill_first,
                           share_prefix_rows=share)
    got, kp, vp = _run(w)
    check_bf16(got, oracle.prefill_varlen(w, k_pool=kp, v_pool=vp), "config 4 / 8")


def test_chunked_equals_whole():
    """One 512-token chunk vs two 256-token chunks (the first written to the
    cache, the second resuming on it): same rows within tolerance."""
    _announce("chunk composition")
    base = wl.make_workload(name="t", seq_lens=[1536], q_lens=[512], num_q_heads=8,
                            num_kv_heads=2, head_dim=128, seed=49)
    got_whole, kp, vp = _run(base)
    ref = oracle.prefill_varlen(base, k_pool=kp, v_pool=vp)
    check_bf16(got_whole, ref, "whole chunk")
    # second half of the chunk as its own step on the same cache contents
    d = dv.to_device(dataclasses.replace(base, k_pool=kp, v_pool=vp))
    half = dataclasses.replace(base, q_lens=np.array([256], np.int32),
                               query_start_loc=np.array([0, 256], np.int32), q=base.q[256:],
                               k_new=None, v_new=None, writes_new_kv=False, k_pool=kp, v_pool=vp)
    d2 = dv.to_device(half)
    out = torch.empty((256, 8, 128), dtype=torch.bfloat16, device="cuda")
    dv.run_prefill(d2, out)
    first = dataclasses.replace(half, seq_lens=np.array([1280], np.int32), q=base.q[:256])
    d1 = dv.to_device(first)
    out1 = torch.empty((256, 8, 128), dtype=torch.bfloat16, device="cuda")
    dv.run_prefill(d1, out1)
    torch.cuda.synchronize()
    del d
    halves = np.concatenate([dv.bits_of(out1), dv.bits_of(out)])
    check_bf16(halves, ref, "two chunks")


@pytest.mark.parametrize("hq,hkv,d,prefill_first,alibi", [
    (32, 8, 128, False, False), (32, 8, 128, True, True), (16, 8, 64, False, False),
    (8, 8, 128, True, False)])
def test_varlen_one_launch_batches(hq, hkv, d, prefill_first, alibi):
    """Batches with enough decode rows ((rows - 1) x KV heads >= the compute
    units) that pa_prefill_varlen runs prefill tiles and decode rows in one
    launch; every row is checked against the oracle.  Includes a whole
    prompt, a chunk on a cached prefix, a row with no queries, contexts 1, 16
    and 17, and both row orders."""
    _announce(f"varlen one launch hq={hq} hkv={hkv} d={d} prefill_first={prefill_first} "
              f"alibi={alibi}")
    rng = np.random.default_rng(hq * 10 + d)
    n_dec = 40
    dec = [int(x) for x in rng.integers(1, 1500, size=n_dec)]
    dec[:3] = [1, 16, 17]
    pre_sl, pre_ql = [500, 129, 50], [300, 129, 0]
    sl = pre_sl + dec if prefill_first else dec + pre_sl
    ql = pre_ql + [1] * n_dec if prefill_first else [1] * n_dec + pre_ql
    w = wl.make_workload(name="t", seq_lens=sl, q_lens=ql, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, seed=70 + hq + d, bt_extra_cols=2, alibi=alibi)
    got, kp, vp = _run(w)
    check_bf16(got, oracle.prefill_varlen(w, k_pool=kp, v_pool=vp), "varlen one launch")


def test_config4_full_size():
    """Full mixed batch (128 decode rows + 2048-token chunk on 6144 cached
    tokens) in the benchmark's launch configuration: the write's slots and
    pools bit-exact, then every row and head -- the 128 decode rows and all
    2048 rows of the chunk -- against the oracle."""
    _announce("config 4 full size, every row")
    w = full.config(4)
    d = dv.to_device(w)
    sm = torch.empty((w.num_tokens,), dtype=torch.int64, device="cuda")
    dv.write_new_kv_fused(d, sm)
    out = torch.full((w.num_tokens, w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    dv.run_prefill(d, out)
    torch.cuda.synchronize()
    ref_sm, kp, vp = full.after_write(4)
    assert np.array_equal(sm.cpu().numpy(), ref_sm)
    assert np.array_equal(dv.bits_of(d.k_cache), kp) and np.array_equal(dv.bits_of(d.v_cache), vp)
    del d
    got = dv.bits_of(out)
    ref = full.prefill_ref(4)
    pre = int(w.query_start_loc[-2])            # the prefill row's first token
    check_bf16(got[:pre], ref[:pre], "config 4 decode rows")
    check_bf16(got[pre:], ref[pre:], "config 4 prefill chunk")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_chunk_invariance_config4_shape(cache):
    """A chunk resumes on the cached blocks of the earlier chunks and sees
    exactly what an unchunked pass sees ("第11章 分块预填充与混合批处理"
    §11.6; "vLLM 深度解析（二）" §5.2): at the mixed batch's chunk shape (32 q
    / 8 KV heads, d 128), one 2048-token chunk on a 6144-token prefix against
    the same tokens as two 1024-token chunks -- the first written to the
    cache and computed on the 6144 prefix, the second written and computed on
    the 7168 prefix.  Pools after both writes are bit-identical; both
    outputs are within tolerance of the oracle and of each other."""
    _announce(f"chunk invariance at the config-4 shape, {cache}")
    w = wl.make_workload(name="t", seq_lens=[8192], q_lens=[2048], num_q_heads=32,
                         num_kv_heads=8, head_dim=128, seed=88, cache_dtype=cache,
                         bt_extra_cols=1)
    def pools(d):
        if cache == "bf16":
            return dv.bits_of(d.k_cache), dv.bits_of(d.v_cache)
        return d.k_cache.cpu().numpy(), d.v_cache.cpu().numpy()
    shape = (2048, 32, 128)
    # one chunk
    d = dv.to_device(w)
    sm = torch.empty((2048,), dtype=torch.int64, device="cuda")
    dv.write_new_kv(d, sm)
    whole = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dv.run_prefill(d, whole)
    torch.cuda.synchronize()
    kp1, vp1 = pools(d)
    del d
    # two chunks over one set of pools
    d = dv.to_device(w)
    halves = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    for c, seq in ((0, 7168), (1, 8192)):
        rows = slice(1024 * c, 1024 * (c + 1))
        wc = dataclasses.replace(w, seq_lens=np.array([seq], np.int32),
                                 q_lens=np.array([1024], np.int32),
                                 query_start_loc=np.array([0, 1024], np.int32), q=w.q[rows],
                                 k_new=w.k_new[rows], v_new=w.v_new[rows])
        dc = dataclasses.replace(
            d, w=wc, q=d.q[rows], k_new=d.k_new[rows], v_new=d.v_new[rows],
            seq_lens=torch.tensor([seq], dtype=torch.int32, device="cuda"),
            query_start_loc=torch.tensor([0, 1024], dtype=torch.int32, device="cuda"),
            max_seq_len=seq, max_query_len=1024)
        smc = torch.empty((1024,), dtype=torch.int64, device="cuda")
        dv.write_new_kv(dc, smc)
        dv.run_prefill(dc, halves[rows])
        torch.cuda.synchronize()
        assert np.array_equal(smc.cpu().numpy(), sm[rows].cpu().numpy())
    kp2, vp2 = pools(d)
    del d
    assert np.array_equal(kp1, kp2) and np.array_equal(vp1, vp2)
    ref = oracle.prefill_varlen(w, k_pool=kp1, v_pool=vp1)
    g_whole, g_halves = dv.bits_of(whole), dv.bits_of(halves)
    check_bf16(g_whole, ref, f"one chunk ({cache})")
    check_bf16(g_halves, ref, f"two chunks ({cache})")
    check_bf16(g_halves, oracle.bf16_bits_to_f64(g_whole), f"two chunks vs one ({cache})")


@pytest.mark.parametrize("hq,hkv,d,cache", [(32, 8, 128, "bf16"), (28, 4, 128, "fp8"),
                                            (4, 2, 64, "bf16")])
def test_prefill_alibi(hq, hkv, d, cache):
    """ALiBi slopes (2^(-8(h+1)/Hq)) on the mixed batch: prefill rows take
    slope * (t - p), the decode rows slope * (t - seq_len + 1)."""
    _announce(f"prefill alibi hq={hq} hkv={hkv} d={d} {cache}")
    w = wl.make_workload(name="t", num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                         seed=60 + hq + d, cache_dtype=cache, alibi=True, **MIX)
    got, kp, vp = _run(w)
    check_bf16(got, oracle.prefill_varlen(w, k_pool=kp, v_pool=vp), "prefill alibi")


def test_prefill_fp8_cache_with_new_tokens():
    """The whole fp8 step: quantising write of the new tokens, then prefill
    and decode rows over the fp8 cache."""
    _announce("prefill fp8 with quantising write")
    w = wl.make_workload(name="t", num_q_heads=28, num_kv_heads=4, head_dim=128, seed=61,
                         cache_dtype="fp8", **MIX)
    got, kp, vp = _run(w)
    check_bf16(got, oracle.prefill_varlen(w, k_pool=kp, v_pool=vp), "prefill fp8 + write")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_prefill_zero_query_is_causal_mean(cache):
    """Q = 0: every visible weight is exp(0) = 1, exact in any precision, so
    query i's output is the plain mean of V over keys 0..p_i (a closed form,
    computed here from the gathered cache rows, not from the oracle's
    softmax).  Checks the causal window, the partial last tile and that the
    softmax denominator counts exactly the weights multiplied into V."""
    _announce(f"prefill zero query {cache}")
    w = wl.make_workload(name="t", seq_lens=[300, 129, 2000, 65], q_lens=[300, 64, 500, 65],
                         num_q_heads=8, num_kv_heads=2, head_dim=128, seed=48,
                         cache_dtype=cache, writes_new_kv=False, zero_q=True)
    got, _, _ = _run(w, write=False)
    vals = oracle.cache_values(w.v_pool, w.cache_dtype, float(w.v_scale))
    ref = np.full((w.num_tokens, w.num_q_heads, w.head_dim), np.nan)
    for r in range(w.num_reqs):
        L, ql = int(w.seq_lens[r]), int(w.q_lens[r])
        V = oracle.gather_kv(vals, w.block_table[r], L, 16)          # [L, Hkv, d]
        cum = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None, None]
        row0 = int(w.query_start_loc[r])
        for i, p in enumerate(oracle.token_positions(L, ql)):
            for h in range(w.num_q_heads):
                ref[row0 + i, h] = cum[p, h // w.group_size]
    check_bf16(got, ref, f"prefill zero query {cache}")
