"""GPU parity of the write path and the block addressing (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_77_amd import workloads as wl
from paged_kv_cache_77_amd import device as dv
import paged_kv_cache_77_amd as pa

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def test_fp8_conversion_all_codes():
    _announce("fp8 e4m3fn decode, 256 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    pa.pa_debug_fp8_to_f32(codes, out)
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.fp8_e4m3fn_to_f64(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_fp8_to_f16_conversion_all_codes():
    """The f16 conversion of the decode kernels' FP8 V path, all 256 codes:
    exact (every finite E4M3FN value is an f16 value), NaN stays NaN."""
    _announce("fp8 e4m3fn -> f16, 256 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    out = torch.empty(256, dtype=torch.int16, device="cuda")
    pa.pa_debug_fp8_to_f16(codes, out)
    got = out.cpu().numpy().view(np.float16).astype(np.float64)
    ref = oracle.fp8_e4m3fn_to_f64(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def _write_and_check(w):
    d = dv.to_device(w)
    T = w.num_tokens
    sm = torch.full((T,), -7, dtype=torch.int64, device="cuda")
    dv.write_new_kv(d, sm)
    torch.cuda.synchronize()
    ref_sm = oracle.slot_mapping(w.block_table, w.query_start_loc, w.seq_lens, 16)
    got_sm = sm.cpu().numpy()
    assert np.array_equal(got_sm, ref_sm), "slot mapping"
    kp, vp = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.k_new, w.v_new, ref_sm, 16)
    assert np.array_equal(dv.bits_of(d.k_cache), kp), "K pool after scatter"
    assert np.array_equal(dv.bits_of(d.v_cache), vp), "V pool after scatter"
    return d, kp, vp


@pytest.mark.parametrize("cfg,sd", [(1, None), (2, None), (4, 8)])
def test_slot_mapping_and_scatter_configs(cfg, sd):
    _announce(f"slot mapping + scatter, config {cfg} scale_down {sd}")
    _write_and_check(wl.config_workload(cfg, scale_down=sd))


def test_scatter_ragged_and_padding_slots():
    _announce("scatter ragged q_lens, negative slots skipped")
    w = wl.make_workload(name="t", seq_lens=[1, 16, 17, 40, 300, 33], q_lens=[1, 16, 3, 0, 40, 2],
                         num_q_heads=8, num_kv_heads=4, head_dim=128, seed=21, pool_blocks=40)
    d, kp, vp = _write_and_check(w)
    # padding: slot -1 leaves the cache untouched
    before = dv.bits_of(d.k_cache)
    sm = torch.full((w.num_tokens,), -1, dtype=torch.int64, device="cuda")
    pa.pa_reshape_and_cache(d.layout, d.k_cache, d.v_cache, d.v_new, d.k_new, sm)
    torch.cuda.synchronize()
    assert np.array_equal(dv.bits_of(d.k_cache), before)


@pytest.mark.parametrize("d_head,cache", [(64, "bf16"), (128, "bf16"), (128, "fp8"), (64, "fp8")])
def test_gather_bit_exact(d_head, cache):
    _announce(f"debug gather d={d_head} {cache}")
    w = wl.make_workload(name="t", seq_lens=[1, 16, 17, 100, 513], q_lens=[1] * 5,
                         num_q_heads=4, num_kv_heads=2, head_dim=d_head, seed=22,
                         cache_dtype=cache, writes_new_kv=False, pool_blocks=60)
    d = dv.to_device(w)
    cu = np.zeros(w.num_reqs + 1, np.int32)
    cu[1:] = np.cumsum(w.seq_lens)
    tot = int(cu[-1])
    dt = torch.uint8 if cache == "fp8" else torch.bfloat16
    ko = torch.empty((tot, 2, d_head), dtype=dt, device="cuda")
    vo = torch.empty_like(ko)
    pa.pa_debug_gather_kv(d.layout, ko, vo, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                          torch.from_numpy(cu).cuda(), d.max_seq_len)
    torch.cuda.synchronize()
    conv = (lambda t: t.cpu().numpy()) if cache == "fp8" else dv.bits_of
    gk, gv = conv(ko), conv(vo)
    for r in range(w.num_reqs):
        n = int(w.seq_lens[r])
        assert np.array_equal(gk[cu[r]:cu[r + 1]], oracle.gather_kv(w.k_pool, w.block_table[r], n, 16))
        assert np.array_equal(gv[cu[r]:cu[r + 1]], oracle.gather_kv(w.v_pool, w.block_table[r], n, 16))


@pytest.mark.parametrize("cfg,sd", [(1, None), (2, None), (4, 8)])
def test_fused_slot_mapping_and_scatter(cfg, sd):
    """pa_reshape_and_cache_varlen == slot mapping + scatter, bit for bit."""
    _announce(f"fused write, config {cfg} scale_down {sd}")
    w = wl.config_workload(cfg, scale_down=sd)
    d = dv.to_device(w)
    sm = torch.full((w.num_tokens,), -7, dtype=torch.int64, device="cuda")
    dv.write_new_kv_fused(d, sm)
    torch.cuda.synchronize()
    ref_sm = oracle.slot_mapping(w.block_table, w.query_start_loc, w.seq_lens, 16)
    assert np.array_equal(sm.cpu().numpy(), ref_sm)
    kp, vp = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.k_new, w.v_new, ref_sm, 16)
    assert np.array_equal(dv.bits_of(d.k_cache), kp)
    assert np.array_equal(dv.bits_of(d.v_cache), vp)


def test_fused_write_ragged_with_empty_requests():
    _announce("fused write, ragged with q_len 0 requests")
    w = wl.make_workload(name="t", seq_lens=[5, 16, 0, 17, 40, 300, 33, 1],
                         q_lens=[1, 16, 0, 3, 0, 40, 2, 1], num_q_heads=8, num_kv_heads=4,
                         head_dim=64, seed=23, pool_blocks=60)
    d = dv.to_device(w)
    dv.write_new_kv_fused(d, None)
    torch.cuda.synchronize()
    ref_sm = oracle.slot_mapping(w.block_table, w.query_start_loc, w.seq_lens, 16)
    kp, vp = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.k_new, w.v_new, ref_sm, 16)
    assert np.array_equal(dv.bits_of(d.k_cache), kp)
    assert np.array_equal(dv.bits_of(d.v_cache), vp)


@pytest.mark.parametrize("scale", [1.0, 0.0371, 2.0 ** -8, 3.0])
def test_fp8_quantising_scatter_all_bf16_inputs(scale):
    """All 65,536 bf16 bit patterns (NaN, inf, subnormals, +-0 included) as K
    and, reversed, as V; written to an fp8 cache through a shuffled slot
    mapping, by both write entry points: codes bit-exact vs the oracle."""
    _announce(f"fp8 quantising write, all bf16 inputs, scale {scale}")
    T, Hkv, D = 512, 1, 128
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(T, Hkv, D)
    vbits = np.ascontiguousarray(bits[::-1])
    NB = 40
    rng = np.random.default_rng(5)
    slots = rng.permutation(NB * 16)[:T].astype(np.int64)
    lay = pa.make_layout(NB, Hkv, D, pa.PA_CACHE_FP8_E4M3)
    ks = torch.tensor([scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([scale * 0.5], dtype=torch.float32, device="cuda")
    key, value = dv.bf16_tensor(bits, "cuda"), dv.bf16_tensor(vbits, "cuda")
    fill = np.full((NB, Hkv, 16, D), 0x5A, dtype=np.uint8)
    kp_ref, vp_ref = oracle.reshape_and_cache(fill, fill, bits, vbits, slots, 16,
                                              cache_dtype="fp8", k_scale=np.float32(scale),
                                              v_scale=np.float32(scale * 0.5))
    kc = torch.from_numpy(fill.copy()).cuda()
    vc = torch.from_numpy(fill.copy()).cuda()
    pa.pa_reshape_and_cache(lay, kc, vc, key, value, torch.from_numpy(slots).cuda(), ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), kp_ref)
    assert np.array_equal(vc.cpu().numpy(), vp_ref)
    # the fused entry point: one request of 512 tokens over a shuffled table
    bt = rng.permutation(NB)[None, :].astype(np.int32)
    qsl = np.array([0, T], np.int32)
    sl = np.array([T], np.int32)
    sm_ref = oracle.slot_mapping(bt, qsl, sl, 16)
    kp2, vp2 = oracle.reshape_and_cache(fill, fill, bits, vbits, sm_ref, 16, cache_dtype="fp8",
                                        k_scale=np.float32(scale),
                                        v_scale=np.float32(scale * 0.5))
    kc2 = torch.from_numpy(fill.copy()).cuda()
    vc2 = torch.from_numpy(fill.copy()).cuda()
    pa.pa_reshape_and_cache_varlen(lay, kc2, vc2, key, value, torch.from_numpy(bt).cuda(),
                                   torch.from_numpy(qsl).cuda(), torch.from_numpy(sl).cuda(),
                                   None, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(kc2.cpu().numpy(), kp2)
    assert np.array_equal(vc2.cpu().numpy(), vp2)


def test_fp8_write_config4_scaled_bit_exact():
    """The mixed-batch write at 1/8 scale into an fp8 cache (2,176/8 tokens,
    8 KV heads): slot mapping and codes bit-exact."""
    _announce("fp8 fused write, mixed batch / 8")
    w0 = wl.config_workload(4, scale_down=8)
    w = wl.make_workload(name="t", seq_lens=w0.seq_lens, q_lens=w0.q_lens, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, seed=73, cache_dtype="fp8")
    d = dv.to_device(w)
    sm = torch.full((w.num_tokens,), -7, dtype=torch.int64, device="cuda")
    dv.write_new_kv_fused(d, sm)
    torch.cuda.synchronize()
    ref_sm = oracle.slot_mapping(w.block_table, w.query_start_loc, w.seq_lens, 16)
    assert np.array_equal(sm.cpu().numpy(), ref_sm)
    kp, vp = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.k_new, w.v_new, ref_sm, 16,
                                      cache_dtype="fp8", k_scale=w.k_scale, v_scale=w.v_scale)
    assert np.array_equal(d.k_cache.cpu().numpy(), kp)
    assert np.array_equal(d.v_cache.cpu().numpy(), vp)


@pytest.mark.parametrize("pos", ["first", "middle", "last"])
def test_measure_read_stream_reads_every_chunk(pos):
    """pa_measure_read_stream: a zero buffer leaves the sink alone; a single
    0xffffffff word anywhere (first chunk, inside the unrolled part, the
    last chunk of the tail loop) makes its thread's XOR 0xffffffff and the
    sink gets it -- every 16-byte chunk is read."""
    import paged_kv_cache_77_amd as pa
    print(f"\n[case] read stream, marker {pos}", flush=True)
    n = (64 << 20) + 48                      # not a multiple of the grid stride
    buf = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    pa.pa_measure_read_stream(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == 0
    idx = {"first": 0, "middle": (n // 4) // 2 + 5, "last": n // 4 - 1}[pos]
    buf[idx] = -1
    pa.pa_measure_read_stream(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == -1
