"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case swaps one oracle helper for a plausibly wrong version and runs the
pins that guard it; the pin must fail.  This shows the pins constrain the
oracle rather than merely agree with it.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import pa_oracle as po
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    with pytest.raises((AssertionError, IndexError, ValueError)):
        fn(*args)


def test_swapped_block_and_offset_is_caught(monkeypatch, golden):
    def wrong(bt_row, t, B):
        t = np.asarray(t, np.int64)
        return np.asarray(bt_row, np.int64)[t % B % len(bt_row)], t // B
    monkeypatch.setattr(po, "logical_to_physical", wrong)
    _fails(pins.test_address_examples, golden)


def test_off_by_one_positions_are_caught(monkeypatch, golden):
    monkeypatch.setattr(po, "token_positions",
                        lambda n, q: np.arange(n - q + 1, n + 1, dtype=np.int64))
    _fails(pins.test_varlen_examples, golden)
    _fails(pins.test_address_examples, golden)


def test_interleaved_gqa_map_is_caught(monkeypatch):
    monkeypatch.setattr(po, "kv_head_of", lambda h, G: h % 3)
    _fails(pins.test_decode_gqa_head_map)


def test_missing_score_scale_is_caught(monkeypatch):
    real = po.attend
    monkeypatch.setattr(po, "attend", lambda q, K, V, s, *b: real(q, K, V, 1.0, *b))
    _fails(pins.test_decode_matches_sdpa_contiguous, 4, 2, 64)


def test_merge_without_rescale_is_caught(monkeypatch):
    def wrong(m, l, O, num_parts):
        R, H = m.shape[:2]
        out = np.zeros((R, H, O.shape[-1]))
        for r in range(R):
            n = int(num_parts[r])
            for h in range(H):
                w = l[r, h, :n]                    # forgot e^{m_j - m}
                out[r, h] = (w[:, None] * O[r, h, :n]).sum(0) / w.sum()
        return out
    monkeypatch.setattr(po, "merge_partitions", wrong)
    _fails(pins.test_merge_equals_decode_and_is_order_free)


def test_online_softmax_without_accumulator_rescale_is_caught(monkeypatch):
    def wrong(q, K, V, scale, cuts):
        sc = float(np.float32(scale))
        m, l, A = -np.inf, 0.0, np.zeros(V.shape[1])
        bounds = [0] + list(cuts) + [K.shape[0]]
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            S = (K[lo:hi] @ q) * sc
            mn = max(m, S.max())
            a = math.exp(m - mn) if m != -np.inf else 0.0
            e = np.exp(S - mn)
            l = a * l + e.sum()
            A = A + e @ V[lo:hi]                   # forgot to rescale A
            m = mn
        return A / l
    monkeypatch.setattr(po, "online_softmax_tiles", wrong)
    _fails(pins.test_online_softmax_two_element_hand_case)


def test_fnuz_fp8_bias_is_caught(monkeypatch):
    def wrong(codes):
        c = np.asarray(codes).astype(np.int64)
        s = np.where(c & 0x80, -1.0, 1.0)
        e, m = (c >> 3) & 0xF, c & 7
        return np.where(e == 0, s * np.ldexp(m / 8.0, -7), s * np.ldexp(1 + m / 8.0, e - 8))
    monkeypatch.setattr(po, "fp8_e4m3fn_to_f64", wrong)
    _fails(pins.test_fp8_closed_form_all_codes)


def test_top_left_causal_alignment_is_caught(monkeypatch):
    monkeypatch.setattr(po, "token_positions",
                        lambda n, q: np.arange(0, q, dtype=np.int64))
    _fails(pins.test_prefill_chunks_compose)


def test_gather_with_wrong_token_order_is_caught(monkeypatch):
    def wrong(pool, bt_row, n, B):
        t = np.arange(n, dtype=np.int64)
        phys, off = po.logical_to_physical(bt_row, t, B)
        return pool[phys, :, (B - 1 - off), :]     # reversed inside each block
    monkeypatch.setattr(po, "gather_kv", wrong)
    _fails(pins.test_decode_matches_sdpa_contiguous, 4, 2, 64)
    _fails(pins.test_scatter_then_gather_roundtrip)


def test_fp8_ties_away_from_zero_is_caught(monkeypatch):
    real = po.fp8_e4m3fn_encode

    def wrong(y):
        y = np.asarray(y, np.float64)
        mags = po.fp8_e4m3fn_to_f64(np.arange(127))
        a = np.abs(y)
        hi = np.clip(np.searchsorted(mags, np.nan_to_num(a), side="left"), 0, 126)
        lo = np.clip(hi - 1, 0, 126)
        code = np.where(mags[hi] - a <= a - mags[lo], hi, lo)     # ties go up
        code = np.where(a >= 448, 126, code)
        return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)
    monkeypatch.setattr(po, "fp8_e4m3fn_encode", wrong)
    _fails(pins.test_fp8_encode_ties_saturation_and_specials)
    _fails(pins.test_fp8_encode_matches_torch_cast_on_all_bf16_inputs)
    assert real is not wrong


def test_fp8_without_saturation_is_caught(monkeypatch):
    real = po.fp8_e4m3fn_encode

    def wrong(y):
        y = np.asarray(y, np.float64)
        return np.where(np.abs(y) > 448, np.uint8(0x7F), real(y)).astype(np.uint8)
    monkeypatch.setattr(po, "fp8_e4m3fn_encode", wrong)
    _fails(pins.test_fp8_encode_ties_saturation_and_specials)


def test_alibi_sign_flip_is_caught(monkeypatch):
    real = po.alibi_bias
    monkeypatch.setattr(po, "alibi_bias", lambda s, k, q: -real(s, k, q))
    _fails(pins.test_alibi_decode_closed_form)
    _fails(pins.test_alibi_prefill_closed_form_per_query_position)


def test_alibi_key_offset_instead_of_position_is_caught(monkeypatch):
    real = po.alibi_bias
    monkeypatch.setattr(po, "alibi_bias",
                        lambda s, k, q: real(s, np.asarray(k) % 16, np.asarray(q) % 16))
    _fails(pins.test_alibi_decode_closed_form)


def test_alibi_slope_of_kv_head_is_caught(monkeypatch):
    real = po._slopes

    def wrong(w, a):
        s = real(w, a)
        return None if s is None else s[(np.arange(len(s)) // w.group_size) * w.group_size]
    monkeypatch.setattr(po, "_slopes", wrong)
    _fails(pins.test_alibi_decode_closed_form)


def _pins_blocks():
    from tests import test_oracle_blocks as tb
    return tb


def test_unhashed_blocks_queued_at_tail_is_caught(monkeypatch, golden):
    from oracle import block_pool as bpm

    def wrong(self, blocks):
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0 and b != 0:
                self.queue.append(b)              # partial blocks kept like cached ones
    monkeypatch.setattr(bpm.BlockPoolModel, "free_blocks", wrong)
    _fails(_pins_blocks().test_lru_model_hit_tokens, golden)


def test_no_last_token_rule_is_caught(monkeypatch):
    from oracle import block_pool as bpm
    real = bpm.BlockPoolModel.allocate_prompt

    def wrong(self, hashes, num_tokens, block_size):
        return real(self, hashes, num_tokens + 1, block_size) if num_tokens % block_size == 0 \
            else real(self, hashes, num_tokens, block_size)
    monkeypatch.setattr(bpm.BlockPoolModel, "allocate_prompt", wrong)
    _fails(_pins_blocks().test_last_token_is_always_computed)


def test_touch_leaving_block_queued_is_caught(monkeypatch):
    from oracle import block_pool as bpm

    def wrong(self, blocks):
        for b in blocks:
            self.ref[b] += 1                      # forgot to take it off the queue
    monkeypatch.setattr(bpm.BlockPoolModel, "touch", wrong)
    _fails(_pins_blocks().test_pool_conservation_under_random_use)


def test_hash_without_parent_is_caught(monkeypatch):
    from oracle import block_pool as bpm
    real = bpm.block_hash
    monkeypatch.setattr(bpm, "block_hash", lambda parent, tokens, extra=0:
                        real(bpm.NONE_HASH, tokens, extra))
    _fails(_pins_blocks().test_block_hash_chain_property)


def test_fp8_dequant_dividing_by_the_scale_is_caught(monkeypatch):
    def wrong(pool, cache_dtype, scale=1.0):
        if cache_dtype == "fp8":
            return po.fp8_e4m3fn_to_f64(pool) / np.float64(np.float32(scale))
        return po.bf16_bits_to_f64(pool)
    monkeypatch.setattr(po, "cache_values", wrong)
    _fails(pins.test_fp8_dequant_multiplies_by_its_scale)
    _fails(pins.test_decode_fp8_each_scale_applies_to_its_tensor)
    _fails(pins.test_prefill_fp8_each_scale_applies_to_its_tensor)


def test_fp8_write_of_v_with_k_scale_is_caught(monkeypatch):
    real = po.reshape_and_cache

    def wrong(k_pool, v_pool, key, value, slots, block_size, cache_dtype="bf16",
              k_scale=1.0, v_scale=1.0):
        return real(k_pool, v_pool, key, value, slots, block_size, cache_dtype,
                    k_scale, k_scale)
    monkeypatch.setattr(po, "reshape_and_cache", wrong)
    _fails(pins.test_fp8_scatter_writes_codes_of_the_quotient)


def test_fp8_read_of_v_with_k_scale_is_caught(monkeypatch):
    def wrong(w, r, k_pool=None, v_pool=None):
        kp = w.k_pool if k_pool is None else k_pool
        vp = w.v_pool if v_pool is None else v_pool
        n = int(w.seq_lens[r])
        K = po.cache_values(po.gather_kv(kp, w.block_table[r], n, w.block_size),
                            w.cache_dtype, w.k_scale)
        V = po.cache_values(po.gather_kv(vp, w.block_table[r], n, w.block_size),
                            w.cache_dtype, w.k_scale)
        return K, V
    monkeypatch.setattr(po, "_request_kv", wrong)
    _fails(pins.test_decode_fp8_each_scale_applies_to_its_tensor)
    _fails(pins.test_prefill_fp8_each_scale_applies_to_its_tensor)
