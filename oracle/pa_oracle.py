"""CPU fp64 oracle for paged attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
library's product path never does, and this module shares no code with it.

Plain, slow, obviously correct definitions, written from these pages:
  [P1] "vLLM 深度解析（二）：PagedAttention 核心机制"
  [P2] "第11章 分块预填充与混合批处理"
  [P3] "vllm 深度解析：一切从 PagedAttention 谈起"
  [P4] "LLM 推理基础与 vLLM 内部机制：KV 缓存、PagedAttention、调度器"

Every floating-point step is fp64.  Cache values are widened exactly from
their stored bits (bf16) or decoded from their codes (fp8 e4m3fn, times the
per-tensor fp32 scale).  ``scale`` is the fp32 value the GPU receives, widened.

The method computes exact attention (P1 §2.1 table: both the direct form and
the IO-aware tiled form give exact attention), so attention here is the
direct definition softmax(Q Kᵀ · scale) V over K/V gathered in logical order
through the block table.  Parity pins for every function live in
tests/test_oracle_pins.py; none is "parity unpinned".

Readings of points the pages leave open:
  * seq_lens[r] includes the tokens written in this step (P2 §11.6: the decode
    request's K/V length is its history plus the new token), so the newest
    token of a request sits at position seq_len - 1 and attends to itself;
  * in chunked prefill, query i of a request with q_len queries sits at
    position seq_len - q_len + i and sees keys 0..that position (causal,
    aligned at the bottom right);
  * query head h reads K/V head h // G, G = num_q_heads / num_kv_heads;
  * no epsilon in the softmax denominator (the result is exact, P1 §2.2);
  * a request with seq_len == 0 produces an all-zero output row;
  * a negative slot_mapping entry means "skip this token" (padding);
  * writing into an FP8 cache stores the E4M3FN code nearest to the fp32
    quotient x / scale (ties to the even code, saturating at ±448, NaN kept
    as NaN) -- the inverse of the read-side "code value times scale";
  * the ALiBi term of P1 §3.2.4, slope_h · (t − seq_len + 1) for the decode
    query, is slope_h · (t − p) for a query at position p in prefill (the
    same relative distance; the decode query sits at p = seq_len − 1).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

# ---------------------------------------------------------------------------
# value decoding


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64, exactly (bf16 is the top half of an fp32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN code -> fp64 by its closed form.

    sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (2^-6 · m/8); S.1111.111 is NaN; there is no infinity.  The
    pages only say FP8 K/V are loaded quantised and converted with a scale
    (P1 §3.2.1 / §3.2.4) and that FP8 storage takes one byte (P4 §2).
    """
    # the closed form is evaluated once for each of the 256 codes; a code's
    # value is then looked up (the same numbers, without re-deriving them for
    # every element of a large cache)
    c = np.arange(256, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    sub = sign * np.ldexp(m / 8.0, -6)
    value_of_code = np.where((e == 15) & (m == 7), np.nan, np.where(e == 0, sub, normal))
    return value_of_code[np.asarray(codes).astype(np.uint8)]


def cache_values(pool: np.ndarray, cache_dtype: str, scale: float = 1.0) -> np.ndarray:
    """Stored cache elements -> fp64 values (fp8: code value times its scale)."""
    if cache_dtype == "bf16":
        return bf16_bits_to_f64(pool)
    if cache_dtype == "fp8":
        return fp8_e4m3fn_to_f64(pool) * np.float64(np.float32(scale))
    raise ValueError(cache_dtype)


def fp8_e4m3fn_encode(y) -> np.ndarray:
    """fp32 values -> OCP FP8 E4M3FN codes (uint8).

    The code whose value (fp8_e4m3fn_to_f64) is nearest to y; at a tie the
    code with the even mantissa (round to nearest even).  |y| >= 448, the
    largest finite E4M3FN value, saturates to ±448 (the format has no
    infinity); NaN becomes S.1111.111; the sign of y is kept, zeros
    included.  Written as a search over the 127 non-negative finite values.
    """
    y = np.asarray(y, dtype=np.float64)
    mags = fp8_e4m3fn_to_f64(np.arange(127))          # codes 0x00..0x7E, increasing
    a = np.abs(y)
    hi = np.clip(np.searchsorted(mags, np.nan_to_num(a, nan=0.0), side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a >= 448.0, 126, code)
    code = np.where(np.isnan(y), 127, code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_fp8(bits: np.ndarray, scale: float) -> np.ndarray:
    """bf16 bit patterns -> E4M3FN codes for a cache whose per-tensor scale is
    ``scale`` (reading: the inverse of the read side's code · scale).  The
    code is decided from the fp32 quotient x / scale, correctly rounded,
    which is the precision the writing kernel works in."""
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        x = bf16_bits_to_f64(bits).astype(np.float32)     # exact
        return fp8_e4m3fn_encode(x / np.float32(scale))


def alibi_bias(slope: float, key_pos: np.ndarray, query_pos) -> np.ndarray:
    """ALiBi term added to the scaled score (P1 §3.2.4: slope times
    (token index − seq_len + 1) for the decode query, i.e. the signed
    distance from the query's own position).  ``slope`` is the fp32 value
    the GPU receives, widened."""
    return float(np.float32(slope)) * (np.asarray(key_pos, np.float64) -
                                       np.asarray(query_pos, np.float64))


def _slopes(w, alibi_slopes):
    s = getattr(w, "alibi_slopes", None) if alibi_slopes is None else alibi_slopes
    return None if s is None else np.asarray(s, dtype=np.float32)


# ---------------------------------------------------------------------------
# addressing (P1 §3.1; P3 BlockTable figure "position=18")


def logical_to_physical(bt_row: np.ndarray, t, block_size: int):
    """Token position t -> (physical block, offset in block).

    logical_block = t // B, offset = t mod B, physical_block =
    block_table[request][logical_block]  (P1 §3.1 equations).
    """
    t = np.asarray(t, dtype=np.int64)
    logical_block = t // block_size
    offset = t % block_size
    physical = np.asarray(bt_row, dtype=np.int64)[logical_block]
    return physical, offset


def token_positions(seq_len: int, q_len: int) -> np.ndarray:
    """Positions of the q_len tokens a request computes in this step.

    They are the last q_len of its seq_len visible tokens (P2 §11.6 example:
    query_start_loc [0,1024,1025,1153], seq_lens [2048,2049,128] put the
    chunk at 1024..2047, the decode token at 2048 and the short prompt at
    0..127).
    """
    return np.arange(seq_len - q_len, seq_len, dtype=np.int64)


def slot_mapping(block_table: np.ndarray, query_start_loc: np.ndarray,
                 seq_lens: np.ndarray, block_size: int) -> np.ndarray:
    """slot = physical_block * B + offset for every token of the flattened
    batch (P1 §3.1, simplified single-group slot formula; P3
    ``_compute_slot_mappings_kernel``).  int64, one entry per token."""
    T = int(query_start_loc[-1])
    out = np.empty(T, dtype=np.int64)
    for r in range(len(seq_lens)):
        lo, hi = int(query_start_loc[r]), int(query_start_loc[r + 1])
        pos = token_positions(int(seq_lens[r]), hi - lo)
        phys, off = logical_to_physical(block_table[r], pos, block_size)
        out[lo:hi] = phys * block_size + off
    return out


def reshape_and_cache(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray,
                      value: np.ndarray, slots: np.ndarray, block_size: int,
                      cache_dtype: str = "bf16", k_scale: float = 1.0,
                      v_scale: float = 1.0):
    """Write each new token's K/V rows to its slot, returning new pools.  The
    pool layout is [block][kv_head][offset][dim], so slot s lands at block
    s // B, offset s % B for every KV head (P3 ``reshape_and_cache`` writes
    new K/V through slot_mapping; P1 §3.1 table: slot_mapping writes,
    block_table reads).  bf16 caches get a bit copy; FP8 caches get the
    codes of quantize_fp8 with the pool's scale."""
    kp = k_pool.copy()
    vp = v_pool.copy()
    for j, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        blk, off = s // block_size, s % block_size
        if cache_dtype == "fp8":
            kp[blk, :, off, :] = quantize_fp8(key[j], k_scale)
            vp[blk, :, off, :] = quantize_fp8(value[j], v_scale)
        else:
            kp[blk, :, off, :] = key[j]
            vp[blk, :, off, :] = value[j]
    return kp, vp


def gather_kv(pool: np.ndarray, bt_row: np.ndarray, seq_len: int,
              block_size: int) -> np.ndarray:
    """Logical K (or V) of one request: row t is the cache row at
    (block_table[t // B], t mod B) for every KV head.  [seq_len, Hkv, d]
    (P1 §3.1; P1 §3.2.3: one block-table row per request)."""
    t = np.arange(seq_len, dtype=np.int64)
    phys, off = logical_to_physical(bt_row, t, block_size)
    return pool[phys, :, off, :]


# ---------------------------------------------------------------------------
# attention


def kv_head_of(h: int, group_size: int) -> int:
    """Query head h reads KV head h // G (contiguous GQA groups, P4 §2)."""
    return h // group_size


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           bias: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(q Kᵀ · scale + bias) V for query rows q [n, d] over K, V [t, d]
    (P1 §2.1: S = QKᵀ, P = softmax(S), O = PV; bias: the ALiBi term of
    P1 §3.2.4, added after scaling).  fp64.  The row max is subtracted before
    exponentiating, which leaves softmax unchanged."""
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]))
    s = (q @ K.T) * float(np.float32(scale))
    if bias is not None:
        s = s + bias
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return (p @ V) / p.sum(axis=-1, keepdims=True)


def _request_kv(w, r: int, k_pool=None, v_pool=None):
    kp = w.k_pool if k_pool is None else k_pool
    vp = w.v_pool if v_pool is None else v_pool
    n = int(w.seq_lens[r])
    K = cache_values(gather_kv(kp, w.block_table[r], n, w.block_size), w.cache_dtype, w.k_scale)
    V = cache_values(gather_kv(vp, w.block_table[r], n, w.block_size), w.cache_dtype, w.v_scale)
    return K, V


def decode(w, q: Optional[np.ndarray] = None, k_pool=None, v_pool=None,
           requests: Optional[Iterable[int]] = None, alibi_slopes=None) -> np.ndarray:
    """Single-query decode for every request: out[r, h] = attention of query
    row r, head h over all seq_len[r] tokens of KV head h // G.
    [R, Hq, d] fp64 (rows not in ``requests`` stay NaN).

    q defaults to the workload's query rows (one per request); ALiBi slopes
    (one per query head) default to the workload's, if any."""
    qb = w.q if q is None else q
    R, H, d = w.num_reqs, w.num_q_heads, w.head_dim
    G = w.group_size
    slopes = _slopes(w, alibi_slopes)
    out = np.full((R, H, d), np.nan)
    for r in (range(R) if requests is None else requests):
        K, V = _request_kv(w, r, k_pool, v_pool)
        qr = bf16_bits_to_f64(qb[r])
        n = int(w.seq_lens[r])
        for h in range(H):
            g = kv_head_of(h, G)
            bias = None if slopes is None else alibi_bias(slopes[h], np.arange(n), n - 1)
            out[r, h] = attend(qr[h][None, :], K[:, g, :], V[:, g, :], w.scale, bias)[0]
    return out


def decode_partitions(w, partition_size: int, q: Optional[np.ndarray] = None,
                      k_pool=None, v_pool=None, requests=None, alibi_slopes=None):
    """Per-partition softmax statistics of decode (P1 §3.2.7 and §3.3: V2
    splits the context into fixed partitions and keeps, per partition, the
    max logit, the exp-sum and the partition's normalised output).

    Partition p of request r covers tokens [p·P, min((p+1)·P, seq_len)).
    Returns m, l: [R, Hq, Pmax] and O: [R, Hq, Pmax, d], NaN where unused;
    m is in natural-log units of the scaled scores."""
    qb = w.q if q is None else q
    R, H, d, G = w.num_reqs, w.num_q_heads, w.head_dim, w.group_size
    P = int(partition_size)
    pmax = max(1, max((int(s) + P - 1) // P for s in w.seq_lens))
    m = np.full((R, H, pmax), np.nan)
    l = np.full((R, H, pmax), np.nan)
    O = np.full((R, H, pmax, d), np.nan)
    sc = float(np.float32(w.scale))
    slopes = _slopes(w, alibi_slopes)
    for r in (range(R) if requests is None else requests):
        K, V = _request_kv(w, r, k_pool, v_pool)
        qr = bf16_bits_to_f64(qb[r])
        n = int(w.seq_lens[r])
        for p in range((n + P - 1) // P):
            lo, hi = p * P, min((p + 1) * P, n)
            for h in range(H):
                g = kv_head_of(h, G)
                s = (K[lo:hi, g, :] @ qr[h]) * sc
                if slopes is not None:
                    s = s + alibi_bias(slopes[h], np.arange(lo, hi), n - 1)
                mp = s.max()
                e = np.exp(s - mp)
                m[r, h, p] = mp
                l[r, h, p] = e.sum()
                O[r, h, p] = (e @ V[lo:hi, g, :]) / e.sum()
    return m, l, O


def merge_partitions(m: np.ndarray, l: np.ndarray, O: np.ndarray,
                     num_parts: np.ndarray) -> np.ndarray:
    """Cross-partition merge (P1 §3.2.9 equations):
        m = max_j m_j,  L = Σ_j l_j e^{m_j − m},  O = Σ_j O_j l_j e^{m_j − m} / L.
    m, l: [R, H, Pmax]; O: [R, H, Pmax, d]; num_parts: [R]."""
    R, H = m.shape[:2]
    out = np.zeros((R, H, O.shape[-1]))
    for r in range(R):
        n = int(num_parts[r])
        if n == 0:
            continue
        for h in range(H):
            mj, lj, Oj = m[r, h, :n], l[r, h, :n], O[r, h, :n]
            M = mj.max()
            wgt = lj * np.exp(mj - M)
            out[r, h] = (wgt[:, None] * Oj).sum(axis=0) / wgt.sum()
    return out


def online_softmax_tiles(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                         tile_bounds: Iterable[int]) -> np.ndarray:
    """FlashAttention's running (m, l, A) over K/V tiles (P1 §2.2):
        m' = max(m, max S_j)
        l' = e^{m−m'} l + Σ e^{S_j − m'}
        A' = e^{m−m'} A + Σ e^{S_j − m'} V_j,   O = A'/l'.
    q [d]; K, V [t, d]; tile_bounds: increasing cut points inside (0, t)."""
    sc = float(np.float32(scale))
    m, l, A = -np.inf, 0.0, np.zeros(V.shape[1])
    cuts = [0] + [int(c) for c in tile_bounds] + [K.shape[0]]
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        if hi <= lo:
            continue
        S = (K[lo:hi] @ q) * sc
        m_new = max(m, S.max())
        a = math.exp(m - m_new) if m != -np.inf else 0.0
        e = np.exp(S - m_new)
        l = a * l + e.sum()
        A = a * A + e @ V[lo:hi]
        m = m_new
    return A / l


def prefill_varlen(w, rows: Optional[Iterable[tuple]] = None, k_pool=None,
                   v_pool=None, alibi_slopes=None) -> np.ndarray:
    """Varlen (chunked) prefill over the paged cache (P2 §11.6: the varlen
    batch is cut by query_start_loc; seq_lens give each request's visible
    K/V length; block_table addresses it).  Query i of request r at
    position p = seq_len − q_len + i attends keys 0..p (causal).

    Returns out [T, Hq, d] fp64.  ``rows``: optional iterable of (token, head)
    pairs to compute (others stay NaN) for sampled checks at full size."""
    T, H, d, G = w.num_tokens, w.num_q_heads, w.head_dim, w.group_size
    slopes = _slopes(w, alibi_slopes)
    out = np.full((T, H, d), np.nan)
    want = None
    if rows is not None:
        want = {}
        for (t, h) in rows:
            want.setdefault(int(t), set()).add(int(h))
    qsl = w.query_start_loc
    for r in range(w.num_reqs):
        lo, hi = int(qsl[r]), int(qsl[r + 1])
        if hi == lo:
            continue
        toks = range(lo, hi) if want is None else [t for t in range(lo, hi) if t in want]
        if not toks:
            continue
        K, V = _request_kv(w, r, k_pool, v_pool)
        n = int(w.seq_lens[r])
        pos = token_positions(n, hi - lo)
        qf = bf16_bits_to_f64(w.q[list(toks)])          # [k, H, d]
        for h in range(H):
            g = kv_head_of(h, G)
            sel = [i for i, t in enumerate(toks) if want is None or h in want[t]]
            if not sel:
                continue
            qs = qf[sel, h, :]
            s = (qs @ K[:, g, :].T) * float(np.float32(w.scale))  # [k, n]
            p_abs = pos[[toks[i] - lo for i in sel]]
            if slopes is not None:
                s = s + alibi_bias(slopes[h], np.arange(n)[None, :], p_abs[:, None])
            visible = np.arange(n)[None, :] <= p_abs[:, None]
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=-1, keepdims=True)
            e = np.exp(s)
            o = (e @ V[:, g, :]) / e.sum(axis=-1, keepdims=True)
            for k, i in enumerate(sel):
                out[toks[i], h] = o[k]
    return out


# ---------------------------------------------------------------------------
# sizing (P1 §1 equation; P4 §2 table)


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    """KV bytes per token = 2 (K and V) × layers × KV heads × head_dim × bytes."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Physical blocks needed to hold num_tokens tokens (last block partial)."""
    return -(-num_tokens // block_size)


# ---------------------------------------------------------------------------
# output rounding, for comparisons


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (via fp32), round to nearest even."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float32) \
        .to(torch.bfloat16).to(torch.float64).numpy()
