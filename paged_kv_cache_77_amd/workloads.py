"""Seeded synthetic inputs for paged attention over a block-table KV cache.

This module only draws random numbers and lays out metadata the way an
allocator and a scheduler would hand it to the attention kernels: context
lengths, per-step query counts, a random permutation of physical blocks, the
cache contents of each physical block, queries and the new tokens' K/V.  It
computes nothing that the attention method computes (no slot mapping, no
scatter, no gather, no softmax); both the CPU oracle and the HIP path consume
what it returns.

Conventions (the pages leave them open):
  * cache pools are ``[num_blocks][num_kv_heads][block_size][head_dim]``,
    bf16 stored as uint16 bit patterns, fp8 (OCP e4m3fn) as uint8 codes;
  * ``seq_lens[r]`` counts every K/V token request ``r`` can see in this step,
    including the tokens written in this step (vLLM chunked-prefill page,
    varlen metadata section: the decode request's K/V length is history plus
    the new token);
  * when ``writes_new_kv`` is set, the last ``q_lens[r]`` tokens of each
    request are *not* in the pool yet: their slots hold poison and the new
    K/V arrive in ``k_new``/``v_new``; otherwise the pool already holds all
    ``seq_lens[r]`` tokens;
  * unused pool slots hold NaN (bf16 0x7FC0, fp8 0x7F) when ``poison`` is set,
    zero otherwise; unused block-table entries hold INT32_MIN.

Random draw order for a workload (one PCG64 stream seeded with ``seed``):
  1. context / query lengths;
  2. the block permutation (its own stream when ``perm_seed`` is given);
  3. Q;
  4. K then V history per block, in logical order (shared prefix group first,
     then each request's private blocks), so the data do not depend on the
     permutation;
  5. new-token K then V;
  6. fp8 scales and codes (no further draws).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 16
BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
TABLE_PAD = np.int32(np.iinfo(np.int32).min)
FP8_E4M3_MAX = 448.0


@dataclasses.dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    cache_dtype: str                 # "bf16" | "fp8"
    seq_lens: np.ndarray             # int32 [R]
    q_lens: np.ndarray               # int32 [R]
    query_start_loc: np.ndarray      # int32 [R+1]
    block_table: np.ndarray          # int32 [R, W]
    num_blocks: int
    k_pool: np.ndarray               # uint16|uint8 [NB, Hkv, B, d]
    v_pool: np.ndarray
    q: np.ndarray                    # uint16 [T, Hq, d]
    k_new: Optional[np.ndarray]      # uint16 [T, Hkv, d] or None
    v_new: Optional[np.ndarray]
    scale: np.float32
    k_scale: np.float32
    v_scale: np.float32
    writes_new_kv: bool
    seed: int
    partition_size: int = 512
    alibi_slopes: Optional[np.ndarray] = None   # fp32 [Hq] or None

    @property
    def num_reqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])

    def digest(self) -> dict:
        """SHA-256 of every input buffer (logged next to results)."""
        out = {}
        for name in ("seq_lens", "q_lens", "query_start_loc", "block_table",
                     "k_pool", "v_pool", "q", "k_new", "v_new", "alibi_slopes"):
            a = getattr(self, name)
            if a is None:
                continue
            out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
        return out


# ---------------------------------------------------------------------------
# rounding helpers (input construction only)

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_fp8_codes(x: np.ndarray, scale: np.float32) -> np.ndarray:
    """fp32 / scale -> OCP e4m3fn codes, round to nearest even (torch's CPU cast).

    ``scale`` is chosen so that |x / scale| <= 448 for every finite x, so the
    cast never overflows.
    """
    y = np.ascontiguousarray(x, dtype=np.float32) / np.float32(scale)
    t = torch.from_numpy(y).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


# ---------------------------------------------------------------------------
# generic generator

def make_workload(*, name: str, seq_lens: Sequence[int], q_lens: Sequence[int],
                  num_q_heads: int, num_kv_heads: int, head_dim: int,
                  cache_dtype: str = "bf16", writes_new_kv: bool = True,
                  shared_blocks: int = 0, share: Optional[Sequence[int]] = None,
                  k_boost: Optional[tuple] = None, pool_blocks: Optional[int] = None,
                  bt_extra_cols: int = 0, seed: int = 0,
                  perm_seed: Optional[int] = None, identity_perm: bool = False,
                  poison: bool = True, rng: Optional[np.random.Generator] = None,
                  partition_size: int = 512, zero_q: bool = False,
                  alibi: bool = False) -> Workload:
    """Build a workload from explicit lengths.

    shared_blocks / share: a prefix group of ``shared_blocks`` physical blocks
      whose data are drawn once; request r maps its first ``share[r]`` logical
      blocks onto the first ``share[r]`` blocks of the group (prefix caching's
      repeated physical ids).  Shared blocks must hold history only.
    k_boost: (period, factor): K rows at logical positions t with
      t % period == period - 1 are multiplied by ``factor`` (a power of two,
      exact in bf16).
    alibi: attach per-head ALiBi slopes, the geometric sequence
      2^(-8(h+1)/Hq) of the ALiBi paper (no draws).
    fp8 caches with new tokens: the per-tensor scales cover the history and
      the new tokens (amax / 448), so writes do not saturate.
    """
    B = BLOCK_SIZE
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    R = int(seq_lens.shape[0])
    assert q_lens.shape == (R,)
    assert num_q_heads % num_kv_heads == 0
    assert np.all(q_lens >= 0) and np.all(seq_lens >= q_lens)
    hist = seq_lens - q_lens if writes_new_kv else seq_lens.copy()
    share = np.zeros(R, np.int64) if share is None else np.asarray(share, np.int64)
    assert np.all(share <= shared_blocks)
    assert np.all(share * B <= hist), "shared blocks must hold history only"

    # -- 2. physical block allocation: a random permutation of the pool
    nblk = (seq_lens + B - 1) // B
    private = nblk - share
    used = shared_blocks + int(private.sum())
    NB = used if pool_blocks is None else int(pool_blocks)
    assert NB >= used
    if identity_perm:
        perm = np.arange(NB, dtype=np.int64)
    else:
        prng = rng if perm_seed is None else np.random.Generator(np.random.PCG64(perm_seed))
        perm = prng.permutation(NB).astype(np.int64)
    group_ids = perm[:shared_blocks]
    W = int(nblk.max()) + bt_extra_cols if R else 1
    W = max(W, 1)
    block_table = np.full((R, W), TABLE_PAD, dtype=np.int32)
    cursor = shared_blocks
    private_ids = []
    for r in range(R):
        ids = perm[cursor:cursor + private[r]]
        cursor += int(private[r])
        private_ids.append(ids)
        block_table[r, :share[r]] = group_ids[:share[r]]
        block_table[r, share[r]:nblk[r]] = ids

    # -- 3. queries
    T = int(q_lens.sum())
    H, Hkv, d = num_q_heads, num_kv_heads, head_dim
    if zero_q:
        q = np.zeros((T, H, d), dtype=np.uint16)
    else:
        q = to_bf16_bits(rng.standard_normal((T, H, d), dtype=np.float32))

    # -- 4. history K/V, block by block in logical order
    fp8 = cache_dtype == "fp8"
    store_dtype = np.float32 if fp8 else np.uint16
    fill = np.float32(np.nan) if fp8 else (BF16_NAN if poison else np.uint16(0))
    if fp8 and not poison:
        fill = np.float32(0.0)
    k_pool = np.full((NB, Hkv, B, d), fill, dtype=store_dtype)
    v_pool = np.full((NB, Hkv, B, d), fill, dtype=store_dtype)

    # scratch buffers reused across requests (large fresh allocations are slow)
    max_n = int(max([shared_blocks] + [int(x) for x in private])) if R else 0
    fbuf = np.empty((max(max_n, 1), Hkv, B, d), dtype=np.float32)
    ubuf = np.empty((max(max_n, 1), Hkv, B, d), dtype=np.uint32)
    hbuf = np.empty((max(max_n, 1), Hkv, B, d), dtype=np.uint16)

    def draw_into(pool, ids, first_logical: int, valid_tokens: int, boost):
        """Draw data for len(ids) consecutive logical blocks and store them
        at physical blocks ``ids``; slots at or past ``valid_tokens`` get
        the fill value."""
        n = len(ids)
        f = fbuf[:n]
        rng.standard_normal(out=f, dtype=np.float32)
        if boost is not None:
            period, factor = boost
            t = first_logical * B + np.arange(n * B).reshape(n, B)
            bi, oi = np.nonzero((t % period) == period - 1)
            f[bi, :, oi, :] *= np.float32(factor)
        # first dead slot, if any, is in logical block (valid_tokens // B)
        last_dead = None
        dead_b = valid_tokens // B - first_logical
        if dead_b < n:
            last_dead = (max(dead_b, 0), valid_tokens - (first_logical + max(dead_b, 0)) * B)
        if fp8:
            if last_dead is not None:
                b0, o0 = last_dead
                f[b0, :, max(o0, 0):, :] = fill
                f[b0 + 1:] = fill
            pool[ids] = f
            return
        u = ubuf[:n]
        bits = f.view(np.uint32)
        np.right_shift(bits, 16, out=u)          # round to nearest even
        np.bitwise_and(u, 1, out=u)
        np.add(u, 0x7FFF, out=u)
        np.add(u, bits, out=u)
        np.right_shift(u, 16, out=u)
        h = hbuf[:n]
        np.copyto(h, u, casting="unsafe")
        if last_dead is not None:
            b0, o0 = last_dead
            h[b0, :, max(o0, 0):, :] = fill
            h[b0 + 1:] = fill
        pool[ids] = h

    if shared_blocks:
        draw_into(k_pool, group_ids, 0, shared_blocks * B, k_boost)
        draw_into(v_pool, group_ids, 0, shared_blocks * B, None)
    for r in range(R):
        if private[r] == 0:
            continue
        draw_into(k_pool, private_ids[r], int(share[r]), int(hist[r]), k_boost)
        draw_into(v_pool, private_ids[r], int(share[r]), int(hist[r]), None)

    # -- 5. new-token K/V
    k_new = v_new = None
    if writes_new_kv:
        k_new = to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))
        v_new = to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))

    # -- 6. fp8 scales and codes
    k_scale = v_scale = np.float32(1.0)
    if fp8:
        def amax(pool, new):
            m = float(np.nanmax(np.abs(pool))) if not np.all(np.isnan(pool)) else 0.0
            if new is not None and new.size:
                m = max(m, float(np.abs((new.astype(np.uint32) << 16).view(np.float32)).max()))
            return np.float32(max(m, 1e-6) / FP8_E4M3_MAX)
        k_scale = amax(k_pool, k_new)
        v_scale = amax(v_pool, v_new)
        kc = to_fp8_codes(k_pool, k_scale)
        vc = to_fp8_codes(v_pool, v_scale)
        kdead = np.isnan(k_pool)
        vdead = np.isnan(v_pool)
        pz = FP8_NAN if poison else np.uint8(0)
        kc[kdead] = pz
        vc[vdead] = pz
        k_pool, v_pool = kc, vc

    qsl = np.zeros(R + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    return Workload(
        name=name, num_q_heads=H, num_kv_heads=Hkv, head_dim=d, block_size=B,
        cache_dtype=cache_dtype, seq_lens=seq_lens.astype(np.int32),
        q_lens=q_lens.astype(np.int32), query_start_loc=qsl,
        block_table=block_table, num_blocks=NB, k_pool=k_pool, v_pool=v_pool,
        q=q, k_new=k_new, v_new=v_new, scale=np.float32(1.0 / np.sqrt(d)),
        k_scale=k_scale, v_scale=v_scale, writes_new_kv=writes_new_kv,
        seed=seed, partition_size=partition_size,
        alibi_slopes=(np.exp2(-8.0 * np.arange(1, H + 1) / H).astype(np.float32)
                      if alibi else None))


# ---------------------------------------------------------------------------
# the five one-layer configurations

CONFIG_NAMES = {
    1: "tiny_decode",
    2: "batched_decode",
    3: "long_context_split_kv",
    4: "mixed_chunked_prefill",
    5: "shared_prefix_fp8_decode",
}


def config_workload(cfg: int, *, poison: bool = True, perm_seed: Optional[int] = None,
                    identity_perm: bool = False, prefill_first: bool = False,
                    share_prefix_rows: int = 0, scale_down: Optional[int] = None) -> Workload:
    """One of the five configurations, seeded with PCG64(7700 + cfg).

    scale_down: divide request counts (and, for the long-context case, the
      context length) by this factor, keeping head shapes, for oracle-sized
      parity runs of the same structure.
    share_prefix_rows (config 4 only): that many decode rows map their first 64
      logical blocks onto the prefill row's first 64 prefix blocks.
    """
    seed = 7700 + cfg
    rng = np.random.Generator(np.random.PCG64(seed))
    common = dict(seed=seed, perm_seed=perm_seed, identity_perm=identity_perm,
                  poison=poison, rng=rng)
    sd = scale_down or 1
    if cfg == 1:
        ctx = [1, 17, 33, 100]
        return make_workload(name=CONFIG_NAMES[1], seq_lens=ctx, q_lens=[1] * 4,
                             num_q_heads=4, num_kv_heads=2, head_dim=64,
                             pool_blocks=64, **common)
    if cfg == 2:
        R = max(1, 64 // sd)
        ctx = rng.integers(512, 4096 + 1, size=R)
        return make_workload(name=CONFIG_NAMES[2], seq_lens=ctx, q_lens=np.ones(R, np.int64),
                             num_q_heads=32, num_kv_heads=8, head_dim=128, **common)
    if cfg == 3:
        R = max(1, 8 // sd)
        L = 32768 // sd
        ctx = np.full(R, L, dtype=np.int64)
        return make_workload(name=CONFIG_NAMES[3], seq_lens=ctx, q_lens=np.ones(R, np.int64),
                             num_q_heads=32, num_kv_heads=8, head_dim=128,
                             writes_new_kv=False, k_boost=(64, 8.0),
                             partition_size=512, **common)
    if cfg == 4:
        R = max(1, 128 // sd)
        ctx = rng.integers(1024, 8192 + 1, size=R)
        pre_q = 2048 // sd
        pre_seq = 8192 // sd
        seq = list(ctx) + [pre_seq]
        ql = [1] * R + [pre_q]
        share = None
        shared = 0
        if share_prefix_rows:
            shared = 64 // sd
            share = [shared if i < share_prefix_rows else 0 for i in range(R)] + [shared]
        if prefill_first:
            seq = seq[-1:] + seq[:-1]
            ql = ql[-1:] + ql[:-1]
            if share is not None:
                share = share[-1:] + share[:-1]
        return make_workload(name=CONFIG_NAMES[4], seq_lens=seq, q_lens=ql,
                             num_q_heads=32, num_kv_heads=8, head_dim=128,
                             shared_blocks=shared, share=share, **common)
    if cfg == 5:
        R = max(1, 256 // sd)
        prefix_blocks = 256 // sd
        tails = rng.integers(64, 1024 + 1, size=R)
        seq = prefix_blocks * BLOCK_SIZE + tails
        return make_workload(name=CONFIG_NAMES[5], seq_lens=seq, q_lens=np.ones(R, np.int64),
                             num_q_heads=28, num_kv_heads=4, head_dim=128,
                             cache_dtype="fp8", writes_new_kv=False,
                             shared_blocks=prefix_blocks,
                             share=np.full(R, prefix_blocks), **common)
    raise ValueError(f"unknown config {cfg}")


def decode_q(w: Workload) -> np.ndarray:
    """Queries as ``[R, Hq, d]`` for decode workloads (one query row per request)."""
    assert np.all(w.q_lens == 1)
    return w.q
