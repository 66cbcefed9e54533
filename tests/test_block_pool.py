"""The C++ block manager (include/pa_blocks.h, via paged_kv_cache_77_amd.blocks)
against the oracle model: hashes, the pinned scenarios, and random operation
sequences compared step by step (integer results: exact)."""
import numpy as np
import pytest

from oracle import block_pool as bp
from paged_kv_cache_77_amd import blocks as pb
import paged_kv_cache_77_amd as pa
from tests.test_oracle_blocks import golden_timeline, lru_scan, ref_count_timeline


@pytest.mark.parametrize("B", [1, 16, 32])
def test_block_hashes_match_oracle(B):
    rng = np.random.default_rng(B)
    for n in (0, B - 1, B, 5 * B + 3):
        toks = rng.integers(-(1 << 31), 1 << 31, size=max(n, 0)).tolist()
        for extra in (0, 12345, (1 << 64) - 1):
            assert pb.block_hashes(toks, B, extra) == bp.block_hashes(toks, B, extra)


def test_ref_count_timeline(golden):
    p = pb.BlockPool(8)
    got = ref_count_timeline(p, p.ref_count, lambda b: p.ref_count(b) == 0 and p.num_free() == 7)
    assert got == golden_timeline(golden)


def test_lru_model_hit_tokens(golden):
    got = lru_scan(pb.BlockPool, pb.block_hashes, golden("lru_model.txt"))
    assert [g for g, _ in got] == [w for _, w in got] == [0, 0, 21488]


def _state(pool_ref, n):
    return [pool_ref(b) for b in range(n)]


@pytest.mark.parametrize("seed,caching", [(0, True), (1, True), (2, False), (3, True)])
def test_random_sequences_match_model(seed, caching):
    rng = np.random.default_rng(seed)
    N = 48
    c, m = pb.BlockPool(N, caching), bp.BlockPoolModel(N, caching)
    live = []
    seen_hashes = set()
    for step in range(400):
        op = rng.random()
        if live and (op < 0.4 or c.num_free() < 6):
            row = live.pop(int(rng.integers(len(live))))
            c.free_request(row)
            m.free_request(row)
        else:
            prefix = int(rng.integers(0, 3))
            toks = [prefix] * 16 * int(rng.integers(0, 4)) + \
                rng.integers(0, 50, size=int(rng.integers(1, 70))).tolist()
            h = bp.block_hashes(toks, 16)
            seen_hashes.update(h)
            try:
                want = m.allocate_prompt(h, len(toks), 16)
            except ValueError:
                with pytest.raises(pa.PaError):
                    c.allocate_prompt(h, len(toks), 16)
                continue
            got = c.allocate_prompt(h, len(toks), 16)
            assert got == want, step
            if rng.random() < 0.8:                      # sometimes never committed
                c.commit(got[0], h)
                m.commit(got[0], h)
            live.append(got[0])
        assert c.num_free() == m.num_free()
        assert abs(c.usage() - m.usage()) < 1e-12
        assert _state(c.ref_count, N) == m.ref
        for hh in seen_hashes:
            assert c.lookup(hh) == m.lookup(hh)
    # the free queue order: drain it and compare
    n = c.num_free()
    assert c.get_new_blocks(n) == m.get_new_blocks(n)


def test_errors_leave_the_pool_unchanged():
    c = pb.BlockPool(5)
    got = c.get_new_blocks(3)
    with pytest.raises(pa.PaError):
        c.get_new_blocks(2)                              # one block left
    with pytest.raises(pa.PaError):
        c.free_blocks([got[0], got[0]])                  # count would go negative
    assert [c.ref_count(b) for b in got] == [1, 1, 1] and c.num_free() == 1
    with pytest.raises(pa.PaError):
        c.allocate_prompt([], 40, 16)                    # needs 3 blocks, 1 free
    assert c.num_free() == 1
    c.free_blocks(got)
    assert c.num_free() == 4 and c.ref_count(0) == 0 and c.usage() == 0.0
    assert c.ref_count(99) == -1


def test_map_to_kernel_blocks_matches_oracle(golden):
    (k, ids, want), = golden("kernel_blocks.txt")
    assert pb.map_to_kernel_blocks([int(x) for x in ids.split()], int(k)) == \
        [int(x) for x in want.split()]
    rng = np.random.default_rng(5)
    for k in (1, 2, 3, 8):
        ids = rng.integers(-2, 1000, size=33).tolist()
        assert pb.map_to_kernel_blocks(ids, k) == bp.map_to_kernel_blocks(ids, k)
    with pytest.raises(pa.PaError):
        pb.map_to_kernel_blocks([1], 0)
    with pytest.raises(pa.PaError):
        pb.map_to_kernel_blocks([1 << 30], 4)
