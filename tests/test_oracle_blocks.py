"""Pins of the block-manager model (oracle/block_pool.py) against what the
pages and published definitions fix: the FNV-1a and splitmix64 test values,
the chain property of the block hash, the ref_cnt timeline of two requests
sharing a block (tests/golden/ref_count_timeline.txt), the last-token rule
and the block LRU model's 0 / 0 / 21,488 hit tokens
(tests/golden/lru_model.txt)."""
import numpy as np

from oracle import block_pool as bp


def test_fnv1a64_published_values():
    assert bp.fnv1a64(b"") == 0xCBF29CE484222325
    assert bp.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert bp.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_splitmix64_published_sequence():
    # splitmix64 seeded with 0: state += 0x9e3779b97f4a7c15, output = mix(state)
    s, out = 0, []
    for _ in range(3):
        s = (s + 0x9E3779B97F4A7C15) & bp.MASK
        out.append(bp.splitmix64_finalise(s))
    assert out == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_block_hash_chain_property():
    rng = np.random.default_rng(1)
    a = rng.integers(0, 50000, size=80).tolist()
    ha = bp.block_hashes(a, 16)
    assert len(ha) == 5 and len(bp.block_hashes(a[:79], 16)) == 4
    b = list(a)
    b[40] += 1                                   # block 2 changes
    hb = bp.block_hashes(b, 16)
    assert hb[:2] == ha[:2] and all(x != y for x, y in zip(hb[2:], ha[2:]))
    c = [7] * 16 + a[16:]                        # same later tokens, other prefix
    hc = bp.block_hashes(c, 16)
    assert hc[0] != ha[0] and all(x != y for x, y in zip(hc[1:], ha[1:]))
    assert bp.block_hashes(a, 16, extra_key=3) != ha
    assert ha[0] == bp.block_hash(bp.NONE_HASH, a[:16])


def ref_count_timeline(pool, ref_of, queued_of):
    """Requests A and B whose first 16 tokens agree ("Hello, how are"): the
    shared block's (ref count, queued) after each event of the timeline."""
    shared = list(range(100, 116))
    A, B = shared + [1], shared + [2, 3]
    hA, hB = bp.block_hashes(A, 16), bp.block_hashes(B, 16)
    rowA, _ = pool.allocate_prompt(hA, len(A), 16)
    pool.commit(rowA, hA)
    p = rowA[0]
    seen = [(ref_of(p), queued_of(p))]
    rowB, cachedB = pool.allocate_prompt(hB, len(B), 16)
    assert rowB[0] == p and cachedB == 16          # B reads A's block
    seen.append((ref_of(p), queued_of(p)))
    pool.free_request(rowA)
    seen.append((ref_of(p), queued_of(p)))
    pool.free_request(rowB)
    seen.append((ref_of(p), queued_of(p)))
    assert pool.lookup(hA[0]) == p                 # count 0, still cached
    return seen


def golden_timeline(golden):
    return [(int(r[3]), r[4] == "yes") for r in golden("ref_count_timeline.txt")]


def test_ref_count_timeline(golden):
    m = bp.BlockPoolModel(8)
    assert ref_count_timeline(m, lambda b: m.ref[b], lambda b: b in m.queue) == \
        golden_timeline(golden)


def test_last_token_is_always_computed():
    """A prompt whose every full block is cached still computes its last
    token: 32 cached tokens reuse one block, 33 reuse both."""
    m = bp.BlockPoolModel(16)
    toks = list(range(33))
    h = bp.block_hashes(toks, 16)
    row, cached = m.allocate_prompt(h, 32, 16)
    m.commit(row, h)
    m.free_request(row)
    assert cached == 0
    row2, cached2 = m.allocate_prompt(h, 32, 16)
    assert cached2 == 16 and row2[0] == row[0]
    m.free_request(row2)
    row3, cached3 = m.allocate_prompt(h, 33, 16)
    assert cached3 == 32 and row3[:2] == row[:2]


def lru_scan(pool_factory, hashes_fn, golden_rows):
    params = [r for r in golden_rows if r[0] == "params"][0]
    B, usable, docs, n = (int(x) for x in params[1:])
    pool = pool_factory(usable + 1)
    docs_tokens = [[d * 100000 + t for t in range(n)] for d in range(docs)]
    doc_hashes = [hashes_fn(t, B) for t in docs_tokens]
    got = []
    for r in [r for r in golden_rows if r[0] == "round"]:
        order = range(docs) if r[2] == "forward" else reversed(range(docs))
        hit = 0
        for d in order:
            row, cached = pool.allocate_prompt(doc_hashes[d], n, B)
            pool.commit(row, doc_hashes[d])
            pool.free_request(row)
            hit += cached
        got.append((hit, int(r[3])))
    return got


def test_lru_model_hit_tokens(golden):
    got = lru_scan(bp.BlockPoolModel, bp.block_hashes, golden("lru_model.txt"))
    assert [g for g, _ in got] == [w for _, w in got] == [0, 0, 21488]


def test_pool_conservation_under_random_use():
    rng = np.random.default_rng(3)
    m = bp.BlockPoolModel(64)
    live = []
    for step in range(300):
        if live and (rng.random() < 0.45 or m.num_free() < 10):
            m.free_request(live.pop(int(rng.integers(len(live)))))
        else:
            prefix = int(rng.integers(0, 4))
            toks = [prefix] * 16 * int(rng.integers(0, 3)) + \
                rng.integers(0, 99, size=int(rng.integers(1, 60))).tolist()
            h = bp.block_hashes(toks, 16)
            try:
                row, _ = m.allocate_prompt(h, len(toks), 16)
            except ValueError:
                continue
            m.commit(row, h)
            live.append(row)
        held = sum(m.ref)
        assert m.num_free() + sum(1 for b in range(1, 64) if m.ref[b] > 0) == 63
        assert all(m.ref[b] == 0 for b in m.queue) and len(set(m.queue)) == len(m.queue)
        assert held == sum(len(r) for r in live)


def test_map_to_kernel_blocks_page_example(golden):
    (k, ids, want), = golden("kernel_blocks.txt")
    ids = [int(x) for x in ids.split()]
    assert bp.map_to_kernel_blocks(ids, int(k)) == [int(x) for x in want.split()]


def test_map_to_kernel_blocks_covers_the_same_tokens():
    """Token t of a request sits in manager block t // (16k), kernel block
    t // 16: the expanded row must name the kernel block that holds it."""
    rng = np.random.default_rng(4)
    for k in (1, 2, 4):
        ids = rng.permutation(50)[:7].tolist()
        row = bp.map_to_kernel_blocks(ids, k)
        assert len(row) == 7 * k
        for t in range(7 * 16 * k):
            mgr = ids[t // (16 * k)]
            within = (t % (16 * k)) // 16           # kernel block inside the manager block
            assert row[t // 16] == mgr * k + within
    assert bp.map_to_kernel_blocks([3, -1], 2) == [6, 7, -1, -1]
