"""CPU reference model of the host block manager (pool, reference counts,
free queue, prefix-cache index).

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` may import it; the library's block
manager (C++, include/pa_blocks.h) shares no code with it.

Written from these pages:
  [P1] "vLLM 深度解析（二）：PagedAttention 核心机制" §4.1: full blocks get a
       chained hash H_i = H(H_{i-1}, token_ids_i, extra_keys_i) with a fixed
       NONE_HASH before the first block; only full blocks are cached;
       touch() takes a block with count 0 off the free queue and adds one;
       free_blocks() subtracts one and queues blocks that reach zero; a fully
       cached prompt still recomputes its last token.
  [P3] "vllm 深度解析：一切从 PagedAttention 谈起": BlockPool (block 0 is the
       null block, taken at creation; get_new_blocks pops the queue head and
       evicts the popped block's cached hash; get_usage), the LRU free queue
       (head = evicted first), the hash index (several blocks per hash, pop
       by block id) and the two-request ref_cnt timeline.
  [P4] "LLM 推理基础与 vLLM 内部机制：KV 缓存、PagedAttention、调度器" §9-§10:
       the block LRU model (tail blocks queued first, partial blocks have no
       hash and are reused at once) and its 0 / 0 / 21,488 hit tokens.

Readings (the same as the library's): the hash H is 64-bit FNV-1a over the
little-endian bytes of (parent, the block's int32 token ids, extra key)
followed by the splitmix64 finaliser, NONE_HASH = 0x9e3779b97f4a7c15; freed
blocks with no cached hash go to the head of the free queue (given order),
cached ones to the tail.
"""
from __future__ import annotations

MASK = (1 << 64) - 1
NONE_HASH = 0x9E3779B97F4A7C15
FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a: xor each byte in, then multiply by the FNV prime."""
    h = FNV_OFFSET
    for c in data:
        h = ((h ^ c) * FNV_PRIME) & MASK
    return h


def splitmix64_finalise(z: int) -> int:
    """The output mix of splitmix64 (two xor-shift-multiply rounds, xor-shift)."""
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def block_hash(parent: int, tokens, extra_key: int = 0) -> int:
    """H(parent, token ids of one full block, extra key) (P1 §4.1)."""
    data = parent.to_bytes(8, "little")
    for t in tokens:
        data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    data += (extra_key & MASK).to_bytes(8, "little")
    return splitmix64_finalise(fnv1a64(data))


def block_hashes(tokens, block_size: int, extra_key: int = 0) -> list:
    """Chained hashes of the full blocks of ``tokens`` (a partial tail has none)."""
    out, parent = [], NONE_HASH
    for i in range(len(tokens) // block_size):
        parent = block_hash(parent, tokens[i * block_size:(i + 1) * block_size], extra_key)
        out.append(parent)
    return out


def map_to_kernel_blocks(ids, blocks_per_kv_block: int) -> list:
    """Manager block b of k kernel blocks covers kernel blocks b*k .. b*k+k-1
    (P3 BlockTable.map_to_kernel_blocks); padding (negative) stays as is."""
    k = blocks_per_kv_block
    out = []
    for b in ids:
        for j in range(k):
            out.append(b if b < 0 else b * k + j)
    return out


class BlockPoolModel:
    """Plain-list model of the block pool (P3 BlockPool)."""

    def __init__(self, num_blocks: int, caching: bool = True):
        self.n = num_blocks
        self.caching = caching
        self.ref = [0] * num_blocks
        self.queue = list(range(num_blocks))
        self.queue.pop(0)                         # the null block never circulates
        self.hash_of = {}                         # block -> hash
        self.index = {}                           # hash -> [blocks], insertion order

    # -- queries
    def num_free(self) -> int:
        return len(self.queue)

    def usage(self) -> float:
        return 1.0 - len(self.queue) / (self.n - 1) if self.n > 1 else 0.0

    def lookup(self, h: int) -> int:
        blocks = self.index.get(h)
        return blocks[0] if blocks else -1

    # -- block operations
    def _evict(self, b: int) -> None:
        h = self.hash_of.pop(b, None)
        if h is not None:
            self.index[h].remove(b)
            if not self.index[h]:
                del self.index[h]

    def get_new_blocks(self, n: int) -> list:
        if n > len(self.queue):
            raise ValueError("not enough free blocks")
        out = []
        for _ in range(n):
            b = self.queue.pop(0)                 # least recently freed
            self._evict(b)
            self.ref[b] += 1
            out.append(b)
        return out

    def touch(self, blocks) -> None:
        for b in blocks:
            if self.ref[b] == 0 and b != 0 and b in self.queue:
                self.queue.remove(b)
            self.ref[b] += 1

    def free_blocks(self, blocks) -> None:
        blocks = list(blocks)
        for b in blocks:
            if self.ref[b] - blocks.count(b) < 0:
                raise ValueError("count below zero")
        front = []
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0 and b != 0:
                if b in self.hash_of:
                    self.queue.append(b)
                else:
                    front.append(b)
        self.queue = front + self.queue

    def cache_block(self, b: int, h: int) -> None:
        if not self.caching or b in self.hash_of:
            return
        self.hash_of[b] = h
        self.index.setdefault(h, []).append(b)

    # -- request level
    def allocate_prompt(self, hashes, num_tokens: int, block_size: int):
        """(block-table row, tokens already cached) for a prompt."""
        nblk = -(-num_tokens // block_size)
        hits = []
        if self.caching:
            for i, h in enumerate(hashes):
                if (i + 1) * block_size > num_tokens - 1:
                    break                          # the last token is always computed
                b = self.lookup(h)
                if b < 0:
                    break
                hits.append(b)
        queued_hits = sum(1 for b in hits if self.ref[b] == 0 and b in self.queue)
        need = nblk - len(hits)
        if need > len(self.queue) - queued_hits:
            raise ValueError("not enough free blocks")
        self.touch(hits)
        return hits + self.get_new_blocks(need), len(hits) * block_size

    def commit(self, blocks, hashes) -> None:
        for b, h in zip(blocks, hashes):
            self.cache_block(b, h)

    def free_request(self, blocks) -> None:
        self.free_blocks(list(reversed(list(blocks))))   # tail evicted first
