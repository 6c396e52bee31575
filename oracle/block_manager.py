"""Reference KV-cache block manager: plain Python, the pages' rules.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): only the tests and
``__graft_entry__.smoke()`` use it; the library never does.

Rules, from the vLLM manual (doramagic.ai/projects/vllm/manual):
  * "KVCacheManager -- cache block management": the free blocks form a deque
    holding 0 .. num_blocks-1 at start; a request of n tokens takes
    ceil(n / block_size) blocks from the deque's front; freeing a request
    puts its blocks back at the deque's end, in the request's block order;
    an empty deque means the KV cache is exhausted.
  * "sharing mechanism": blocks shared between requests carry a reference
    count and go back to the free deque only when it reaches zero.
  * "cache allocation strategy" (dynamic extension at run time): a request
    that grows past its last block gets one more block from the front.
Readings where the printed code is silent or would lose state:
  * an allocation that does not fit fails before taking any block;
  * allocating an id that already holds blocks is an error;
  * sharing hands the first k whole blocks of one request to a new request
    (its length becomes k * block_size), one more reference each;
  * forking hands every block of a request to a new one (same length;
    "vLLM 2026 推理引擎全解" (chenxutan.com) §2.1: parallel sampling and beam
    search share a prompt's pages), one more reference each;
  * appending one token to a request whose length is a multiple of the
    block size takes a new block first; a token that would land in a last
    block other requests still map gets a fresh block in its place, whose
    contents the caller copies from the shared one (copy-on-write); the
    token's slot is block_table[(L-1) // bs] * bs + (L-1) % bs for the new
    length L (same page, §2.2: page_id * BLOCK_SIZE + page_offset).
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List


class KVCacheExhausted(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free_blocks = deque(range(num_blocks))
        self.refcount = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}

    def _take(self, n: int) -> List[int]:
        if n > len(self.free_blocks):
            raise KVCacheExhausted("KV cache exhausted")
        out = []
        for _ in range(n):
            b = self.free_blocks.popleft()
            self.refcount[b] = 1
            out.append(b)
        return out

    def allocate(self, rid: int, num_tokens: int) -> List[int]:
        if rid in self.tables or num_tokens < 0:
            raise ValueError("bad request id or length")
        need = -(-num_tokens // self.block_size)
        blocks = self._take(need)
        self.tables[rid] = blocks
        self.lengths[rid] = num_tokens
        return list(blocks)

    def share(self, src: int, dst: int, num_blocks: int) -> None:
        if src not in self.tables or dst in self.tables or num_blocks < 0:
            raise ValueError("bad request ids")
        if num_blocks * self.block_size > self.lengths[src]:
            raise ValueError("only whole blocks of the source can be shared")
        blocks = self.tables[src][:num_blocks]
        for b in blocks:
            self.refcount[b] += 1
        self.tables[dst] = list(blocks)
        self.lengths[dst] = num_blocks * self.block_size

    def fork(self, src: int, dst: int) -> None:
        if src not in self.tables or dst in self.tables:
            raise ValueError("bad request ids")
        for b in self.tables[src]:
            self.refcount[b] += 1
        self.tables[dst] = list(self.tables[src])
        self.lengths[dst] = self.lengths[src]

    def append(self, rid: int):
        """One more token: returns (slot, copy) with copy = (shared block,
        fresh block) when the request had to leave a shared block, else None."""
        if rid not in self.tables:
            raise ValueError("unknown request")
        L = self.lengths[rid]
        tab = self.tables[rid]
        copy = None
        if L % self.block_size == 0:
            tab += self._take(1)
        elif self.refcount[tab[-1]] > 1:
            fresh = self._take(1)[0]
            self.refcount[tab[-1]] -= 1
            copy = (tab[-1], fresh)
            tab[-1] = fresh
        L += 1
        self.lengths[rid] = L
        t = L - 1
        return tab[t // self.block_size] * self.block_size + t % self.block_size, copy

    def free(self, rid: int) -> None:
        if rid not in self.tables:
            return
        for b in self.tables.pop(rid):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free_blocks.append(b)
        del self.lengths[rid]

    def table(self, rid: int) -> List[int]:
        return list(self.tables[rid])

    def num_free(self) -> int:
        return len(self.free_blocks)


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """Block copy of the copy-on-write step, on host arrays [N, Hkv, bs, D]:
    every (src, dst) pair gets block src of both caches written onto block
    dst (sources read before any destination is written)."""
    pairs = [(int(a), int(b)) for a, b in pairs]
    ks = [k_cache[a].copy() for a, _ in pairs]
    vs = [v_cache[a].copy() for a, _ in pairs]
    for (_, b), kb, vb in zip(pairs, ks, vs):
        k_cache[b] = kb
        v_cache[b] = vb
