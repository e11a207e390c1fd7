"""Block pool with reference counts and copy-on-write -- test infrastructure only.

What the pages fix:
* "PagedAttention 机制" (cs-knowledge-wiki) §5.3.4, BlockAllocator: every
  physical block has a reference count; allocating takes a free block and
  sets its count to 1 (no free block: out of memory); freeing decrements the
  count and returns the block to the free list when it reaches 0;
  incr_ref adds a reference for sharing.
* "01. PagedAttention 详解" (vLLM learning book) 自检 Q3: the free list is a
  queue; get_new_blocks takes blocks from its head (least recently freed
  first) and free_blocks appends a block whose count reaches 0 to its tail.
  (The wiki's sketch pops the end of a plain list instead; the book's queue
  order is the reading taken.) The pool starts with every block free, in id
  order.
* The book's §6: a block shared by several tables (count > 1) is copied
  before one of them writes into it -- copy-on-write: the writer gets a fresh
  block holding a copy, and the shared block loses that reference.

Plain Python; the pins in ``tests/test_block_pool.py`` tie it to the pages'
statements and figures.
"""
from __future__ import annotations

from collections import deque
from typing import List, Optional, Tuple

import numpy as np

__all__ = ["BlockPool", "OutOfBlocks", "copy_blocks"]


class OutOfBlocks(RuntimeError):
    """Fewer free blocks than requested (the wiki's OutOfMemoryError)."""


class BlockPool:
    def __init__(self, num_blocks: int):
        self.num_blocks = int(num_blocks)
        self.ref = [0] * self.num_blocks
        self.free_queue = deque(range(self.num_blocks))

    def num_free(self) -> int:
        return len(self.free_queue)

    def allocate(self, n: int) -> List[int]:
        """n blocks from the head of the free queue, each with count 1."""
        if n > len(self.free_queue):
            raise OutOfBlocks(f"{n} blocks requested, {len(self.free_queue)} free")
        out = []
        for _ in range(n):
            b = self.free_queue.popleft()
            self.ref[b] = 1
            out.append(b)
        return out

    def free(self, blocks) -> None:
        """Drop one reference of each listed block; at 0 it goes to the queue's tail.

        All or nothing: a block listed more often than it is referenced, or
        not allocated, leaves the pool unchanged.
        """
        blocks = list(blocks)
        for b in set(blocks):
            if not 0 <= b < self.num_blocks or self.ref[b] < blocks.count(b):
                raise ValueError(f"block {b} is not allocated that often")
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free_queue.append(b)

    def share(self, blocks) -> None:
        """One more reference to each block (a second table points at it).

        All or nothing: a block that is not allocated leaves the pool unchanged.
        """
        blocks = list(blocks)
        for b in blocks:
            if not 0 <= b < self.num_blocks or self.ref[b] == 0:
                raise ValueError(f"block {b} is not allocated")
        for b in blocks:
            self.ref[b] += 1

    def copy_on_write(self, block: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """The block a writer may write into, and the (src, dst) copy it needs.

        A block with one reference is written in place. A shared one keeps its
        other references; the writer gets a fresh block that must first receive
        a copy of the shared block's contents.
        """
        if not 0 <= block < self.num_blocks or self.ref[block] == 0:
            raise ValueError(f"block {block} is not allocated")
        if self.ref[block] == 1:
            return block, None
        (new,) = self.allocate(1)
        self.ref[block] -= 1
        return new, (block, new)


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray,
                pairs) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the caches with block dst := block src for every (src, dst)."""
    kc = key_cache.copy()
    vc = value_cache.copy()
    for src, dst in pairs:
        kc[dst] = key_cache[src]
        vc[dst] = value_cache[src]
    return kc, vc
