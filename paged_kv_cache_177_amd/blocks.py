"""Host-side block management for the paged KV pool.

NeuroGrid releases, v0.7.0 "Paged KV Cache": the cache is carved into fixed 16-token blocks,
allocated on demand by an O(1) allocator, and each sequence maps its logical blocks to physical
ones through its own block table.

The library's kernels never allocate blocks: block tables are caller-owned int32 device arrays.
This module is the caller side of that contract, in plain Python (no device work): a LIFO free
list with O(1) ``alloc``/``free`` and a per-sequence table that grows by one block whenever a
token lands on a 16-token boundary.
"""

from __future__ import annotations

from typing import Iterable

import numpy as np

BLOCK_SIZE = 16


class BlockAllocator:
    """LIFO free list of physical block ids.

    ``alloc`` pops the most recently freed (or, initially, the last listed) id; ``free`` pushes ids
    back. Both are O(1) per block. Double frees and foreign ids raise ``ValueError``.
    """

    def __init__(self, free_ids: Iterable[int]):
        self._stack = [int(i) for i in free_ids]
        self._free = set(self._stack)
        if len(self._free) != len(self._stack):
            raise ValueError("duplicate block id in the initial free list")
        self._known = set(self._stack)

    @property
    def num_free(self) -> int:
        return len(self._stack)

    def alloc(self) -> int:
        if not self._stack:
            raise MemoryError("paged KV pool exhausted")
        blk = self._stack.pop()
        self._free.discard(blk)
        return blk

    def free(self, ids: Iterable[int]) -> None:
        for i in ids:
            i = int(i)
            if i not in self._known:
                raise ValueError(f"block {i} was never owned by this allocator")
            if i in self._free:
                raise ValueError(f"double free of block {i}")
            self._stack.append(i)
            self._free.add(i)

    def adopt(self, ids: Iterable[int]) -> None:
        """Register ids that start out in use (handed to sequences before any ``alloc``)."""
        for i in ids:
            i = int(i)
            if i in self._known:
                raise ValueError(f"block {i} already known")
            self._known.add(i)


class SequenceBlocks:
    """Logical-to-physical block list of one sequence."""

    def __init__(self, blocks: Iterable[int] = ()):
        self.blocks = [int(b) for b in blocks]

    def ensure_token(self, token_index: int, allocator: BlockAllocator) -> None:
        """Make sure the block holding ``token_index`` exists (a new block on a 16-token boundary)."""
        need = token_index // BLOCK_SIZE + 1
        while len(self.blocks) < need:
            self.blocks.append(allocator.alloc())


def block_table_array(seqs: list[SequenceBlocks], stride: int, pad_block: int) -> np.ndarray:
    """Pack per-sequence block lists into a [B][stride] int32 table; unused entries -> ``pad_block``."""
    bt = np.full((len(seqs), stride), pad_block, dtype=np.int32)
    for b, s in enumerate(seqs):
        if len(s.blocks) > stride:
            raise ValueError(f"row {b} has {len(s.blocks)} blocks > stride {stride}")
        bt[b, : len(s.blocks)] = s.blocks
    return bt
