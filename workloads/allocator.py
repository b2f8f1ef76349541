"""Caller-side bookkeeping for a paged KV cache: block pool, block tables, slot mapping.

This is the host half of the method, the part a serving engine owns and hands to
the device as three small integer arrays (block tables, slot mapping, context
lengths).  It is re-implemented here only to build and check inputs; the library
never allocates blocks.

Sources (cited by page title and section):
  * "4.6 PagedAttention & KV-Cache Memory Management" (LLM stack book), sections
    "Block Tables, the Allocator & Copy-on-Write", "Copy-on-write for shared
    prefixes", "From Python bookkeeping to the tensors the kernel actually takes"
    and "Putting It Together" (grow the table before computing the slot).
  * "Paged KV cache" (ai-infra-handbooks), sections "Implementation" (block pool
    with a FIFO free queue and reference counts; allocation that reports a
    shortfall instead of raising) and "Block tables and slot mapping".
  * "Allocate the Cache: Blocks, Waste, and PagedAttention", section "How the
    Block Table Works" (logical block = t // B, offset = t % B).
"""
from __future__ import annotations

from collections import deque
from typing import Iterable, Sequence

import numpy as np


class BlockPool:
    """A fixed number of physical blocks: a FIFO queue of free ids and a refcount each.

    Blocks released by :meth:`free` go to the back of the queue, so freshly freed
    blocks are reused last (the ai-infra-handbooks "Paged KV cache" page, section
    "Implementation", prints the resulting order in its doctest).
    """

    def __init__(self, num_blocks: int):
        if num_blocks < 0:
            raise ValueError("num_blocks must be non-negative")
        self.num_blocks = int(num_blocks)
        self.ref_cnt = [0] * self.num_blocks
        self._free = deque(range(self.num_blocks))

    def num_free(self) -> int:
        return len(self._free)

    def allocate(self, n: int) -> list[int] | None:
        """Take ``n`` free blocks (refcount 1 each), or return None if fewer are free."""
        if n > len(self._free):
            return None
        got = []
        for _ in range(n):
            blk = self._free.popleft()
            self.ref_cnt[blk] = 1
            got.append(blk)
        return got

    def share(self, blk: int) -> None:
        """Add one more reference to an allocated block (prefix sharing)."""
        if self.ref_cnt[blk] <= 0:
            raise ValueError(f"block {blk} is not allocated")
        self.ref_cnt[blk] += 1

    def free(self, blocks: Iterable[int]) -> None:
        """Drop one reference per listed block; a block whose count reaches 0 is free again."""
        for blk in blocks:
            if self.ref_cnt[blk] <= 0:
                raise ValueError(f"block {blk} freed more often than allocated")
            self.ref_cnt[blk] -= 1
            if self.ref_cnt[blk] == 0:
                self._free.append(blk)


class BlockManager:
    """Per-sequence block tables over a :class:`BlockPool`.

    Semantics follow the LLM stack book, section "Block Tables, the Allocator &
    Copy-on-Write": allocation on demand, an exhausted pool raises MemoryError,
    a decode step grows the table only when the write position starts a new
    block, and copy-on-write hands back the (source, destination) pair of a
    block that must be copied before the write.
    """

    def __init__(self, num_blocks: int, block_size: int, pool: BlockPool | None = None):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.block_size = int(block_size)
        self.pool = pool if pool is not None else BlockPool(num_blocks)
        self.block_tables: dict = {}

    # -- helpers -----------------------------------------------------------
    def _take(self, n: int) -> list[int]:
        got = self.pool.allocate(n)
        if got is None:
            raise MemoryError("KV block pool exhausted; the scheduler must preempt a sequence")
        return got

    def blocks_for(self, num_tokens: int) -> int:
        return -(-int(num_tokens) // self.block_size)

    # -- allocation --------------------------------------------------------
    def allocate(self, seq_id, num_tokens: int) -> list[int]:
        """Give a new sequence ceil(num_tokens / block_size) blocks (after its prefill)."""
        table = self._take(self.blocks_for(num_tokens))
        self.block_tables[seq_id] = table
        return table

    def append_token(self, seq_id, cur_len: int) -> None:
        """Make room for the token at position ``cur_len`` before it is written.

        A new block is needed exactly when ``cur_len`` is a multiple of the block
        size; doing this before :meth:`slot_index` covers a prompt whose length is
        an exact multiple of the block size.
        """
        if cur_len % self.block_size == 0:
            self.block_tables[seq_id].append(self._take(1)[0])

    def slot_index(self, seq_id, pos: int) -> int:
        """Flat pool slot of logical position ``pos``: physical block * B + pos % B."""
        table = self.block_tables[seq_id]
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    # -- sharing -----------------------------------------------------------
    def fork(self, parent_id, child_id) -> None:
        """Child shares every block of the parent: the table is copied, refcounts bumped."""
        parent = self.block_tables[parent_id]
        for blk in parent:
            self.pool.share(blk)
        self.block_tables[child_id] = list(parent)

    def cow_append(self, seq_id, logical_block: int) -> tuple[int, int]:
        """Ensure ``seq_id`` owns ``logical_block`` privately before writing into it.

        Returns (src, dst).  If they differ the caller copies block src to dst on
        the device and then writes; the table entry already points at dst.
        """
        table = self.block_tables[seq_id]
        src = table[logical_block]
        if self.pool.ref_cnt[src] == 1:
            return src, src
        dst = self._take(1)[0]
        self.pool.free([src])
        table[logical_block] = dst
        return src, dst

    def free_seq(self, seq_id) -> None:
        self.pool.free(self.block_tables.pop(seq_id))

    # -- queries -----------------------------------------------------------
    def num_free_blocks(self) -> int:
        return self.pool.num_free()

    def can_allocate(self, num_tokens: int) -> bool:
        return self.blocks_for(num_tokens) <= self.pool.num_free()


def slot_mapping_for(block_table: Sequence[int], positions: Iterable[int], block_size: int) -> list[int]:
    """Slots of ``positions`` in one sequence: table[p // B] * B + p % B."""
    return [int(block_table[p // block_size]) * block_size + p % block_size for p in positions]


def build_step_tensors(tables: Sequence[Sequence[int]], cur_lens: Sequence[int], block_size: int):
    """The three int32 arrays of one decode step, for sequences with ``cur_lens`` cached tokens.

    * block_tables [B, max_blocks], right-padded with 0 (padding is never read);
    * slot_mapping [B], the slot of the token written this step (position cur_len);
    * context_lens [B] = cur_len + 1, valid tokens after this step's write.

    Each table must already cover position cur_len (call append_token first).
    """
    nseq = len(tables)
    max_blocks = max((len(t) for t in tables), default=0)
    bt = np.zeros((nseq, max(max_blocks, 1)), dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = np.asarray(t, dtype=np.int32)
    slots = np.array([slot_mapping_for(t, [n], block_size)[0] for t, n in zip(tables, cur_lens)],
                     dtype=np.int32)
    ctx = np.array([n + 1 for n in cur_lens], dtype=np.int32)
    return bt, slots, ctx
