"""Block manager: free list, reference counts, block tables, copy-on-write
(oracle; test infrastructure only).

Follows:
* "What is PagedAttention" (tecyfy), "How it works": fixed-size blocks are
  handed out as a sequence grows; a sequence holds only the blocks it has
  filled plus part of the last one; a table records where its blocks are.
* chipfoundryservices glossary "pagedattention vllm": "Memory Management >
  Block Allocation" (a free list; allocate from it on demand; give blocks back
  when a sequence completes), "Copy-on-Write Sharing > Reference Counting"
  (count the references to each block; a block is free again when its count
  reaches zero) and "> Divergence Handling" (before a sequence writes into a
  shared block, copy the block and point that sequence's table at the copy;
  other sequences are unaffected).

Deterministic policy (the pages leave it open): the free list starts in a
given order; blocks are taken from its front; blocks whose count drops to
zero are put back at its front, in table order.  A fork gives the child the
parent's table and length and adds one reference to every shared block.
Appending at position t allocates a block when t % B == 0; otherwise, if the
last block has more than one reference, it is copied first and the pair
(shared, copy) is reported for the device-side block copy.  With a sliding
window, blocks wholly before the window are released and their table
entries set to -1.
"""
from __future__ import annotations

from collections import deque


class BlockManagerError(Exception):
    pass


class NoFreeBlocks(BlockManagerError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise BlockManagerError("free order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.refcount = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}

    def add_seq(self, seq: int) -> None:
        if seq in self.tables:
            raise BlockManagerError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lengths[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables or child in self.tables:
            raise BlockManagerError("fork needs an existing parent and a new child")
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            if b >= 0:
                self.refcount[b] += 1

    def _take(self) -> int:
        if not self.free:
            raise NoFreeBlocks("block pool exhausted")
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def append(self, seq: int):
        """Reserve the slot of the next token.  Returns (slot, cow) where cow
        is None or the (shared source, private copy) pair to copy first."""
        if seq not in self.tables:
            raise BlockManagerError(f"unknown sequence {seq}")
        table, t, B = self.tables[seq], self.lengths[seq], self.block_size
        cow = None
        if t % B == 0:
            table.append(self._take())
        else:
            last = table[-1]
            if self.refcount[last] > 1:
                copy = self._take()
                self.refcount[last] -= 1
                table[-1] = copy
                cow = (last, copy)
        self.lengths[seq] = t + 1
        return table[t // B] * B + t % B, cow

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise BlockManagerError(f"unknown sequence {seq}")
        for b in self.tables.pop(seq):
            if b < 0:
                continue
            if self.refcount[b] <= 0:
                raise BlockManagerError("reference count underflow")
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.appendleft(b)
        del self.lengths[seq]

    def move_seq(self, other: "BlockManager", seq: int):
        """Move a sequence to another pool ("Memory Management > Swapping":
        blocks swap between GPU and CPU memory).  Each of its blocks gets a
        fresh block of `other` (taken from its free list in table order) and
        loses this sequence's reference here; released entries (-1) stay -1.
        Returns the (block here, block there) pairs to copy.  The sequence id
        moves with it.  If `other` lacks free blocks nothing changes."""
        if seq not in self.tables or seq in other.tables:
            raise BlockManagerError("move needs a sequence here and its id free there")
        if other.block_size != self.block_size:
            raise BlockManagerError("pools of different block sizes")
        table = self.tables[seq]
        live = [b for b in table if b >= 0]
        if len(other.free) < len(live):
            raise NoFreeBlocks("destination pool exhausted")
        pairs, new_table = [], []
        for b in table:
            if b < 0:
                new_table.append(-1)
                continue
            nb = other._take()
            pairs.append((b, nb))
            new_table.append(nb)
        other.tables[seq] = new_table
        other.lengths[seq] = self.lengths[seq]
        self.free_seq(seq)
        return pairs

    def slide_window(self, seq: int, window: int) -> int:
        """Release the blocks that hold no token of the last `window` tokens
        ("pagedattention vllm" glossary, "Advanced Features > Sliding Window":
        only recent blocks are kept).  Their table entries become -1; table
        positions do not move.  Returns how many entries were released."""
        if seq not in self.tables or window <= 0:
            raise BlockManagerError("unknown sequence or empty window")
        first = self.lengths[seq] - window
        n = first // self.block_size if first > 0 else 0
        table = self.tables[seq]
        released = 0
        for i in range(min(n, len(table))):
            b = table[i]
            if b < 0:
                continue
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.appendleft(b)
            table[i] = -1
            released += 1
        return released

    def block_table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def seq_len(self, seq: int) -> int:
        return self.lengths[seq]

    def num_free(self) -> int:
        return len(self.free)
