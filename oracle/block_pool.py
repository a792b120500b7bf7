"""Plain-Python model of the block pool (test infrastructure only).

spindle ("Paging") describes the allocator: fixed-size blocks handed out from one
pool, each sequence finding its blocks through its own table, so at most the last,
partly filled block of a sequence is wasted; forks share blocks by reference count
(copy-on-write).  The page's worked example: a 16-token parent forked into four
sequences gives them 64 tokens to attend while the pool stores only 16.

Readings where the page is silent:
* the free list is FIFO over a given initial order; freed blocks go to its tail;
* the pool never infers a length: callers name the token range they will
  write (spindle, "Two bugs worth recording"), and the pool makes exactly the
  blocks covering that range present and exclusively owned;
* a write into a block whose reference count is above one first copies it to a
  freshly taken block (the copy is reported to the caller, who moves the data),
  drops one reference from the old block and points the table at the copy.
"""

from __future__ import annotations

from collections import deque


class OutOfBlocks(RuntimeError):
    pass


class BlockPool:
    def __init__(self, num_blocks, block_size=16, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(self.num_blocks) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.free = deque(order)
        self.refcount = [0] * self.num_blocks
        self.tables = {}
        self._next_seq = 0

    # -- sequences ----------------------------------------------------------------
    def add_sequence(self):
        sid = self._next_seq
        self._next_seq += 1
        self.tables[sid] = []
        return sid

    def _take(self):
        if not self.free:
            raise OutOfBlocks("block pool exhausted")
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def _drop(self, b):
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    def prepare_write(self, sid, start, n):
        """Make positions [start, start+n) present and exclusively owned.

        Returns the list of (src, dst) block copies the caller must perform
        before writing.  Positions beyond the table grow it with fresh blocks;
        logical blocks must be filled in order (no holes).
        """
        if n <= 0:
            return []
        table = self.tables[sid]
        bs = self.block_size
        first, last = start // bs, (start + n - 1) // bs
        if first > len(table):
            raise ValueError("write would leave a hole in the block table")
        # All-or-nothing: count what is needed before touching anything.
        need = 0
        for j in range(first, last + 1):
            if j >= len(table) or self.refcount[table[j]] > 1:
                need += 1
        if need > len(self.free):
            raise OutOfBlocks("block pool exhausted")
        copies = []
        for j in range(first, last + 1):
            if j >= len(table):
                table.append(self._take())
            elif self.refcount[table[j]] > 1:
                old = table[j]
                new = self._take()
                copies.append((old, new))
                self._drop(old)
                table[j] = new
        return copies

    def fork(self, parent):
        """New sequence sharing every block of ``parent`` (reference counts +1)."""
        child = self.add_sequence()
        self.tables[child] = list(self.tables[parent])
        for b in self.tables[child]:
            self.refcount[b] += 1
        return child

    def free_sequence(self, sid):
        for b in self.tables.pop(sid):
            self._drop(b)

    # -- views --------------------------------------------------------------------
    def table(self, sid):
        return list(self.tables[sid])

    def num_free(self):
        return len(self.free)

    def physical_in_use(self):
        return sum(1 for r in self.refcount if r > 0)
