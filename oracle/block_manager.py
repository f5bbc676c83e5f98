"""Block-manager model (oracle; test infrastructure only).

What the pages fix ("Paged Attention: Virtual Memory for the KV Cache",
§The fix borrowed from operating systems and §Sharing comes almost for free;
"Paged Attention as a Memory Manager", §Virtual Memory as the Blueprint and
§How the Kernel Executes Paged Attention; glossary "What is Paged
Attention?"):

* the cache is split into fixed-size blocks that are all interchangeable and
  live in one shared pool (a free list);
* each request keeps a block table, an ordered list of physical block ids; at
  prefill logical blocks are numbered in order and blocks come from the free
  list on demand;
* a request takes a new block only when its last one is full, and gives all of
  them back the moment it finishes;
* several tables may reference one physical block (prefix sharing); a sharer
  about to write into a shared block first gets its own copy (copy-on-write).

Policy fixed here where the pages are silent (the C++ allocator follows the
same written policy, so integer results are unique):

* free list = LIFO stack; a new pool is stacked so that the first allocation
  returns ``order[0]`` (identity when no order is given);
* ``add_seq(n)`` takes ceil(n / BS) blocks in logical order;
  slot(t) = table[t // BS] * BS + t % BS;
* ``append`` at position pos = len: if pos % BS == 0 a fresh block is taken;
  otherwise, if the last block is shared (refcount > 1), a fresh block is
  taken, the last block's refcount drops by one, the table points at the fresh
  block and the pair (old, fresh) is reported for a whole-block copy; the last
  remaining sharer (refcount 1) writes in place.  Batched appends run in list
  order;
* ``fork`` copies the parent's table and raises every block's refcount;
* ``free_seq`` drops refcounts in logical order and pushes a block the moment
  its count reaches zero;
* a call that cannot get the blocks it needs raises ``OutOfBlocks`` and
  changes nothing; unknown or duplicate sequence ids raise ``InvalidOp`` and
  change nothing.

Preemption by swap ("Paged Attention: Virtual Memory for the KV Cache",
§What it does not fix: once memory runs out a sequence must be evicted, its
blocks moved off the device and brought back later):

* ``swap_out`` releases the sequence's blocks exactly like ``free_seq`` and
  keeps its length; it returns the table (logical order) so the caller can
  copy the blocks to host memory before anything reuses them;
* ``swap_in`` takes ceil(len / BS) fresh blocks in logical order (all or
  nothing) for the copy back; a block that was shared comes back private;
* a swapped-out id is neither live nor free: ``add_seq`` and ``fork`` reject
  it, and only ``swap_in`` brings it back.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["BlockManagerModel", "OutOfBlocks", "InvalidOp"]


class OutOfBlocks(Exception):
    pass


class InvalidOp(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, order: Optional[Sequence[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise InvalidOp("bad pool")
        if order is None:
            order = range(num_blocks)
        order = [int(b) for b in order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidOp("order must be a permutation of the block ids")
        self.N = num_blocks
        self.BS = block_size
        self.free: List[int] = list(reversed(order))   # top of stack = end
        self.rc = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.swapped: Dict[int, int] = {}
        self.cow_count = 0

    # -- queries -------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        return self.rc[block]

    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lens[seq]

    def slot(self, seq: int, pos: int) -> int:
        t = self.tables[seq]
        return t[pos // self.BS] * self.BS + pos % self.BS

    def stats(self) -> Tuple[int, int, int, int, int]:
        """(free, used, shared, cow_count, waste_tokens); waste is each
        sequence's unused room in its last block."""
        used = sum(1 for c in self.rc if c > 0)
        shared = sum(1 for c in self.rc if c > 1)
        waste = sum(len(self.tables[s]) * self.BS - self.lens[s] for s in self.tables)
        return len(self.free), used, shared, self.cow_count, waste

    # -- operations ----------------------------------------------------------
    def _pop(self) -> int:
        b = self.free.pop()
        self.rc[b] = 1
        return b

    def add_seq(self, seq: int, n: int) -> List[int]:
        if seq in self.tables or seq in self.swapped or n < 0:
            raise InvalidOp("sequence exists or negative length")
        need = -(-n // self.BS)
        if need > len(self.free):
            raise OutOfBlocks()
        self.tables[seq] = [self._pop() for _ in range(need)]
        self.lens[seq] = n
        return [self.slot(seq, t) for t in range(n)]

    def append(self, seqs: Sequence[int]):
        """One token for each listed sequence.  Returns (slots, cow_pairs)."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs) or any(s not in self.tables for s in seqs):
            raise InvalidOp("unknown or repeated sequence")
        # dry run: count the fresh blocks this batch takes
        rc = {}
        need = 0
        for s in seqs:
            pos = self.lens[s]
            if pos % self.BS == 0:
                need += 1
            else:
                last = self.tables[s][-1]
                c = rc.get(last, self.rc[last])
                if c > 1:
                    need += 1
                    rc[last] = c - 1
        if need > len(self.free):
            raise OutOfBlocks()
        slots, pairs = [], []
        for s in seqs:
            pos = self.lens[s]
            t = self.tables[s]
            if pos % self.BS == 0:
                t.append(self._pop())
            elif self.rc[t[-1]] > 1:
                old = t[-1]
                nb = self._pop()
                self.rc[old] -= 1
                t[-1] = nb
                pairs.append((old, nb))
                self.cow_count += 1
            slots.append(self.slot(s, pos))
            self.lens[s] = pos + 1
        return slots, pairs

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables or child in self.tables or child in self.swapped:
            raise InvalidOp("bad fork")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.rc[b] += 1

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise InvalidOp("unknown sequence")
        for b in self.tables.pop(seq):
            self.rc[b] -= 1
            if self.rc[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    def swap_out(self, seq: int) -> List[int]:
        if seq not in self.tables:
            raise InvalidOp("unknown sequence")
        table = list(self.tables[seq])
        self.swapped[seq] = self.lens[seq]
        self.free_seq(seq)
        return table

    def swap_in(self, seq: int) -> List[int]:
        if seq not in self.swapped:
            raise InvalidOp("not swapped out")
        n = self.swapped[seq]
        need = -(-n // self.BS)
        if need > len(self.free):
            raise OutOfBlocks()
        del self.swapped[seq]
        self.tables[seq] = [self._pop() for _ in range(need)]
        self.lens[seq] = n
        return list(self.tables[seq])

    def swapped_len(self, seq: int) -> int:
        return self.swapped.get(seq, -1)

    def export(self, seqs: Sequence[int], stride: int):
        """int32 tables [n][stride] padded with -1, int32 context lengths [n]."""
        seqs = [int(s) for s in seqs]
        tab = np.full((len(seqs), stride), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            if s not in self.tables:
                raise InvalidOp("unknown sequence")
            t = self.tables[s]
            if len(t) > stride:
                raise InvalidOp("table longer than stride")
            tab[i, :len(t)] = t
            lens[i] = self.lens[s]
        return tab, lens
