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

Prefix caching across requests ("Paged Attention: Virtual Memory for the KV
Cache", §Sharing comes almost for free and §Why this matters…: a prompt
prefix that many requests share is stored once and reused; the pages give no
keying or eviction rule, the readings below are this model's):

* a full block of a sequence added with its token ids is cached under the key
  (content id of the previous block, the block's BS token ids); the first
  block's parent is content id 0 and every newly cached block gets the next
  content id, so a key names the whole prefix up to the block's end, exactly
  (no hash is trusted);
* ``add_seq_cached(seq, tokens)`` walks the prompt's full blocks from the start
  and reuses every block found, stopping at the first miss and never reusing
  the block that holds the last token (at least one token is computed); it
  returns the slots of all tokens and the number of reused tokens, whose K/V
  the caller does not write again;
* fresh full blocks of such a sequence are cached at once (the caller writes
  their K/V on the stream before anything reads them); a key already cached
  is not cached twice;
* a cached block whose count drops to zero is not freed but becomes evictable,
  in least-recently-released order; a sequence's blocks are released from its
  last block to its first, so the end of a prefix is evicted before its start;
* a fresh block comes from the free stack, and only when it is empty from the
  evictable list (the oldest first, dropping its key); the blocks a call can
  get are the free ones plus the evictable ones it does not itself reuse.
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
        # prefix cache
        self.cache: Dict[Tuple[int, Tuple[int, ...]], Tuple[int, int]] = {}   # key -> (content id, block)
        self.block_key: Dict[int, Tuple[int, Tuple[int, ...]]] = {}
        self.evictable: List[int] = []                                       # oldest first
        self.next_cid = 1
        self.hit_blocks = 0
        self.query_blocks = 0

    # -- queries -------------------------------------------------------------
    def num_free(self) -> int:
        """Blocks a call can get: the free stack plus the evictable cached blocks."""
        return len(self.free) + len(self.evictable)

    def cache_stats(self) -> Tuple[int, int, int, int]:
        """(cached blocks, evictable blocks, reused blocks so far, full
        blocks looked up so far)."""
        return len(self.block_key), len(self.evictable), self.hit_blocks, self.query_blocks

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
        return self.num_free(), used, shared, self.cow_count, waste

    # -- operations ----------------------------------------------------------
    def _pop(self) -> int:
        if self.free:
            b = self.free.pop()
        else:
            b = self.evictable.pop(0)
            del self.cache[self.block_key.pop(b)]
        self.rc[b] = 1
        return b

    def _release(self, table: Sequence[int]) -> None:
        """Drop one reference of each block, in logical order; a block that
        reaches zero goes on the free stack, or, if cached, becomes evictable
        (the sequence's cached blocks in reverse logical order)."""
        cached = []
        for b in table:
            self.rc[b] -= 1
            if self.rc[b] == 0:
                if b in self.block_key:
                    cached.append(b)
                else:
                    self.free.append(b)
        self.evictable.extend(reversed(cached))

    def add_seq(self, seq: int, n: int) -> List[int]:
        if seq in self.tables or seq in self.swapped or n < 0:
            raise InvalidOp("sequence exists or negative length")
        need = -(-n // self.BS)
        if need > self.num_free():
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
        if need > self.num_free():
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
        self._release(self.tables.pop(seq))
        del self.lens[seq]

    def add_seq_cached(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], int]:
        """add_seq with the prompt's token ids: reuses cached full blocks of
        its prefix.  Returns (slots of all tokens, reused tokens)."""
        tokens = [int(t) for t in tokens]
        if seq in self.tables or seq in self.swapped:
            raise InvalidOp("sequence exists")
        n, BS = len(tokens), self.BS
        nb = -(-n // BS)
        full = n // BS
        lookable = (n - 1) // BS if n else 0          # the block of the last token is computed
        parent, hits = 0, []
        for i in range(lookable):
            key = (parent, tuple(tokens[i * BS:(i + 1) * BS]))
            if key not in self.cache:
                break
            parent, b = self.cache[key]
            hits.append(b)
        revived = sum(1 for b in hits if self.rc[b] == 0)
        if nb - len(hits) > self.num_free() - revived:
            raise OutOfBlocks()
        self.query_blocks += lookable
        self.hit_blocks += len(hits)
        for b in hits:
            if self.rc[b] == 0:
                self.evictable.remove(b)
            self.rc[b] += 1
        table = list(hits)
        for i in range(len(hits), nb):
            b = self._pop()
            table.append(b)
            if i < full:
                key = (parent, tuple(tokens[i * BS:(i + 1) * BS]))
                if key in self.cache:
                    parent = self.cache[key][0]
                else:
                    cid = self.next_cid
                    self.next_cid += 1
                    self.cache[key] = (cid, b)
                    self.block_key[b] = key
                    parent = cid
        self.tables[seq] = table
        self.lens[seq] = n
        return [self.slot(seq, t) for t in range(n)], len(hits) * BS

    def cache_clear(self) -> None:
        """Forget every cached prefix; evictable blocks go on the free stack,
        oldest first."""
        self.free.extend(self.evictable)
        self.evictable = []
        self.cache.clear()
        self.block_key.clear()

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
        if need > self.num_free():
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
