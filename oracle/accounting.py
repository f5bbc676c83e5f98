"""Memory accounting of the two ways of holding a KV cache that the pages
compare — TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``reserve_max_waste`` — the fraction of reserved cache that is never
  touched when every request reserves room for the longest allowed context
  the moment it is admitted and uses only its own length ("Paged Attention as
  a Memory Manager", §The KV-Cache Fragmentation Problem, internal
  fragmentation; "Paged Attention: Virtual Memory for the KV Cache", §The
  problem is fragmentation, not capacity).  Written out from its definition:
  1 - (tokens used) / (requests x reserved length).
* ``paged_slack`` — the unused room when each request holds whole blocks of
  block_size tokens taken one at a time as it grows: only the part of its last
  block past its length ("Paged Attention: Virtual Memory for the KV Cache",
  §The fix borrowed from operating systems: at most one partly filled block
  per request).
* ``admit`` — the admission test of a paged pool: the blocks a request needs
  now plus the headroom kept for the growth of live requests must be free
  (§What it buys in practice: a request is admitted without committing to its
  worst case, and the server knows how close it is to the ceiling).
"""
from __future__ import annotations

from typing import Iterable, Tuple


def reserve_max_waste(lengths: Iterable[int], max_len: int) -> float:
    """Unused fraction of n reservations of max_len tokens holding `lengths`."""
    ls = [int(x) for x in lengths]
    if not ls or max_len <= 0 or any(x < 0 or x > max_len for x in ls):
        raise ValueError("lengths must lie in [0, max_len]")
    return 1.0 - sum(ls) / (len(ls) * max_len)


def paged_slack(lengths: Iterable[int], block_size: int) -> Tuple[int, int]:
    """(unused slots, slots held) when each length holds ceil(len / BS) blocks."""
    held = slack = 0
    for x in lengths:
        blocks = -(-int(x) // block_size)
        held += blocks * block_size
        slack += blocks * block_size - int(x)
    return slack, held


def admit(free_blocks: int, num_tokens: int, block_size: int, reserve_blocks: int) -> bool:
    """Whether a request of num_tokens is admitted with reserve_blocks kept free."""
    need = -(-num_tokens // block_size)
    return need + reserve_blocks <= free_blocks
