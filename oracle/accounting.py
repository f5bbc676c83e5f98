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
* ``SlabAllocator`` — the layout the pages describe before paging: one
  contiguous run of token slots per request in a pool of fixed size ("Paged
  Attention: Virtual Memory for the KV Cache", §The problem is fragmentation,
  not capacity: the next request also needs one contiguous run; "Paged
  Attention as a Memory Manager", §The KV-Cache Fragmentation Problem: freed
  slabs leave scattered holes that cannot be combined).  The pages name no
  placement rule; the plainest one is taken: first fit (the lowest-addressed
  free run long enough), and a released run merges with free neighbours.
* ``replay_admissions`` — one trace of arrivals and departures replayed
  against a slab pool (reserving the longest context, or the request's own
  length) and against a paged pool of the same token slots, counting
  refusals, refusals while the free total would have covered the request
  (external fragmentation: free memory that is "scattered in pieces, none of
  them large enough"), concurrency and unused reserved room.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

from .block_manager import BlockManagerModel

__all__ = ["reserve_max_waste", "paged_slack", "admit", "SlabAllocator", "replay_admissions"]


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


class SlabAllocator:
    """Contiguous reservations over ``capacity`` token slots, first fit.

    ``holes`` lists the free runs as [start, length], sorted by start, never
    empty and never touching (a released run is merged with the free runs on
    either side)."""

    def __init__(self, capacity: int):
        if capacity < 0:
            raise ValueError("negative capacity")
        self.capacity = int(capacity)
        self.holes: List[List[int]] = [[0, self.capacity]] if capacity else []
        self.runs: Dict[int, Tuple[int, int]] = {}

    def free_slots(self) -> int:
        return sum(length for _, length in self.holes)

    def largest_hole(self) -> int:
        return max((length for _, length in self.holes), default=0)

    def reserve(self, rid: int, n: int) -> Optional[int]:
        """Start of a run of n slots for request rid, or None if no free run
        is long enough (nothing changes then)."""
        if rid in self.runs or n <= 0:
            raise ValueError("request exists or empty reservation")
        for i, (start, length) in enumerate(self.holes):
            if length >= n:
                if length == n:
                    del self.holes[i]
                else:
                    self.holes[i] = [start + n, length - n]
                self.runs[rid] = (start, n)
                return start
        return None

    def release(self, rid: int) -> None:
        start, n = self.runs.pop(rid)
        holes = self.holes
        i = 0
        while i < len(holes) and holes[i][0] < start:
            i += 1
        holes.insert(i, [start, n])
        if i + 1 < len(holes) and holes[i][0] + holes[i][1] == holes[i + 1][0]:
            holes[i][1] += holes[i + 1][1]
            del holes[i + 1]
        if i > 0 and holes[i - 1][0] + holes[i - 1][1] == holes[i][0]:
            holes[i - 1][1] += holes[i][1]
            del holes[i]


def replay_admissions(events: Sequence[tuple], policy: str, capacity_tokens: int, block_size: int,
                      max_len: int) -> dict:
    """Replay ``events`` — ("arrive", rid, length) and ("depart", rid), in
    time order — against one pool of ``capacity_tokens`` slots.

    policy:
      "slab_max"    a contiguous run of max_len slots per request (reserve the
                    longest context at admission);
      "slab_exact"  a contiguous run of the request's own length;
      "paged"       ceil(length / block_size) blocks of a shared free list of
                    capacity_tokens // block_size interchangeable blocks
                    (``BlockManagerModel``), admitted by ``admit`` with no
                    headroom.
    An arrival that cannot be placed is refused (not queued); the departure
    of a refused request is ignored.  After every arrival the live requests
    are sampled.  Returns counts and means:
      admitted, refused,
      refused_with_room   refusals while the free slots covered what the
                          request asks for (external fragmentation),
      peak_live, mean_live,
      reserved_unused     mean over samples of (reserved - used) / reserved,
      used_fraction       mean over samples of used tokens / capacity_tokens.
    """
    if policy not in ("slab_max", "slab_exact", "paged"):
        raise ValueError(policy)
    slab = SlabAllocator(capacity_tokens) if policy != "paged" else None
    bm = BlockManagerModel(capacity_tokens // block_size, block_size) if policy == "paged" else None
    live: Dict[int, int] = {}
    admitted = refused = with_room = peak = 0
    live_sum = unused_sum = used_sum = 0.0
    samples = 0
    for ev in events:
        if ev[0] == "depart":
            rid = int(ev[1])
            if rid in live:
                del live[rid]
                if slab is not None:
                    slab.release(rid)
                else:
                    bm.free_seq(rid)
            continue
        if ev[0] != "arrive":
            raise ValueError(ev[0])
        rid, n = int(ev[1]), int(ev[2])
        if n <= 0 or n > max_len:
            raise ValueError("length outside [1, max_len]")
        if slab is not None:
            ask = max_len if policy == "slab_max" else n
            ok = slab.reserve(rid, ask) is not None
            room = slab.free_slots() >= ask
        else:
            ok = admit(bm.num_free(), n, block_size, 0)
            if ok:
                bm.add_seq(rid, n)
            room = bm.num_free() * block_size >= -(-n // block_size) * block_size
        if ok:
            admitted += 1
            live[rid] = n
        else:
            refused += 1
            with_room += int(room)
        used = sum(live.values())
        if slab is not None:
            reserved = sum(length for _, length in slab.runs.values())
        else:
            reserved = (bm.N - bm.num_free()) * block_size
        peak = max(peak, len(live))
        live_sum += len(live)
        unused_sum += (reserved - used) / reserved if reserved else 0.0
        used_sum += used / capacity_tokens if capacity_tokens else 0.0
        samples += 1
    s = max(samples, 1)
    return {"admitted": admitted, "refused": refused, "refused_with_room": with_room, "peak_live": peak,
            "mean_live": live_sum / s, "reserved_unused": unused_sum / s, "used_fraction": used_sum / s}
