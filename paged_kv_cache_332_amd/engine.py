"""Host runtime around libpa: one layer's K/V pools, the block manager and the
device copies of its bookkeeping, driven one decode step at a time.

A decode step is: the block manager hands each sequence a slot for its new
token (taking a block when the last is full, or copying a shared last block
first); the copy pairs, slots, tables and context lengths go to the device
through pinned staging buffers on the compute stream; then pa_copy_blocks,
pa_write_kv and pa_decode (partition pass + log-sum-exp merge) run on that
stream.  Staging buffers rotate through a small ring guarded by events so the
host can prepare step k+1 while the device still reads step k's copy.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import (PA_KERNEL_AUTO, PA_KERNEL_STREAM, STEP_ALL, BlockManager, alloc_cache, pa_copy_blocks, pa_decode_stream_grid,
               pa_decode_variant, pa_decode_workspace_bytes, pa_step_layer, pa_write_kv, step_args, step_call,
               step_record_words, stream_class_finish)

__all__ = ["PagedKVEngine", "rebalance"]


_MAX_GRID = 1024     # the most workgroups the stream kernel launches


XCDS = 8     # accelerator dies of the GPU; workgroup b of a launch runs on die b mod 8
# Where the feedback starts: the even dies sustain about 10% more of the
# stream pass than the odd ones.  Learned weights after 200 steps put them at
# 1065-1105 against 943-1006 in every run on every MI355X measured (about 30
# runs, many boxes); starting there instead of at equal shares saves the
# feedback the first dozens of steps.  The feedback still corrects any box.
DIE_PRIOR = np.array([1075, 973] * (XCDS // 2), dtype=np.int32)


def class_finish(stamps: np.ndarray, g: int, groups: int = XCDS) -> np.ndarray:
    """Mean finish time of each class of workgroups (index modulo ``groups``)
    in one completed step.  ``stamps`` holds, for the 4 waves of each of the
    ``g`` workgroups in order, the start and end of the wave (low 32 bits of
    a 100 MHz counter); a workgroup's finish counts from the first start of
    any wave to the last end of its own."""
    t = np.asarray(stamps[: 8 * g], dtype=np.int64).reshape(g, 4, 2)
    rel = (t - t[0, 0, 0] + (1 << 31)) % (1 << 32) - (1 << 31)      # signed 32-bit differences
    finish = (rel[:, :, 1].max(axis=1) - rel[:, :, 0].min()).astype(np.float64)
    cls = np.arange(g) % groups
    cnt = np.bincount(cls, minlength=groups)
    return np.bincount(cls, weights=finish, minlength=groups) / np.maximum(cnt, 1)


def rebalance_classes(weights: np.ndarray, mean_c: np.ndarray, rate: float = 0.5,
                      groups: int = XCDS) -> np.ndarray:
    """New weights from class finish times (see rebalance)."""
    g = weights.shape[0]
    cls = np.arange(g) % groups
    cnt = np.bincount(cls, minlength=groups)
    w_c = np.bincount(cls, weights=weights.astype(np.float64), minlength=groups) / np.maximum(cnt, 1)
    target = np.maximum(mean_c[cnt > 0].mean(), 1.0)
    f = w_c * (target / np.maximum(mean_c, 1.0)) ** rate
    f = f[cls]
    f *= 1024.0 / f.mean()
    return np.clip(np.rint(f), 64, 16384).astype(np.int32)


def rebalance(weights: np.ndarray, stamps: np.ndarray, rate: float = 0.5, groups: int = XCDS) -> np.ndarray:
    """New stream-kernel workgroup weights from one completed step.

    Workgroups are pooled in ``groups`` classes by index modulo ``groups``
    (the dies workgroups are dispatched to in turn, which run at measurably
    different speeds; single workgroups only add noise).  Each class's weight
    (its share of the tile list) moves towards what would have let it finish
    with the others, w <- w * (mean / class mean) ** rate; the result is
    scaled to a mean of 1024 and kept within 64..16384.  The weights move
    where items are cut between waves, so the decode's results change with
    them in the last bits (fp32 rounding of a different summation order);
    an engine with ``balance=False`` keeps equal shares and gives the same
    bits on every run."""
    return rebalance_classes(weights, class_finish(stamps, weights.shape[0], groups), rate, groups)


class _Staging:
    """One step's bookkeeping in a single pinned host buffer and its device
    mirror, laid out [slots B | copy pairs 2B | context lengths B | tables
    B x stride | tile prefix sums B + 1 | stream plan], so a whole step
    needs one host-to-device copy; plus a pinned buffer the stream kernel
    writes its wave start/end stamps into."""

    def __init__(self, max_seqs: int, stride: int, num_kv_heads: int, device):
        self.stride = stride
        self.max_seqs = max_seqs
        words = step_record_words(max_seqs, stride, num_kv_heads)
        # zero-filled: every page of the pinned record is touched here, not by
        # the first step that uses the record (which measured 40-55 us more on
        # the host, while the GPU waited for it)
        self.h = torch.zeros(words, dtype=torch.int32, pin_memory=True)
        self.d = torch.empty(words, dtype=torch.int32, device=device)
        self.h_slots, self.h_pairs, self.h_ctx, self.h_tables = self._views(self.h, max_seqs)
        self.d_slots, self.d_pairs, self.d_ctx, self.d_tables = self._views(self.d, max_seqs)
        self.times = torch.zeros(8 * _MAX_GRID, dtype=torch.int32, pin_memory=True)
        self.times_key = None     # (balance key, weight version) of the step whose stamps `times` holds
        self.event: Optional[torch.cuda.Event] = None
        self.h_ptr, self.d_ptr, self.t_ptr = self.h.data_ptr(), self.d.data_ptr(), self.times.data_ptr()
        self.words = min(self.h.numel(), self.d.numel())

    def _views(self, t, b):
        s = self.stride
        return (t[:b], t[b:3 * b].view(b, 2), t[3 * b:4 * b], t[4 * b:4 * b + b * s].view(b, s))

    def packed(self, n):
        """Views of an n-sequence step, packed at the front of both buffers:
        (host, device) x (slots, pairs, ctx, tables)."""
        h = self._views(self.h, n)
        d = self._views(self.d, n)
        return h, d, 4 * n + n * self.stride

    def wait(self):
        if self.event is not None:
            self.event.synchronize()


class PagedKVEngine:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, dtype,
                 order: Optional[Sequence[int]] = None, device: str = "cuda", poison: bool = True,
                 max_seqs: int = 256, max_context: int = 4096, ring: int = 8, guard_every: int = 4,
                 balance: bool = True, balance_rate: float = 0.2, balance_steps: int = 8):
        self.N, self.H, self.D, self.BS, self.dtype = num_blocks, num_kv_heads, head_dim, block_size, dtype
        self.device = torch.device(device)
        self.bm = BlockManager(num_blocks, block_size, order)
        self.k_cache, self.v_cache = alloc_cache(num_blocks, num_kv_heads, head_dim, block_size, dtype,
                                                 device=self.device, poison=poison)
        self.max_seqs = max_seqs
        self.stride = -(-max_context // block_size)
        self._ring = [_Staging(max_seqs, self.stride, num_kv_heads, self.device) for _ in range(ring)]
        self._ri = 0
        # an event packet between kernels costs the stream ~4 us, so only every
        # guard_every-th record is guarded; a slot is reused ring records later,
        # so the host waits on the newest guard at least ring - guard_every back
        assert 1 <= guard_every <= ring // 2
        self._guard_every = guard_every
        self._uses = 0
        self._pending = []
        self._ws = torch.empty(0, dtype=torch.uint8, device=self.device)
        # workgroup weights of the stream kernel per (batch size, query heads),
        # fed back from the wave stamps of completed steps (see _balance)
        self.balance, self.balance_rate, self.balance_steps = balance, balance_rate, balance_steps
        self._weights = {}
        self._wver = {}
        self._wacc = {}
        self._finish = np.zeros(XCDS)
        # guard events, reused in turn: a guard is recorded again only after
        # every slot it covered has been reused (and waited on)
        self._guards = []
        self._gi = 0
        self._call_key = None
        self._last_view = None

    # ------------------------------------------------------------- helpers
    def _next(self) -> _Staging:
        """The next staging record; returns once no queued work reads it."""
        st = self._ring[self._ri]
        self._ri = (self._ri + 1) % len(self._ring)
        # the guard recorded after this slot's last use, or after a later one
        # of the previous lap, has completed before the slot is rewritten
        st.wait()
        if st.times_key is not None:
            self._balance(st)
        return st

    def _balance(self, st: _Staging) -> None:
        """Feedback from completed steps (see rebalance).  Stamps arrive a
        ring's length of steps late, so only steps that ran with the current
        weights count: feedback from older weights would correct the same
        error again and make the loop oscillate.  A die's speed also varies
        from step to step, so the class finish times of ``balance_steps``
        such steps are averaged before one update."""
        (key, version), st.times_key = st.times_key, None
        w = self._weights.get(key)
        if w is None or version != self._wver.get(key):
            return
        acc = self._wacc.get(key)
        if acc is None or acc[0] != version:
            acc = self._wacc[key] = [version, np.zeros(XCDS), 0]
        acc[1] += stream_class_finish(st.t_ptr, w.shape[0], XCDS, self._finish)
        acc[2] += 1
        if acc[2] >= self.balance_steps:
            w[:] = rebalance_classes(w, acc[1] / acc[2], self.balance_rate)
            self._wver[key] = version + 1

    def weights(self, num_seqs: int, num_q_heads: int) -> Optional[np.ndarray]:
        """The stream kernel's workgroup weights for this shape (None when the
        stream kernel is not used or balancing is off)."""
        if not self.balance or self.dtype == torch.float32:
            return None
        key = (num_seqs, num_q_heads)
        w = self._weights.get(key)
        if w is None:
            g = pa_decode_stream_grid(num_seqs, num_q_heads, self.H, self.D)
            if g <= 0:
                return None
            w = self._weights[key] = DIE_PRIOR[np.arange(g) % XCDS].copy()
            self._wver[key] = 0
        return w

    def _record(self, st: _Staging, stream):
        """Guard the records used so far: every guard_every-th use records an
        event on the stream and hands it to the slots of the last
        guard_every uses (they are reused only after it completes)."""
        self._uses += 1
        self._pending.append(st)
        if self._uses % self._guard_every:
            return      # the slot keeps its previous guard until the next one is recorded
        if len(self._guards) < 4:
            self._guards.append(torch.cuda.Event())
        ev = self._guards[self._gi % len(self._guards)]
        self._gi += 1
        ev.record(stream)
        for p in self._pending:
            p.event = ev
        self._pending = []

    def workspace(self, num_seqs: int, num_q_heads: int, max_ctx: int, partition_size: int = 0):
        """Decode workspace, grown on demand and reused across calls."""
        key = (num_seqs, num_q_heads, max_ctx, partition_size)
        if getattr(self, "_ws_key", None) != key:
            need = pa_decode_workspace_bytes(num_seqs, num_q_heads, self.H, self.D, max_ctx, partition_size)
            if need > self._ws.numel():
                self._ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            self._ws_key = key
        return self._ws

    # ----------------------------------------------------------- sequences
    def add_seq(self, seq: int, k_rows: Optional[torch.Tensor], v_rows: Optional[torch.Tensor], n: int,
                stream=None) -> np.ndarray:
        """New sequence of n tokens; writes their K/V rows ([n][Hkv][D], device) if given."""
        slots = self.bm.add_seq(seq, n)
        if k_rows is not None and n:
            d_slots = torch.from_numpy(slots).to(self.device, non_blocking=False)
            pa_write_kv(self.k_cache, self.v_cache, k_rows, v_rows, d_slots, stream=stream)
        return slots

    def fork(self, parent: int, child: int) -> None:
        self.bm.fork(parent, child)

    def free_seq(self, seq: int) -> None:
        self.bm.free_seq(seq)

    def append(self, seqs: Sequence[int], k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        """One token per sequence: copy-on-write copies, then the K/V write."""
        stream = stream or torch.cuda.current_stream()
        n = len(seqs)
        st = self._next()
        slots, pairs = self.bm.append_slots(seqs)
        st.h_slots[:n].numpy()[:] = slots
        st.d_slots[:n].copy_(st.h_slots[:n], non_blocking=True)
        if len(pairs):
            st.h_pairs[: len(pairs)].numpy()[:] = pairs
            st.d_pairs[: len(pairs)].copy_(st.h_pairs[: len(pairs)], non_blocking=True)
            pa_copy_blocks(self.k_cache, self.v_cache, st.d_pairs[: len(pairs)], stream=stream)
        pa_write_kv(self.k_cache, self.v_cache, k_new, v_new, st.d_slots[:n], stream=stream)
        self._record(st, stream)
        return slots, pairs

    def export(self, seqs: Sequence[int]):
        st = self._next()
        n = len(seqs)
        tab, ctx = self.bm.export(seqs, self.stride, st.h_tables[:n].numpy(), st.h_ctx[:n].numpy())
        return st, tab, ctx

    def decode(self, seqs: Sequence[int], q: torch.Tensor, out: Optional[torch.Tensor] = None,
               out_dtype=torch.float32, partition_size: int = 0, kernel: int = PA_KERNEL_AUTO,
               stream=None) -> torch.Tensor:
        """Attention of q [n][Hq][D] over each listed sequence's whole context."""
        stream = stream or torch.cuda.current_stream()
        n = len(seqs)
        st, tab, ctx = self.export(seqs)
        self._last_view = (tab, ctx)      # views of the pinned staging buffers
        max_ctx = int(ctx.max()) if n else 0
        st.d_tables[:n].copy_(st.h_tables[:n], non_blocking=True)
        st.d_ctx[:n].copy_(st.h_ctx[:n], non_blocking=True)
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=self.device)
        ws = self.workspace(n, q.shape[1], max_ctx, partition_size)
        pa_decode_variant(out, q, self.k_cache, self.v_cache, st.d_tables[:n], st.d_ctx[:n], max_ctx,
                          1.0 / float(self.D) ** 0.5, partition_size, ws if ws.numel() else None,
                          stream=stream, kernel=kernel)
        self._record(st, stream)
        return out

    def step(self, seqs, k_new, v_new, q, out=None, out_dtype=torch.float32, partition_size: int = 0,
             kernel: int = PA_KERNEL_AUTO, stream=None, pass_events=None) -> torch.Tensor:
        """One decode step for the listed sequences, in one native call
        (pa_step): the block manager gives each its new token's slot
        (copy-on-write pairs first), the slots, pairs, context lengths and
        block tables go to the device in one copy, then pa_copy_blocks,
        pa_write_kv and the decode pass and merge run on the stream.
        ``pass_events`` = (start, end) CUDA events (already created) recorded
        around the decode pass."""
        stream = stream or torch.cuda.current_stream()
        n = len(seqs)
        st = self._next()
        key = tuple(seqs)
        if getattr(self, "_seq_key", None) != key:
            self._seq_key, self._seq_arr = key, np.ascontiguousarray(seqs, dtype=np.int64)
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=self.device)
        # the workspace is sized for the longest context the tables can hold
        ws = self.workspace(n, q.shape[1], self.stride * self.BS, partition_size)
        w = self.weights(n, q.shape[1]) if kernel in (PA_KERNEL_AUTO, PA_KERNEL_STREAM) else None
        # one argument list per step shape; per step only the record, the
        # events and the stamps change
        call_key = (key, k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), out.data_ptr(), out.dtype, q.shape[1],
                    partition_size, kernel, stream if isinstance(stream, int) else stream.cuda_stream, ws.data_ptr(),
                    ws.numel(), id(w))
        if call_key != self._call_key:
            self._call_args = step_args(self.bm, self._seq_arr, self.stride, self.k_cache, self.v_cache, k_new, v_new,
                                        q, out, 1.0 / float(self.D) ** 0.5, partition_size,
                                        ws if ws.numel() else None, kernel, stream, w)
            self._call_key, self._call_w = call_key, w
        args = self._call_args
        args[3], args[4], args[5] = st.h_ptr, st.d_ptr, st.words
        args[26], args[27] = (None, None) if pass_events is None else (pass_events[0].cuda_event,
                                                                       pass_events[1].cuda_event)
        args[31] = None if w is None else st.t_ptr
        max_ctx = step_call(args)
        st.times_key = None if w is None else ((n, q.shape[1]), self._wver[(n, q.shape[1])])
        self._last_view = (st, n)
        self.last_max_ctx = max_ctx
        self._last = (st, n, kernel, partition_size)
        self._record(st, stream)
        return out

    @property
    def last_tables(self) -> np.ndarray:
        """Block tables of the last step or decode ([n][stride], views of the
        pinned record)."""
        return self._last_tc()[0]

    @property
    def last_ctx(self) -> np.ndarray:
        return self._last_tc()[1]

    def _last_tc(self):
        v = self._last_view
        if v is not None and isinstance(v[0], _Staging):
            (hs, hp, hc, ht), _, _ = v[0].packed(v[1])
            return ht.numpy(), hc.numpy()
        return v

    def step_layer(self, k_cache, v_cache, k_new, v_new, q, out, phases: int = STEP_ALL, stream=None,
                   pass_events=None) -> torch.Tensor:
        """The device part of the last step again for another layer: its own
        pools (shaped like this engine's), new keys/values, queries and output,
        on the same sequences, slots, tables and split.  Must come before the
        next step() (which may reuse the record)."""
        stream = stream or torch.cuda.current_stream()
        st, n, kernel, partition_size = self._last
        ws = self.workspace(n, q.shape[1], self.stride * self.BS, partition_size)
        pa_step_layer(st.h, st.d, n, self.stride, k_cache, v_cache, k_new, v_new, q, out, 1.0 / float(self.D) ** 0.5,
                      partition_size, ws if ws.numel() else None, kernel, stream, phases, pass_events)
        return out
