"""Seeded synthetic workloads for paged-attention decode.

This module is shared by the HIP path's tests/bench and by the CPU oracle.  It
holds only *inputs*: configuration shapes, seeded random draws (context
lengths, pool orders, churn decisions, K/V/Q values rounded to the storage
dtype) and each configuration's construction script as a flat list of
block-manager operations.  It contains none of the method's arithmetic: no
block allocation policy, no cache layout, no attention.  Each consumer
interprets the script with its own block manager and its own cache.

Workload shapes follow the five decode configurations of the paged-attention
pages' target workload family (tiny fp32 MHA, batch-64 GQA bf16 with a block
size sweep, 13B-like MHA fp16 after allocator churn, prefix sharing with
copy-on-write, long-context split-K).  Where the configuration text leaves a
step open, the reading taken here is stated next to the code.

Seeds: configuration k uses ``numpy.random.default_rng([1000 + k, s])`` with
stream s = 0 (context lengths), 1 (pool order / churn), 2 (K), 3 (V), 4 (Q);
the admission trace uses streams 5 (request lengths) and 6 (lifetimes) of
the 13B-like configuration.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "Workload", "build", "round_to_dtype",
    "ELEM_BYTES", "admission_trace",
]

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
TEMP_SEQ_BASE = 1 << 40  # ids of the single-block sequences used by the churn


@dataclass(frozen=True)
class Config:
    name: str
    index: int            # k of the seed formula (1..5)
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str            # "f32" | "f16" | "bf16"
    partition_size: int = 0   # 0 = let the library choose
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    c.name: c for c in [
        Config("c1_tiny_f32", 1, 4, 8, 8, 64, 16, "f32",
               description="4 seqs ctx {17,64,100,255}, 8/8 heads, D64, BS16, fp32, 64-block pool"),
        Config("c2_gqa_bf16_bs8", 2, 64, 32, 8, 128, 8, "bf16",
               description="batch 64, 32q/8kv, D128, BS8, bf16, ctx U[128,4096]"),
        Config("c2_gqa_bf16", 2, 64, 32, 8, 128, 16, "bf16",
               description="batch 64, 32q/8kv, D128, BS16, bf16, ctx U[128,4096]"),
        Config("c2_gqa_bf16_bs32", 2, 64, 32, 8, 128, 32, "bf16",
               description="batch 64, 32q/8kv, D128, BS32, bf16, ctx U[128,4096]"),
        Config("c3_mha_f16_churn", 3, 256, 40, 40, 128, 16, "f16",
               description="batch 256, 40 MHA heads, D128, BS16, fp16, lognormal ctx, 10k-step churn"),
        Config("c4a_prefix_share", 4, 64, 32, 8, 128, 16, "bf16",
               description="64 seqs share a 2048-token prefix (rc 64) + U[1,512] suffixes"),
        Config("c4b_prefix_cow", 4, 64, 32, 8, 128, 16, "bf16",
               description="64 seqs share a 2040-token prefix; first append COW-copies the partial block"),
        Config("c5_long_splitk", 5, 8, 64, 8, 128, 32, "bf16", partition_size=512,
               description="batch 8, ctx U[32768,131072], 64q/8kv, D128, BS32, 512-token split-K"),
    ]
}


def config(name: str) -> Config:
    return CONFIGS[name]


def _rng(k: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([1000 + k, stream])


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (round to nearest even) and
    return them as float32 again, so every value is exactly representable in
    ``dtype``.  bf16 uses the usual carry trick on the fp32 bit pattern
    (numpy has no bf16); inputs are finite normal draws."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        bits = x.view(np.uint32)
        lsb = (bits >> np.uint32(16)) & np.uint32(1)
        out = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
        return out.view(np.float32)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# construction scripts
#
# An op is a tuple:
#   ("create", num_blocks, order or None)   pool of num_blocks; the first
#                                            allocation returns order[0]
#   ("add_seq", seq, n_tokens, write)      new sequence holding n_tokens; if
#                                            write, its tokens' K/V are written
#   ("fork", parent, child)
#   ("free_seq", seq)
#   ("append", [seq, ...])                  one new token per listed sequence,
#                                            in list order; its K/V is written
#   ("decode", [seq, ...], q_index)         attention for the listed sequences
#                                            with query set q_index
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    cfg: Config
    ctx: np.ndarray                      # final context length per sequence (int64)
    k_rows: np.ndarray                   # [R, Hkv, D] float32, values exact in dtype
    v_rows: np.ndarray                   # [R, Hkv, D]
    q_sets: List[np.ndarray]             # each [B, Hq, D] float32, exact in dtype
    ops: List[tuple]
    num_blocks: int
    # row index of token t of sequence i is row_start[i] + t, except for the
    # shared prefix of the prefix-sharing workloads (see row_of)
    row_start: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    prefix_len: int = 0

    def row_of(self, seq: int, positions: np.ndarray) -> np.ndarray:
        """Row indices into k_rows/v_rows for positions of logical sequence seq."""
        positions = np.asarray(positions, dtype=np.int64)
        if self.prefix_len:
            return np.where(positions < self.prefix_len, positions,
                            self.row_start[seq] + positions - self.prefix_len)
        return self.row_start[seq] + positions


def _ceil_div(a, b):
    return -(-np.asarray(a) // b)


_KV_MEMO: dict = {}


def _draw_kv(cfg: Config, rows: int, k_scale: float = 1.0):
    # the block-size sweep shares its draws: keep the last one
    key = (cfg.index, rows, cfg.num_kv_heads, cfg.head_dim, cfg.dtype, k_scale)
    if key in _KV_MEMO:
        return _KV_MEMO[key]
    _KV_MEMO.clear()
    _KV_MEMO[key] = _draw_kv_uncached(cfg, rows, k_scale)
    return _KV_MEMO[key]


def _draw_kv_uncached(cfg: Config, rows: int, k_scale: float = 1.0):
    shape = (rows, cfg.num_kv_heads, cfg.head_dim)
    k = _rng(cfg.index, 2).standard_normal(shape, dtype=np.float32)
    if k_scale != 1.0:
        k *= np.float32(k_scale)          # power of two: exact in fp32
    k = round_to_dtype(k, cfg.dtype)
    v = round_to_dtype(_rng(cfg.index, 3).standard_normal(shape, dtype=np.float32), cfg.dtype)
    return k, v


def _draw_q(cfg: Config, count: int = 1):
    r = _rng(cfg.index, 4)
    return [round_to_dtype(r.standard_normal((cfg.num_seqs, cfg.num_q_heads, cfg.head_dim),
                                             dtype=np.float32), cfg.dtype)
            for _ in range(count)]


def _prefill_then_decode(ctx: np.ndarray) -> List[tuple]:
    """Prefill ctx-1 tokens per sequence (index order), then one decode step
    that appends the last token of every sequence and attends over all ctx
    tokens (the context length counts the token written in the step)."""
    B = len(ctx)
    ops = [("add_seq", i, int(ctx[i]) - 1, True) for i in range(B)]
    ops.append(("append", list(range(B))))
    ops.append(("decode", list(range(B)), 0))
    return ops


def _pool_size(ctx: np.ndarray, bs: int) -> int:
    need = int(_ceil_div(ctx, bs).sum())
    return int(math.ceil(1.2 * need))


def _ctx_c1():
    return np.array([17, 64, 100, 255], dtype=np.int64)


def _ctx_c2():
    return _rng(2, 0).integers(128, 4097, size=64).astype(np.int64)


def _ctx_c3():
    # lognormal with sigma = 1 and mu chosen so the unclipped mean is 512;
    # rounded to the nearest integer and clipped to [1, 4096]
    sigma = 1.0
    mu = math.log(512.0) - sigma * sigma / 2.0
    x = _rng(3, 0).lognormal(mu, sigma, size=256)
    return np.clip(np.rint(x), 1, 4096).astype(np.int64)


def _ctx_c5():
    return _rng(5, 0).integers(32768, 131073, size=8).astype(np.int64)


def _churn_ops(num_blocks: int, steps: int = 10000) -> List[tuple]:
    """Allocator churn over the shared free list before the batch is admitted.

    Each step, with probability 1/2 (or always when nothing is live) one block
    is taken into a live list L (only if a free block remains); otherwise a
    uniformly chosen member of L is given back.  Afterwards every member of L
    is given back in a seeded random order.  A taken block is modelled as a
    one-block sequence, so the script only uses add_seq/free_seq."""
    r = _rng(3, 1)
    coin = r.random(steps)
    pick = r.random(steps)
    final = r.random(steps)
    ops: List[tuple] = []
    live: List[int] = []
    next_id = TEMP_SEQ_BASE
    for k in range(steps):
        take = coin[k] < 0.5 or not live
        if take:
            if len(live) < num_blocks:
                ops.append(("add_seq", next_id, 1, False))
                live.append(next_id)
                next_id += 1
        else:
            idx = int(pick[k] * len(live))
            ops.append(("free_seq", live.pop(idx)))
    order = np.argsort(final[:len(live)], kind="stable")
    for j in order:
        ops.append(("free_seq", live[int(j)]))
    return ops


def _no_kv(cfg: Config, rows: int, k_scale: float = 1.0):
    z = np.zeros((rows, 0, 0), np.float32)
    return z, z


def _no_q(cfg: Config, count: int = 1):
    return [np.zeros((cfg.num_seqs, 0, 0), np.float32)] * count


def build(name: str, values: bool = True) -> Workload:
    """Draw the inputs and the construction script of configuration ``name``.
    ``values=False`` skips the K/V/Q draws (script and lengths only)."""
    cfg = CONFIGS[name]
    draw_kv, draw_q = (_draw_kv, _draw_q) if values else (_no_kv, _no_q)
    bs = cfg.block_size
    if cfg.index in (1, 2, 5):
        ctx = {1: _ctx_c1, 2: _ctx_c2, 5: _ctx_c5}[cfg.index]()
        nb = 64 if cfg.index == 1 else _pool_size(ctx, bs)
        order = _rng(cfg.index, 1).permutation(nb).astype(np.int64)
        k, v = draw_kv(cfg, int(ctx.sum()), k_scale=0.5 if cfg.index == 5 else 1.0)
        row_start = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int64)
        ops = [("create", nb, order)] + _prefill_then_decode(ctx)
        return Workload(cfg, ctx, k, v, draw_q(cfg), ops, nb, row_start)

    if cfg.index == 3:
        ctx = _ctx_c3()
        nb = _pool_size(ctx, bs)
        k, v = draw_kv(cfg, int(ctx.sum()))
        row_start = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int64)
        ops = [("create", nb, None)] + _churn_ops(nb) + _prefill_then_decode(ctx)
        return Workload(cfg, ctx, k, v, draw_q(cfg), ops, nb, row_start)

    if cfg.index == 4:
        cow = name == "c4b_prefix_cow"
        prefix = 2040 if cow else 2048
        suffix = _rng(4, 0).integers(1, 513, size=64).astype(np.int64)
        ctx = prefix + suffix
        B = len(ctx)
        # pool: 1.2x the blocks the script can hold at once (shared prefix
        # blocks once, every sequence's private blocks, one spare per sequence
        # for the copy of the partial shared block)
        private = _ceil_div(ctx, bs) - prefix // bs
        nb = int(math.ceil(1.2 * (prefix // bs + int(private.sum()) + B)))
        order = _rng(4, 1).permutation(nb).astype(np.int64)
        k, v = draw_kv(cfg, prefix + int(suffix.sum()))
        row_start = np.concatenate([[0], np.cumsum(suffix)[:-1]]).astype(np.int64) + prefix
        ops: List[tuple] = [("create", nb, order), ("add_seq", 0, prefix, True)]
        ops += [("fork", 0, i) for i in range(1, B)]
        q_sets = draw_q(cfg, 2 if cow else 1)
        if cow:
            # first decode step: suffix token 0 for every sequence; sharers
            # 0..62 copy the partial block 127, the last sharer writes in place
            ops.append(("append", list(range(B))))
            ops.append(("decode", list(range(B)), 0))
            done = np.ones(B, np.int64)
        else:
            done = np.zeros(B, np.int64)
        # remaining suffix tokens but the last, step-major in sequence order
        while True:
            step = [i for i in range(B) if done[i] < suffix[i] - 1]
            if not step:
                break
            ops.append(("append", step))
            done[step] += 1
        last = [i for i in range(B) if done[i] < suffix[i]]
        ops.append(("append", last))
        ops.append(("decode", list(range(B)), len(q_sets) - 1))
        return Workload(cfg, ctx, k, v, q_sets, ops, nb, row_start, prefix_len=prefix)

    raise KeyError(name)


def tiny(num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
         dtype="bf16", ctx: Optional[Sequence[int]] = None, seed: int = 0,
         num_blocks: Optional[int] = None, permute: bool = True) -> Workload:
    """Small ad-hoc workload (prefill + one decode step) for unit tests."""
    def rng(stream):
        return np.random.default_rng([7, seed, stream])
    if ctx is None:
        ctx = rng(0).integers(1, 5 * block_size, size=num_seqs)
    ctx = np.asarray(ctx, dtype=np.int64)
    cfg = Config(f"tiny{seed}", 0, len(ctx), num_q_heads, num_kv_heads, head_dim,
                 block_size, dtype)
    nb = num_blocks or max(1, _pool_size(ctx, block_size))
    order = rng(1).permutation(nb).astype(np.int64) if permute else None
    shape = (int(ctx.sum()), num_kv_heads, head_dim)
    k = round_to_dtype(rng(2).standard_normal(shape, dtype=np.float32), dtype)
    v = round_to_dtype(rng(3).standard_normal(shape, dtype=np.float32), dtype)
    q = round_to_dtype(rng(4).standard_normal((len(ctx), num_q_heads, head_dim),
                                              dtype=np.float32), dtype)
    row_start = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int64)
    ops = [("create", nb, order)] + _prefill_then_decode(ctx)
    return Workload(cfg, ctx, k, v, [q], ops, nb, row_start)


def admission_trace(num_requests: int = 3000, mean_live: int = 256):
    """Arrivals and departures shaped like the 13B-like MHA configuration's
    traffic, for the waste and admission accounting.

    Request i arrives at step i with a length drawn like that configuration's
    contexts (lognormal, sigma 1, unclipped mean 512, rounded and clipped to
    [1, 4096]) and leaves d_i steps later, d_i uniform in [1, 2 mean_live - 1]
    (so about mean_live requests are live at once when all are admitted).  At
    each step the departures due come first, in request order, then the
    arrival.  Returns (events, lengths) with events ("arrive", i, length) and
    ("depart", i); the pool it is replayed against is the configuration's own
    (the 1.2x rule over its 256 contexts)."""
    sigma = 1.0
    mu = math.log(512.0) - sigma * sigma / 2.0
    lengths = np.clip(np.rint(_rng(3, 5).lognormal(mu, sigma, size=num_requests)), 1, 4096).astype(np.int64)
    life = _rng(3, 6).integers(1, 2 * mean_live, size=num_requests).astype(np.int64)
    leave = np.arange(num_requests) + life
    by_step: dict = {}
    for i, t in enumerate(leave.tolist()):
        by_step.setdefault(t, []).append(i)
    events: List[tuple] = []
    for step in range(num_requests):
        for i in by_step.get(step, []):
            events.append(("depart", i))
        events.append(("arrive", step, int(lengths[step])))
    for step in sorted(t for t in by_step if t >= num_requests):
        for i in by_step[step]:
            events.append(("depart", i))
    return events, lengths
