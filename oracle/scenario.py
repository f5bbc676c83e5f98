"""Run a workload's construction script through the oracle (test infrastructure only).

Each op of the script is applied to the block-manager model and the cache
model in order; every decode op records the exported tables and context
lengths and the float64 textbook attention of each listed sequence over the
K/V gathered back from the pool through its table (paged ≡ contiguous is
checked separately by the tests).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from .attention import decode_attention
from .block_manager import BlockManagerModel
from .cache import PagedCacheModel

__all__ = ["ScenarioResult", "run_scenario", "table_stride"]


def table_stride(workload) -> int:
    """Width of the exported tables: enough blocks for the longest context."""
    bs = workload.cfg.block_size
    return max(1, int(-(-int(np.max(workload.ctx)) // bs)))


@dataclass
class DecodeRecord:
    seqs: List[int]
    q_index: int
    tables: np.ndarray          # int32 [n, stride]
    ctx: np.ndarray             # int32 [n]
    out: Optional[np.ndarray]   # float64 [n, Hq, D] (rows not in `computed` are NaN)
    computed: List[int] = field(default_factory=list)


@dataclass
class ScenarioResult:
    bm: BlockManagerModel
    cache: PagedCacheModel
    appends: List[dict]
    add_slots: Dict[int, List[int]]
    decodes: List[DecodeRecord]
    stride: int


def run_scenario(w, outputs: bool = True, sample: Optional[Sequence[int]] = None,
                 cache: bool = True) -> ScenarioResult:
    """Apply ``w.ops``.  ``sample`` limits the attention to those sequence
    indices (positions in the decode list); ``cache=False`` skips the pool
    model (integer block-manager results only)."""
    cfg = w.cfg
    bm: Optional[BlockManagerModel] = None
    cm: Optional[PagedCacheModel] = None
    stride = table_stride(w)
    appends, decodes = [], []
    add_slots: Dict[int, List[int]] = {}
    for op in w.ops:
        kind = op[0]
        if kind == "create":
            bm = BlockManagerModel(op[1], cfg.block_size, op[2])
            if cache:
                cm = PagedCacheModel(op[1], cfg.num_kv_heads, cfg.head_dim, cfg.block_size, cfg.dtype)
        elif kind == "add_seq":
            _, seq, n, write = op
            slots = bm.add_seq(seq, n)
            if write:
                add_slots[seq] = slots
                if cm is not None and n:
                    rows = w.row_of(seq, np.arange(n))
                    cm.write(slots, w.k_rows[rows], w.v_rows[rows])
        elif kind == "fork":
            bm.fork(op[1], op[2])
        elif kind == "free_seq":
            bm.free_seq(op[1])
        elif kind == "append":
            seqs = op[1]
            pos = np.array([bm.length(s) for s in seqs], dtype=np.int64)
            slots, pairs = bm.append(seqs)
            appends.append({"seqs": list(seqs), "pos": pos, "slots": slots, "pairs": pairs})
            if cm is not None:
                cm.copy_blocks(pairs)
                rows = np.array([w.row_of(s, np.array([p]))[0] for s, p in zip(seqs, pos)],
                                dtype=np.int64)
                cm.write(slots, w.k_rows[rows], w.v_rows[rows])
        elif kind == "decode":
            seqs, qi = op[1], op[2]
            tab, lens = bm.export(seqs, stride)
            rec = DecodeRecord(list(seqs), qi, tab, lens, None)
            if outputs and cm is not None:
                q = w.q_sets[qi]
                out = np.full((len(seqs), cfg.num_q_heads, cfg.head_dim), np.nan)
                which = range(len(seqs)) if sample is None else sample
                for j in which:
                    K, V = cm.gather(tab[j], int(lens[j]))
                    out[j] = decode_attention(q[seqs[j]], K, V, cfg.scale)
                    rec.computed.append(int(j))
                rec.out = out
            decodes.append(rec)
        else:
            raise ValueError(kind)
    return ScenarioResult(bm, cm, appends, add_slots, decodes, stride)
