"""Replay a block-manager script on the device path.

A script is a list of operations on sequences (create the pool, add a
sequence with its tokens, fork, free, append one token to each of a list of
sequences, decode a list of sequences); the K/V/Q values come with it.  The
replay drives PagedKVEngine — the C++ block manager and the HIP kernels — and
records every integer result (slots, copy pairs, tables, context lengths) and
every decode output, so they can be compared with an independent model.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import PA_KERNEL_AUTO
from .engine import PagedKVEngine

__all__ = ["TORCH_DTYPE", "DeviceRun", "upload_rows", "run_script"]

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def upload_rows(rows: np.ndarray, dtype, device, chunk: int = 1 << 16) -> torch.Tensor:
    """float32 host rows (exactly representable in dtype) -> device tensor of dtype."""
    out = torch.empty(rows.shape, dtype=dtype, device=device)
    for i in range(0, rows.shape[0], chunk):
        out[i:i + chunk] = torch.from_numpy(np.ascontiguousarray(rows[i:i + chunk])).to(device).to(dtype)
    return out


@dataclass
class DeviceDecode:
    seqs: List[int]
    q_index: int
    tables: np.ndarray
    ctx: np.ndarray
    out: torch.Tensor


@dataclass
class DeviceRun:
    engine: PagedKVEngine
    appends: List[dict] = field(default_factory=list)
    add_slots: dict = field(default_factory=dict)
    decodes: List[DeviceDecode] = field(default_factory=list)
    k_dev: Optional[torch.Tensor] = None
    v_dev: Optional[torch.Tensor] = None
    q_dev: List[torch.Tensor] = field(default_factory=list)


def run_script(w, device="cuda", partition_size: int = 0, kernel: int = PA_KERNEL_AUTO,
               out_dtype=torch.float32, poison: bool = True, decode: bool = True,
               extra_context: int = 0, use_step: bool = False, extra_blocks: int = 0,
               on_engine=None) -> DeviceRun:
    """Replay ``w.ops``; ``extra_context`` widens the table stride for tokens
    appended after the script and ``extra_blocks`` adds spare blocks at the
    bottom of the free list (the script's allocations are unchanged; tokens
    appended after it use them).  With ``use_step`` an append directly followed
    by a decode of the same sequences runs as one engine step (one host to
    device copy), the way the benchmark drives it.  ``on_engine(engine)`` is
    called once the engine exists (to set its options before any step)."""
    cfg = w.cfg
    dtype = TORCH_DTYPE[cfg.dtype]
    dev = torch.device(device)
    k_dev = upload_rows(w.k_rows, dtype, dev)
    v_dev = upload_rows(w.v_rows, dtype, dev)
    q_dev = [upload_rows(q, dtype, dev) for q in w.q_sets]
    run: Optional[DeviceRun] = None
    max_ctx = int(np.max(w.ctx)) + extra_context
    ops = list(w.ops)
    i = 0
    while i < len(ops):
        op = ops[i]
        i += 1
        kind = op[0]
        if (use_step and decode and kind == "append" and i < len(ops) and ops[i][0] == "decode"
                and list(ops[i][1]) == list(op[1])):
            seqs, qi = op[1], ops[i][2]
            i += 1
            pos = np.array([run.engine.bm.seq_len(s) for s in seqs], dtype=np.int64)
            rows = np.array([w.row_of(s, np.array([p]))[0] for s, p in zip(seqs, pos)], dtype=np.int64)
            idx = torch.from_numpy(rows).to(dev)
            q = q_dev[qi][torch.tensor(seqs, device=dev)].contiguous()
            before = run.engine.bm.stats()[3]
            out = run.engine.step(seqs, k_dev[idx], v_dev[idx], q, out_dtype=out_dtype,
                                  partition_size=partition_size, kernel=kernel)
            ncow = run.engine.bm.stats()[3] - before
            st = run.engine._ring[(run.engine._ri - 1) % len(run.engine._ring)]
            (hs, hp, _, _), _, _ = st.packed(len(seqs))
            run.appends.append({"seqs": list(seqs), "pos": pos, "slots": hs.numpy().copy(),
                                "pairs": [tuple(int(x) for x in p) for p in hp.numpy()[:ncow]]})
            run.decodes.append(DeviceDecode(list(seqs), qi, run.engine.last_tables.copy(),
                                            run.engine.last_ctx.copy(), out))
            continue
        if kind == "create":
            nb, order = op[1], op[2]
            if extra_blocks:
                base = np.arange(nb) if order is None else np.asarray(order)
                order = np.concatenate([base, np.arange(nb, nb + extra_blocks)])
                nb += extra_blocks
            eng = PagedKVEngine(nb, cfg.num_kv_heads, cfg.head_dim, cfg.block_size, dtype, order,
                                device=dev, poison=poison, max_seqs=cfg.num_seqs, max_context=max_ctx)
            run = DeviceRun(eng, k_dev=k_dev, v_dev=v_dev, q_dev=q_dev)
            if on_engine is not None:
                on_engine(eng)
        elif kind == "add_seq":
            _, seq, n, write = op
            if write and n:
                idx = torch.from_numpy(w.row_of(seq, np.arange(n))).to(dev)
                run.add_slots[seq] = run.engine.add_seq(seq, k_dev[idx], v_dev[idx], n)
            else:
                slots = run.engine.add_seq(seq, None, None, n)
                if write:
                    run.add_slots[seq] = slots
        elif kind == "fork":
            run.engine.fork(op[1], op[2])
        elif kind == "free_seq":
            run.engine.free_seq(op[1])
        elif kind == "append":
            seqs = op[1]
            pos = np.array([run.engine.bm.seq_len(s) for s in seqs], dtype=np.int64)
            rows = np.array([w.row_of(s, np.array([p]))[0] for s, p in zip(seqs, pos)], dtype=np.int64)
            idx = torch.from_numpy(rows).to(dev)
            slots, pairs = run.engine.append(seqs, k_dev[idx], v_dev[idx])
            run.appends.append({"seqs": list(seqs), "pos": pos, "slots": slots.copy(),
                                "pairs": [tuple(int(x) for x in p) for p in pairs]})
        elif kind == "decode":
            seqs, qi = op[1], op[2]
            if not decode:
                continue
            q = q_dev[qi][torch.tensor(seqs, device=dev)].contiguous()
            out = run.engine.decode(seqs, q, out_dtype=out_dtype, partition_size=partition_size,
                                    kernel=kernel)
            run.decodes.append(DeviceDecode(list(seqs), qi, run.engine.last_tables.copy(),
                                            run.engine.last_ctx.copy(), out))
        else:
            raise ValueError(kind)
    torch.cuda.synchronize(dev)
    return run
