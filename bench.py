#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

A step is one decode step of one attention layer for the whole batch: the
host block manager hands every sequence a slot for its new token (taking a
block when the last one is full, copying a shared last block first), the
bookkeeping goes to the device, then pa_copy_blocks, pa_write_kv and
pa_decode (partition pass + log-sum-exp merge) run.  Inputs are the batch-64
GQA bf16 configuration (64 sequences, 32 query / 8 KV heads, head_dim 128,
block 16, contexts uniform in [128, 4096], pool 1.2x the blocks needed in a
seeded random order), prefilled through the same kernels before timing.

Prints one JSON line: whole-step KV read throughput (GB/s of K/V bytes the
attention reads per step / step time), tokens/s, the decode kernel's
roofline against MI355X HBM (8 TB/s), and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per launch of the stream pass from rocprofv3 FETCH_SIZE/WRITE_SIZE
# runs (scaled by a plain copy's counter readings); they describe the kernel
# source they were taken with and are dropped once that source changes
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_stream_c2_gqa_bf16_traffic.json")
STREAM_HOST_MARKER = b"// ==== host side: launch configuration"
STREAM_SRC = os.path.join(ROOT, "paged_kv_cache_332_amd", "csrc", "decode_stream.hip")
STREAM_HEADERS = [os.path.join(ROOT, "paged_kv_cache_332_amd", "csrc", h) for h in ("pa_device.h", "pa_kernels.h")]
METRIC = "paged decode KV read GB/s (% of HBM peak) + tokens/s, batch 64 GQA bf16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=64,
                    help="untimed steps (they also settle the stream kernel's workgroup shares)")
    ap.add_argument("--config", default="c2_gqa_bf16")
    ap.add_argument("--partition", type=int, default=None, help="tokens per split-K partition (0 = library)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma", "stream"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--in-step", type=int, default=4,
                    help="steps run after the timed ones with HIP events around each pass (an event packet "
                         "between kernels costs the stream ~5 us, so the timed steps carry none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the short prefill / prefix-cache / swap measurements added to the decode line")
    ap.add_argument("--cold", type=int, default=8, help="passes timed after evicting the Infinity Cache")
    ap.add_argument("--prefill", type=int, default=0, metavar="L",
                    help="measure pa_prefill instead: the last min(L, ctx) tokens of every sequence of the "
                         "config as one chunk each (prints its own JSON line)")
    ap.add_argument("--swap", type=float, default=0.0, metavar="FRAC",
                    help="measure preemption by swap instead: every k-th sequence (FRAC of the batch) copied "
                         "to pinned host memory and back with pa_swap_blocks (prints its own JSON line)")
    ap.add_argument("--prefix-cache", type=int, default=0, metavar="P",
                    help="measure prefill with prefix caching instead: the config's batch of prompts sharing a "
                         "P-token prefix plus U[128,512] own tokens, prefilled with cached prefix blocks reused "
                         "and again with none (prints its own JSON line)")
    ap.add_argument("--waste", action="store_true",
                    help="measure the block manager instead: admission and occupancy on the 13B-like "
                         "configuration's arrival/departure trace, and the host cost of each pa_bm_* call "
                         "(prints its own JSON line; no GPU work)")
    ap.add_argument("--burst", type=int, default=16,
                    help="back-to-back pass launches timed for the roofline's launch duration")
    ap.add_argument("--pool-order", default="config", choices=["config", "identity"],
                    help="initial free-list order: the config's own (seeded permutation) or identity, so that "
                         "blocks taken in order are physically consecutive")
    ap.add_argument("--l2-model", action="store_true",
                    help="add the modelled L2 read requests of the last step's pass, by class")
    ap.add_argument("--no-balance", action="store_true",
                    help="equal workgroup shares in the stream kernel (no feedback from wave times)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (scales byte counters)")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of known size: what FETCH_SIZE and
    WRITE_SIZE read for it gives the factor from counter units to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "calls": 5}), flush=True)


def kv_bytes(ctx: np.ndarray, hkv: int, d: int, esize: int) -> int:
    """Algorithmic K+V bytes one decode reads: every context token's key and
    value row of every kv head, once."""
    return int(ctx.astype(np.int64).sum()) * hkv * d * 2 * esize


def unique_kv_bytes(tables: np.ndarray, ctx: np.ndarray, block_size: int, hkv: int, d: int, esize: int) -> int:
    """K+V bytes of the distinct physical blocks a decode reads: a block that
    several sequences share counts once, with the most tokens any of them
    uses (the duplication the pages say sharing removes)."""
    used = {}
    for row, n in zip(np.asarray(tables), np.asarray(ctx, np.int64)):
        nb = -(-int(n) // block_size)
        for j in range(nb):
            b = int(row[j])
            used[b] = max(used.get(b, 0), min(block_size, int(n) - j * block_size))
    return sum(used.values()) * hkv * d * 2 * esize


def decode_bytes(ctx, cfg, esize, out_esize=4) -> int:
    """Algorithmic bytes of one pa_decode call: K/V rows, the queries, the
    outputs, the table entries and context lengths it reads."""
    b = len(ctx)
    tables = int((-(-ctx.astype(np.int64) // cfg.block_size)).sum()) * 4
    return (kv_bytes(ctx, cfg.num_kv_heads, cfg.head_dim, esize) + b * cfg.num_q_heads * cfg.head_dim * esize
            + b * cfg.num_q_heads * cfg.head_dim * out_esize + tables + 4 * b)


def stream_device_code_sha(hashlib) -> str:
    """Hash of the stream kernel's device code: the source text before the
    host-side marker (launch code below it does not change what a pass
    reads or writes), followed by the device headers it includes and the
    extra compiler flags the build gives that file."""
    with open(STREAM_SRC, "rb") as f:
        text = f.read().split(STREAM_HOST_MARKER, 1)[0]
    for h in STREAM_HEADERS:
        with open(h, "rb") as f:
            text += f.read()
    import importlib.util
    spec = importlib.util.spec_from_file_location("pa_build_flags", os.path.join(ROOT, "paged_kv_cache_332_amd",
                                                                                 "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    text += " ".join(b.FILE_FLAGS.get(os.path.basename(STREAM_SRC), [])).encode()
    return hashlib.sha256(text).hexdigest()


def measured_traffic(kernel_name: str, config: str, bytes_per_launch: int):
    """HBM bytes per launch from the committed counter profile: (traffic,
    ratio).  ``ratio`` = counted bytes / algorithmic bytes of the counted
    launches, whenever the record is for this kernel source and workload;
    ``traffic`` = the counted bytes only when the counted launches moved the
    same algorithmic bytes as this line's launch (the same steps and warm-up
    of the same workload), else None."""
    import hashlib
    if kernel_name != "stream" or not os.path.exists(TRAFFIC_FILE):
        return None, None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("config") != config or rec.get("source_sha256") != stream_device_code_sha(hashlib):
        return None, None
    counted = int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])
    algo = int(rec.get("algorithmic_bytes_per_launch", 0))
    if algo <= 0:
        return None, None
    return (counted if algo == int(bytes_per_launch) else None), round(counted / algo, 4)


def cpu_baseline(w, budget_s: float):
    """The oracle as it stands, on the host cores: replay of the script
    (untimed), then gather + float64 attention of whole sequences of the
    final decode step until about budget_s seconds have been spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    ref = oracle.run_scenario(w, outputs=False)
    d = ref.decodes[-1]
    cfg = w.cfg
    q = w.q_sets[d.q_index]

    def run(budget):
        done_bytes, seqs = 0, 0
        t0 = time.perf_counter()
        j = 0
        while time.perf_counter() - t0 < budget:
            i = j % len(d.seqs)
            K, V = ref.cache.gather(d.tables[i], int(d.ctx[i]))
            oracle.decode_attention(q[d.seqs[i]], K, V, cfg.scale)
            done_bytes += kv_bytes(np.array([d.ctx[i]]), cfg.num_kv_heads, cfg.head_dim,
                                   W_ELEM[cfg.dtype])
            seqs += 1
            j += 1
        return done_bytes, seqs, time.perf_counter() - t0

    done_bytes, seqs, el = run(budget_s)
    res = {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
           "kind": "oracle",
           "sample": f"{seqs} sequences of the final decode step ({done_bytes / 1e6:.0f} MB of K/V) "
                     f"gathered through the table and attended in float64 in {el:.1f} s; "
                     f"host has {os.cpu_count()} cpus, affinity {len(os.sched_getaffinity(0))}",
           "tokens_per_s": round(seqs / el, 3)}
    # the same on one BLAS thread, for a quarter of the budget
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            b1, s1, e1 = run(budget_s / 4)
        res["one_thread"] = {"value": round(b1 / e1 / 1e9, 4), "unit": "GB/s", "tokens_per_s": round(s1 / e1, 3),
                             "sample": f"{s1} sequences in {e1:.1f} s"}
    except Exception as e:  # pragma: no cover
        res["one_thread"] = f"not measured: {e}"
    return res


W_ELEM = {"f32": 4, "f16": 2, "bf16": 2}


def l2_request_model(ctx, num_kv_heads, group, head_dim, esize, block_size, grid, weights, stride, pa):
    """L2 read requests of one stream pass by class, modelled from the pass's
    split (128-byte lines, one request per distinct line of a wave's load
    instruction): K/V tile lines, block-table lines, query-row lines and the
    start-up metadata (plan entries, lengths, tile prefix sums).  A line is a
    compulsory miss the first time a die (XCD, workgroup b on die b mod 8)
    touches it in the pass; the model counts those too.  Tiles are 16 tokens:
    at block size 8 a tile takes two table entries (the second only when it
    holds a context token, else the first block is read twice and its lanes
    coalesce into half the lines); at 32 two tiles share one entry.  The
    constants mirror the kernel and the step record: tiles staged per table
    read (224) and the tables' offset in the record (after 4 words per
    sequence)."""
    line = 128
    ctx = np.asarray(ctx, np.int64)
    tiles = -(-ctx // 16)
    pre = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)
    starts, _, _ = pa.pa_stream_plan(pre.astype(np.int32), num_kv_heads, grid, weights)
    starts = starts.astype(np.int64)
    B = len(ctx)
    tcap = 224
    tab_base = 16 * B                      # tables follow slots, pairs and lengths in the record
    kv_lines_per_tile = 2 * 16 * head_dim * esize // line
    q_lines = -(-group * head_dim * esize // line)
    seen = [set() for _ in range(8)]
    n_tab = n_tab_first = n_q = n_kv = 0

    def count(die, addrs):
        nonlocal n_tab, n_tab_first
        ls = np.unique(addrs // line)
        n_tab += len(ls)
        for x in ls.tolist():
            if x not in seen[die]:
                seen[die].add(x)
                n_tab_first += 1

    for w in range(4 * grid):
        ga, gb = int(starts[w]), int(starts[w + 1])
        if ga >= gb:
            continue
        die = (w // 4) % 8
        g = np.arange(ga, gb)
        seq = np.searchsorted(num_kv_heads * pre, g, side="right") - 1
        r = g - num_kv_heads * pre[seq]
        nt = tiles[seq]
        t = r % nt
        row = tab_base + seq * stride * 4
        if block_size == 8:
            two = 16 * t + 8 < ctx[seq]
            ax, ay = row + 2 * t * 4, row + np.where(two, 2 * t + 1, 2 * t) * 4
            n_kv += int(np.sum(np.where(two, kv_lines_per_tile, kv_lines_per_tile // 2)))
        else:
            ax, ay = row + (t if block_size == 16 else t // 2) * 4, None
            n_kv += (gb - ga) * kv_lines_per_tile
        # query rows at every item start inside the share, and the first item
        n_q += q_lines * int(np.count_nonzero((t == 0)[1:]) + 1)
        for c0 in range(0, gb - ga, tcap):
            for j in range(c0, min(c0 + tcap, gb - ga), 64):
                e = min(j + 64, c0 + tcap, gb - ga)
                count(die, ax[j:e])
                if ay is not None:
                    count(die, ay[j:e])
    # start-up: each wave reads two plan words, each workgroup B + 1 prefix
    # sums and B lengths (4-byte entries)
    meta = 4 * grid + grid * (-(-(B + 1) * 4 // line) + -(-B * 4 // line))
    meta_lines = -(-(4 * grid + 1) * 4 // line) + 8 * (-(-(B + 1) * 4 // line) + -(-B * 4 // line))
    return {"line_bytes": line, "kv": int(n_kv), "table": int(n_tab), "table_first_touch_per_die": int(n_tab_first),
            "query": int(n_q), "metadata": int(meta), "metadata_first_touch_per_die": int(min(meta, meta_lines)),
            "total": int(n_kv + n_tab + n_q + meta)}


def prefill_bench(args, w, cfg, pa, runner, torch):
    """pa_prefill on the config's pools: every sequence's last min(L, ctx)
    tokens as its chunk, causal over its whole context.  FLOPs count 4 Hq D
    per (query token, visible key): QK^T and PV, multiply and add."""
    dtype = runner.TORCH_DTYPE[cfg.dtype]
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    seqs = list(range(cfg.num_seqs))
    tab, ctx = eng.bm.export(seqs, eng.stride)
    ctx = np.asarray(ctx, dtype=np.int64)
    chunk = np.minimum(args.prefill, ctx)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    T = int(qs[-1])
    g = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn((T, cfg.num_q_heads, cfg.head_dim), generator=g, device="cuda").to(dtype)
    out = torch.empty((T, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    tab_d = torch.from_numpy(np.ascontiguousarray(tab)).to("cuda")
    qs_d = torch.from_numpy(qs).to("cuda")
    ctx_d = torch.from_numpy(ctx.astype(np.int32)).to("cuda")
    scale = 1.0 / cfg.head_dim ** 0.5
    # the workspace lets launches of few workgroups (short chunks) split each
    # context into pieces merged by log-sum-exp
    ws_bytes = pa.pa_prefill_workspace_bytes(int(chunk.max()), int(ctx.max()), cfg.num_seqs, cfg.num_q_heads,
                                             cfg.num_kv_heads, cfg.head_dim)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    run = lambda: pa.pa_prefill(out, q, eng.k_cache, eng.v_cache, tab_d, qs_d, ctx_d, int(chunk.max()),
                                int(ctx.max()), scale, workspace=ws)
    for _ in range(args.warmup):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # visible keys per query token: its position + 1
    keys = sum(int(((c - L + 1) + c) * L // 2) for c, L in zip(ctx, chunk))
    flops = 4.0 * cfg.num_q_heads * cfg.head_dim * keys
    # K/V tiles each workgroup streams (16-token tiles up to its last token),
    # with the workgroup size the library picks for this launch
    G = cfg.num_q_heads // cfg.num_kv_heads
    cb = pa.pa_prefill_column_blocks(cfg.num_q_heads, cfg.num_kv_heads, int(chunk.max()), cfg.num_seqs)
    tpw = 4 * cb * (16 // G)
    tiles = 0
    for c, L in zip(ctx, chunk):
        p0 = c - L
        for b in range(0, int(L), tpw):
            tiles += -(-(p0 + min(L, b + tpw)) // 16)
    kv_bytes = tiles * cfg.num_kv_heads * 2 * 16 * cfg.head_dim * W_ELEM[cfg.dtype]
    tflops = flops / (us * 1e-6) / 1e12
    return {
        "metric": "paged prefill TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 4), "higher_is_better": True,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": args.config, "batch": cfg.num_seqs, "chunk": int(args.prefill),
                   "query_tokens": T, "ctx_mean": round(float(ctx.mean()), 1)},
        "column_blocks_per_wave": cb, "context_split_workspace_bytes": int(ws_bytes),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "kv_bytes_streamed": int(kv_bytes),
                     "kv_GBps": round(kv_bytes / (us * 1e-6) / 1e9, 1)},
    }


def swap_bench(args, w, cfg, pa, runner, torch):
    """pa_swap_blocks on the config's pools: the blocks of every k-th sequence
    (k = round(1 / FRAC)) moved to pinned host memory and back, each direction
    timed on its own with HIP events.  The copy runs over the host link, so a
    plain DMA copy of the same bytes (torch's pinned copy) is timed beside it
    as the link's practical rate; peak = 64 GB/s per direction (PCIe 5.0 x16)."""
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    k = max(1, int(round(1.0 / args.swap)))
    victims = list(range(0, cfg.num_seqs, k))
    tab, ctx = eng.bm.export(victims, eng.stride)
    blocks = np.concatenate([tab[i, : -(-int(c) // cfg.block_size)] for i, c in enumerate(ctx)]).astype(np.int32)
    n = int(blocks.size)
    per_block = eng.k_cache[0].numel()
    tdt = eng.k_cache.dtype
    host_k = torch.empty((n, per_block), dtype=tdt).pin_memory()
    host_v = torch.empty((n, per_block), dtype=tdt).pin_memory()
    ids = torch.from_numpy(blocks).to("cuda")
    nbytes = 2 * n * per_block * eng.k_cache.element_size()
    steps = max(1, min(args.steps, 20))
    ref_k = eng.k_cache[ids.long()].clone()

    def timed(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    us_out = timed(lambda: pa.pa_swap_blocks(eng.k_cache, eng.v_cache, host_k, host_v, ids, to_host=True))
    us_in = timed(lambda: pa.pa_swap_blocks(eng.k_cache, eng.v_cache, host_k, host_v, ids, to_host=False))
    bits = torch.int32 if ref_k.element_size() == 4 else torch.int16      # unwritten slots hold NaN
    assert torch.equal(eng.k_cache[ids.long()].view(bits), ref_k.view(bits)), "swap round trip changed the pool"
    # the host link's rate for one contiguous copy of the same bytes
    flat_d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    flat_h = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    us_dma_out = timed(lambda: flat_h.copy_(flat_d, non_blocking=True))
    us_dma_in = timed(lambda: flat_d.copy_(flat_h, non_blocking=True))
    gbps = lambda us: round(nbytes / (us * 1e-6) / 1e9, 2)
    peak = 64.0
    return {
        "metric": "swap GB/s", "value": gbps(us_out), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": 2, "ms_per_step": round(us_out / 1e3, 4), "higher_is_better": True, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": args.config, "sequences_swapped": len(victims), "blocks": n,
                   "bytes_each_way": int(nbytes)},
        "swap_out": {"us": round(us_out, 1), "GBps": gbps(us_out)},
        "swap_in": {"us": round(us_in, 1), "GBps": gbps(us_in)},
        "dma_copy": {"out_GBps": gbps(us_dma_out), "in_GBps": gbps(us_dma_in)},
        "roofline": {"bound": "host-link", "achieved": gbps(us_out), "peak": peak, "unit": "GB/s",
                     "frac": round(gbps(us_out) / peak, 4), "frac_in": round(gbps(us_in) / peak, 4)},
    }


def prefix_cache_bench(args, cfg, pa, torch):
    """Prompts sharing a P-token prefix (the config's batch, kv shape and
    block size; own tokens U[128, 512], token ids seeded): pa_bm_add_seq_cached
    reuses the prefix's full blocks, K/V is written and pa_prefill run for the
    remaining tokens only.  The same prompts are then added without the cache
    and prefilled whole.  Reports both prefill times, their ratio, and the
    host cost of the cached admission."""
    import time
    from paged_kv_cache_332_amd.engine import PagedKVEngine
    dtype = {"bf16": torch.bfloat16, "f16": torch.float16}[cfg.dtype]
    B, P, bs = cfg.num_seqs, int(args.prefix_cache), cfg.block_size
    hq, hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    rng = np.random.default_rng([77, P])
    prefix = rng.integers(0, 32000, P)
    prompts = [np.concatenate([prefix, rng.integers(0, 32000, int(rng.integers(128, 513)))]).astype(np.int32)
               for _ in range(B)]
    lens = np.array([len(p) for p in prompts])
    blocks = int(sum(-(-int(n) // bs) for n in lens))
    eng = PagedKVEngine(2 * blocks + 64, hkv, d, bs, dtype, max_seqs=max(B, 1), max_context=int(lens.max()) + bs,
                        poison=False)
    g = torch.Generator(device="cuda").manual_seed(5)

    def write(slots, lo):
        n = len(slots) - lo
        if n <= 0:
            return
        k = torch.randn((n, hkv, d), generator=g, device="cuda").to(dtype)
        v = torch.randn((n, hkv, d), generator=g, device="cuda").to(dtype)
        pa.pa_write_kv(eng.k_cache, eng.v_cache, k, v, torch.from_numpy(np.ascontiguousarray(slots[lo:])).to("cuda"))

    # host cost of cached admission on a manager of its own: the first lap
    # shares the prefix; later laps re-admit the released prompts (each finds
    # its own blocks still cached)
    host_us = []
    side = pa.BlockManager(2 * blocks + 64, bs)
    for r in range(5):
        t0 = time.perf_counter()
        for i, p in enumerate(prompts):
            side.add_seq_cached(i, p)
        host_us.append((time.perf_counter() - t0) * 1e6 / B)
        for i in range(B):
            side.free_seq(i)
    side.close()
    res = [eng.bm.add_seq_cached(i, p) for i, p in enumerate(prompts)]
    for slots, hit in res:
        write(slots, hit)
    hits = np.array([h for _, h in res])
    chunks_c = lens - hits

    def run_prefill(seqs, chunks):
        tab, ctx = eng.bm.export(seqs, eng.stride)
        qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
        T = int(qs[-1])
        q = torch.randn((T, hq, d), generator=g, device="cuda").to(dtype)
        out = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
        tab_d = torch.from_numpy(np.ascontiguousarray(tab)).to("cuda")
        qs_d, ctx_d = torch.from_numpy(qs).to("cuda"), torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda")
        nb = pa.pa_prefill_workspace_bytes(int(max(chunks)), int(max(ctx)), len(seqs), hq, eng.H, d)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
        fn = lambda: pa.pa_prefill(out, q, eng.k_cache, eng.v_cache, tab_d, qs_d, ctx_d, int(max(chunks)),
                                   int(max(ctx)), 1.0 / d ** 0.5, workspace=ws)
        for _ in range(3):
            fn()
        steps = max(1, min(args.steps, 20))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        keys = sum(int(((c - L + 1) + c) * L // 2) for c, L in zip(np.asarray(ctx, np.int64), chunks))
        return us, 4.0 * hq * d * keys / (us * 1e-6) / 1e12, T

    us_c, tf_c, T_c = run_prefill(list(range(B)), chunks_c)
    for i, p in enumerate(prompts):
        write(eng.bm.add_seq(1000 + i, len(p)), 0)
    us_u, tf_u, T_u = run_prefill([1000 + i for i in range(B)], lens)
    return {
        "metric": "prefill speedup from the prefix cache", "value": round(us_u / us_c, 3), "unit": "x",
        "n_gpus": 1, "steps": max(1, min(args.steps, 20)), "warmup": 3, "ms_per_step": round(us_c / 1e3, 4),
        "higher_is_better": True, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": args.config + " prompts", "batch": B, "shared_prefix": P, "own_tokens": "U[128,512]",
                   "block_size": bs, "prompt_tokens": int(lens.sum())},
        "cached": {"ms": round(us_c / 1e3, 3), "query_tokens": T_c, "reused_tokens": int(hits.sum()),
                   "TFLOP/s": round(tf_c, 1)},
        "uncached": {"ms": round(us_u / 1e3, 3), "query_tokens": T_u, "TFLOP/s": round(tf_u, 1)},
        "host_us_per_admission": {"shared_prefix_lap": round(host_us[0], 2),
                                  "readmission_median": round(float(np.median(host_us[1:])), 2)},
    }


def waste_bench(pa):
    """The block manager on the 13B-like configuration's traffic
    (workloads.admission_trace: lognormal lengths, about 256 live requests)
    over that configuration's pool: pa_bm_admit with no headroom for each
    arrival (refused requests are dropped), pa_bm_free_seq for each
    departure; after every arrival pa_bm_occupancy is sampled.  Reports
    admissions, refusals, peak and mean live requests, the unused room of
    the blocks held and the slots in use; then the native host cost of each
    pa_bm_* call (the bm_bench tool built beside the library)."""
    import subprocess
    import workloads as W
    wl = W.build("c3_mha_f16_churn", values=False)
    bs = wl.cfg.block_size
    events, lengths = W.admission_trace()
    bm = pa.BlockManager(wl.num_blocks, bs)
    live = set()
    admitted = refused = peak = 0
    live_sum = unused_sum = used_sum = 0.0
    t_admit = t_free = 0.0
    n_free = 0
    for ev in events:
        if ev[0] == "depart":
            if ev[1] in live:
                live.discard(ev[1])
                t0 = time.perf_counter()
                bm.free_seq(ev[1])
                t_free += time.perf_counter() - t0
                n_free += 1
            continue
        t0 = time.perf_counter()
        try:
            bm.admit(ev[1], ev[2], 0)
            ok = True
        except pa.OutOfBlocks:
            ok = False
        t_admit += time.perf_counter() - t0
        if ok:
            admitted += 1
            live.add(ev[1])
        else:
            refused += 1
        held, tokens, slack, free_slots = bm.occupancy()
        peak = max(peak, len(live))
        live_sum += len(live)
        unused_sum += slack / held if held else 0.0
        used_sum += tokens / (wl.num_blocks * bs)
    arrivals = admitted + refused
    tool = os.path.join(ROOT, "paged_kv_cache_332_amd", "bm_bench")
    try:
        ops = json.loads(subprocess.run([tool, "0.3"], capture_output=True, text=True, check=True).stdout)
    except Exception as e:  # reported, not fatal
        ops = {"error": f"{type(e).__name__}: {e}"}
    return {
        "metric": "paged admission on the 13B-like traffic", "value": admitted, "unit": "requests admitted",
        "higher_is_better": True, "n_gpus": 0, "data": "synthetic",
        "config": {"workload": "c3_mha_f16_churn admission trace", "requests": arrivals,
                   "mean_length": round(float(lengths.mean()), 1), "pool_blocks": wl.num_blocks, "block_size": bs,
                   "admission_headroom_blocks": 0},
        "admitted": admitted, "refused": refused, "peak_live": peak, "mean_live": round(live_sum / arrivals, 2),
        "unused_of_held": round(unused_sum / arrivals, 4), "used_fraction": round(used_sum / arrivals, 4),
        "host_ns_per_call_via_python": {"admit": round(t_admit / arrivals * 1e9, 1),
                                        "free_seq": round(t_free / max(n_free, 1) * 1e9, 1)},
        "host_ns_per_call_native": ops,
    }


def next_rows(args, w, cfg, pa, runner, torch):
    """Short measurements of the rows beyond decode on the same workload's
    shapes (each in full by its own flag): paged prefill of 512-token chunks
    (--prefill 512), prefill with a shared 2048-token prefix served from the
    cache (--prefix-cache 2048), preemption by swap of half the batch (--swap
    0.5).  A failure is reported in place of the figures."""
    out = {}
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup = 10, 8
    # (the prefill gets a longer warm-up: it follows the CPU-oracle leg, during
    # which the GPU idled and its clock dropped; 48 launches are about 65 ms)
    for key, run in (("prefill_512", lambda: prefill_bench(_with(sub, prefill=512, warmup=48, steps=20), w, cfg, pa,
                                                           runner, torch)),
                     ("prefix_cache_2048", lambda: prefix_cache_bench(_with(sub, prefix_cache=2048), cfg, pa, torch)),
                     ("swap_half_batch", lambda: swap_bench(_with(sub, swap=0.5), w, cfg, pa, runner, torch))):
        print(f"[bench] next row: {key}", file=sys.stderr, flush=True)
        try:
            r = run()
        except Exception as e:  # reported, not fatal: the decode line above stands on its own
            out[key] = {"error": f"{type(e).__name__}: {e}"}
            continue
        finally:
            torch.cuda.empty_cache()
        if key == "prefill_512":
            out[key] = {"TFLOP/s": r["value"], "frac_of_bf16_peak": r["roofline"]["frac"], "ms": r["ms_per_step"],
                        "query_tokens": r["config"]["query_tokens"], "column_blocks_per_wave": r["column_blocks_per_wave"]}
        elif key == "prefix_cache_2048":
            out[key] = {"speedup": r["value"], "cached_ms": r["cached"]["ms"], "uncached_ms": r["uncached"]["ms"],
                        "reused_tokens": r["cached"]["reused_tokens"]}
        else:
            out[key] = {"out_GBps": r["swap_out"]["GBps"], "in_GBps": r["swap_in"]["GBps"],
                        "frac_of_64GBps": r["roofline"]["frac"], "bytes_each_way": r["config"]["bytes_each_way"]}
    return out


def _with(ns, **kw):
    n = argparse.Namespace(**vars(ns))
    for k, v in kw.items():
        setattr(n, k, v)
    return n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout is a design "
              "note, not a measured path", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.waste:
        import paged_kv_cache_332_amd as pa
        print(json.dumps(waste_bench(pa)), flush=True)
        return
    import torch
    import workloads as W
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    from paged_kv_cache_332_amd.engine import PagedKVEngine

    torch.cuda.init()
    cfg = W.config(args.config)
    part = cfg.partition_size if args.partition is None else args.partition
    kernel = {"auto": pa.PA_KERNEL_AUTO, "valu": pa.PA_KERNEL_VALU, "mfma": pa.PA_KERNEL_MFMA,
              "stream": pa.PA_KERNEL_STREAM}[args.kernel]
    w = W.build(args.config)
    if args.pool_order == "identity" and w.ops[0][0] == "create":
        w.ops[0] = ("create", w.ops[0][1], None)
    dtype = runner.TORCH_DTYPE[cfg.dtype]
    esize = W_ELEM[cfg.dtype]
    print(f"[bench] {args.config}: {cfg.description}; replaying construction script", file=sys.stderr,
          flush=True)

    # replay the construction (prefill + first decode step) on an engine sized
    # for the extra tokens the timed steps append
    total_steps = args.warmup + args.steps + args.in_step
    seqs = list(range(cfg.num_seqs))
    # spare blocks for the tokens the warm-up and timed steps append
    extra_blocks = cfg.num_seqs * (-(-total_steps // cfg.block_size) + 1)
    if args.prefill:
        print(json.dumps(prefill_bench(args, w, cfg, pa, runner, torch)), flush=True)
        return
    if args.swap:
        print(json.dumps(swap_bench(args, w, cfg, pa, runner, torch)), flush=True)
        return
    if args.prefix_cache:
        print(json.dumps(prefix_cache_bench(args, cfg, pa, torch)), flush=True)
        return
    dev = runner.run_script(w, partition_size=part, kernel=kernel, extra_context=total_steps,
                            extra_blocks=extra_blocks)
    eng: PagedKVEngine = dev.engine
    eng.balance = not args.no_balance
    g = torch.Generator(device="cuda").manual_seed(1234)
    k_new = torch.randn((cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim), generator=g, device="cuda").to(dtype)
    v_new = torch.randn((cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim), generator=g, device="cuda").to(dtype)
    q = dev.q_dev[-1][torch.tensor(seqs, device="cuda")].contiguous()
    out = torch.empty((cfg.num_seqs, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    ctx0 = np.array([eng.bm.seq_len(s) for s in seqs], dtype=np.int64)

    def one_step(events=None):
        eng.step(seqs, k_new, v_new, q, out=out, partition_size=part, kernel=kernel, stream=stream,
                 pass_events=events)

    # no garbage-collection pause inside the timed region (the loop allocates
    # little; a collection there would stall the stream for milliseconds).
    # The collection runs before the warm-up: right before the timed steps it
    # evicts the host caches the step's bookkeeping lives in, and the first
    # timed step then took 130-225 us on the host instead of about 35.
    gc.collect()
    gc.disable()
    for i in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ctx_start = ctx0 + args.warmup
    host_s = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        h0 = time.perf_counter()
        one_step()
        host_s.append(time.perf_counter() - h0)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    # the pass alone inside a few more steps (after the timed ones, since the
    # events' own packets would lengthen the steps they sit in)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.in_step)]
    for a, b in ev:          # torch creates an event at its first record
        a.record(stream)
        b.record(stream)
    for e in ev:
        one_step(e)
    torch.cuda.synchronize()
    in_step_ctx = [ctx0 + args.warmup + args.steps + 1 + i for i in range(args.in_step)]
    dec_bytes = [decode_bytes(c, cfg, esize) for c in in_step_ctx]
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev]) if ev else np.zeros(1)
    wts = eng.weights(cfg.num_seqs, cfg.num_q_heads)
    if wts is not None:
        print(f"[bench] workgroup weights by die: {wts[:8].tolist()}", file=sys.stderr, flush=True)

    # each timed step appends one token per sequence before attending
    step_ctx = [ctx_start + 1 + i for i in range(args.steps)]
    kv_total = sum(kv_bytes(c, cfg.num_kv_heads, cfg.head_dim, esize) for c in step_ctx)

    # the pass alone: the last step's pass (same record, plan and data)
    # launched back to back between two events, so that the event packets'
    # own cost (about 4 us each between kernels) stays out of the duration
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rep in range(2):          # the first round warms up
        b0.record(stream)
        for _ in range(args.burst):
            eng.step_layer(eng.k_cache, eng.v_cache, None, None, q, out, phases=pa.STEP_PASS, stream=stream)
        b1.record(stream)
    torch.cuda.synchronize()
    burst_us = b0.elapsed_time(b1) * 1e3 / args.burst
    last_ctx_all = in_step_ctx[-1] if in_step_ctx else step_ctx[-1]
    burst_bytes = decode_bytes(last_ctx_all, cfg, esize)
    achieved = float(burst_bytes / (burst_us * 1e-6) / 1e9)
    # the whole of pa_decode: the pass and the merge of cut items, back to back
    for rep in range(2):
        b0.record(stream)
        for _ in range(args.burst):
            eng.step_layer(eng.k_cache, eng.v_cache, None, None, q, out, phases=pa.STEP_PASS | pa.STEP_MERGE,
                           stream=stream)
        b1.record(stream)
    torch.cuda.synchronize()
    decode_us = b0.elapsed_time(b1) * 1e3 / args.burst

    # the same pass with a cold Infinity Cache: 1 GiB read before each one, so
    # the cache holds clean lines of another buffer (a write would leave dirty
    # lines whose write-back lands in the pass); the read is outside the events
    cold_us = []
    if args.cold:
        scrub = torch.zeros(1 << 27, dtype=torch.int64, device="cuda")
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(args.cold):
            scrub.sum()
            c0.record(stream)
            eng.step_layer(eng.k_cache, eng.v_cache, None, None, q, out, phases=pa.STEP_PASS, stream=stream)
            c1.record(stream)
            torch.cuda.synchronize()
            cold_us.append(c0.elapsed_time(c1) * 1e3)
        del scrub
    value = kv_total / elapsed / 1e9
    # bytes a shared prefix adds to the logical count (constant over the
    # timed steps: they append to private blocks only)
    last_tab, last_ctx = eng.last_tables.copy(), eng.last_ctx.copy()
    dup = kv_bytes(last_ctx, cfg.num_kv_heads, cfg.head_dim, esize) - unique_kv_bytes(
        last_tab, last_ctx, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, esize)
    kname = ("stream" if kernel in (pa.PA_KERNEL_AUTO, pa.PA_KERNEL_STREAM) and cfg.dtype != "f32"
             else args.kernel if args.kernel != "auto" else "valu")
    traffic, traffic_ratio = measured_traffic(kname, args.config, burst_bytes)
    partition = ("stream: equal tile shares per wave, no fixed partition" if kname == "stream" else
                 part or pa.pa_decode_default_partition(cfg.num_seqs, cfg.num_kv_heads, int(step_ctx[-1].max()),
                                                        cfg.block_size))
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": args.config, "batch": cfg.num_seqs, "q_heads": cfg.num_q_heads,
                   "kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim, "block_size": cfg.block_size,
                   "ctx_mean": round(float(np.mean(step_ctx[0])), 1), "partition": partition,
                   "kernel": args.kernel, "balance": eng.balance, "pool_order": args.pool_order,
                   "parallelism": "single GPU"},
        "tokens_per_s": round(cfg.num_seqs * args.steps / elapsed, 1),
        "kv_unique_GBps": round((kv_total - args.steps * dup) / elapsed / 1e9, 2),
        "kv_unique_note": "K/V bytes of distinct physical blocks per step / step time (equal to value "
                          "when no block is shared)",
        "host_us_per_step": round(float(np.median(host_s)) * 1e6, 1),
        "host_us_per_step_max": round(float(np.max(host_s)) * 1e6, 1),
        "host_us_first_steps": [round(x * 1e6, 1) for x in host_s[:6]],
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "pa_decode pass (" + kname + ")",
                     "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_ratio": traffic_ratio, "avg_launch_us": round(burst_us, 2),
                     "bytes_per_launch": int(burst_bytes), "timed_launches": args.burst,
                     "decode_frac": round(burst_bytes / (decode_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "decode": {"avg_us": round(decode_us, 2),
                                "GBps": round(burst_bytes / (decode_us * 1e-6) / 1e9, 2),
                                "note": "pass + merge of cut items (all of pa_decode), back to back"},
                     "cold": None if not cold_us else {
                         "median_us": round(float(np.median(cold_us)), 2),
                         "GBps": round(burst_bytes / (float(np.median(cold_us)) * 1e-6) / 1e9, 2),
                         "launches": len(cold_us),
                         "note": "one pass after reading 1 GiB of another buffer (Infinity Cache evicted); "
                                 "events around the pass alone, so the figure includes one event packet's "
                                 "latency"},
                     "in_step": {"mean_us": round(float(dec_ms.mean()) * 1e3, 2),
                                 "p10_us": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                                 "p90_us": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
                                 "bytes": int(np.mean(dec_bytes)) if dec_bytes else 0, "launches": len(ev),
                                 "note": "events around the pass in steps run after the timed ones; "
                                         "includes the event packets' own latency"}},
        "cpu_baseline": None,
    }
    if args.l2_model and kname == "stream":
        res["l2_request_model"] = l2_request_model(
            last_ctx_all, cfg.num_kv_heads, cfg.group, cfg.head_dim, esize, cfg.block_size,
            pa.pa_decode_stream_grid(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim),
            eng.weights(cfg.num_seqs, cfg.num_q_heads), eng.stride, pa)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    if not args.no_next and cfg.dtype != "f32":
        del dev, eng
        torch.cuda.empty_cache()
        res["next_rows"] = next_rows(args, w, cfg, pa, runner, torch)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
