"""Host-side measurement helpers of bench.py (no GPU): the L2 request model
of a stream pass and the algorithmic byte count, checked against closed
forms on the batch-64 GQA shapes."""
import numpy as np
import pytest

import bench
import workloads as W


def _pa():
    import paged_kv_cache_332_amd as pa
    return pa


@pytest.mark.parametrize("name,bs", [("c2_gqa_bf16", 16), ("c2_gqa_bf16_bs8", 8), ("c2_gqa_bf16_bs32", 32)])
def test_l2_model_classes(name, bs):
    pa = _pa()
    cfg = W.config(name)
    ctx = W.build(name, values=False).ctx + 1
    grid = pa.pa_decode_stream_grid(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim)
    m = bench.l2_request_model(ctx, cfg.num_kv_heads, cfg.group, cfg.head_dim, 2, bs, grid,
                               np.full(grid, 1024, np.int32), -(-4096 // bs) + 8, pa)
    tiles = int((-(-ctx // 16)).sum()) * cfg.num_kv_heads
    # every 16-token tile is 8 KiB of K and V: 64 lines of 128 bytes; at block
    # size 8 a tile whose second block holds no token reads its first block twice
    if bs == 8:
        half = int(np.sum((-(-ctx // 16)) * 16 - ctx >= 8)) * cfg.num_kv_heads
        assert m["kv"] == 64 * tiles - 32 * half
    else:
        assert m["kv"] == 64 * tiles
    # table entries: at least one line per wave with work, at most one per tile
    # (two at block size 8), and a line is first touched on a die once at most
    entries = int((-(-ctx // bs)).sum())
    assert 4 * grid <= m["table"] <= (2 if bs == 8 else 1) * tiles
    assert m["table_first_touch_per_die"] <= min(m["table"], 8 * -(-entries * 4 // 128) + 8 * cfg.num_seqs)
    # one query load (g rows of D) per item start and per wave start
    items = cfg.num_seqs * cfg.num_kv_heads
    q_lines = -(-cfg.group * cfg.head_dim * 2 // 128)
    assert items * q_lines <= m["query"] <= (items + 4 * grid) * q_lines
    assert m["total"] == m["kv"] + m["table"] + m["query"] + m["metadata"]


def test_decode_bytes_closed_form():
    cfg = W.config("c2_gqa_bf16")
    ctx = np.array([1, 16, 17, 4096], dtype=np.int64)
    b = bench.decode_bytes(ctx, cfg, 2)
    kv = int(ctx.sum()) * 2 * cfg.num_kv_heads * cfg.head_dim * 2
    qo = len(ctx) * cfg.num_q_heads * cfg.head_dim * (2 + 4)
    tables = int((-(-ctx // cfg.block_size)).sum()) * 4
    assert b == kv + qo + tables + 4 * len(ctx)


def test_unique_kv_bytes_counts_shared_blocks_once():
    """Two sequences sharing a full first block (id 5) and each holding a
    private partial block: the shared block counts once; a block two tables
    hold with different fill counts counts its fullest use."""
    tables = np.array([[5, 1, -1], [5, 2, -1], [7, -1, -1], [7, -1, -1]], np.int32)
    ctx = np.array([20, 17, 3, 9])
    per_token = 2 * 1 * 4 * 2        # hkv 1, d 4, bf16, K and V
    got = bench.unique_kv_bytes(tables, ctx, 16, 1, 4, 2)
    assert got == (16 + 4 + 1 + 9) * per_token
    assert bench.kv_bytes(ctx, 1, 4, 2) == int(ctx.sum()) * per_token
