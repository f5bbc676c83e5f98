"""Pins of the CPU oracle against things other than itself.

Each ``check_*`` takes the oracle function(s) under test as arguments, so the
same checks run on the real oracle (tests/test_oracle.py) and on planted
mistakes (tests/test_oracle_mutants.py), which every mistake must fail.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- attention
def check_golden_gqa(attn):
    """Hand-derived outputs (tests/golden/attention_gqa_hand.json)."""
    g = load_golden("attention_gqa_hand.json")
    out = attn(np.array(g["q"], float), np.array(g["k"], float), np.array(g["v"], float),
               1.0 / math.sqrt(g["head_dim"]))
    np.testing.assert_allclose(out, np.array(g["out"], float), rtol=0, atol=g["tol"])


def check_sdpa(attn):
    """Equals torch's scaled_dot_product_attention (float64, CPU), a library
    routine, with each kv head repeated for its query group."""
    rng = np.random.default_rng(11)
    for Hq, Hkv, D, n in [(8, 2, 16, 1), (8, 2, 16, 33), (4, 4, 64, 100), (8, 1, 32, 7), (6, 3, 8, 257)]:
        q, K, V = _rand(rng, Hq, D), _rand(rng, n, Hkv, D), _rand(rng, n, Hkv, D)
        out = attn(q, K, V, 1.0 / math.sqrt(D))
        g = Hq // Hkv
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]   # [1,Hq,n,D]
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        qt = torch.from_numpy(q)[None, :, None, :]                                    # [1,Hq,1,D]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[0, :, 0, :].numpy()
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def check_one_block_bruteforce(attn):
    """ctx within one block: a plain loop over tokens with math.exp."""
    rng = np.random.default_rng(12)
    Hq, Hkv, D = 4, 2, 8
    for n in (1, 2, 5, 16):
        q, K, V = _rand(rng, Hq, D), _rand(rng, n, Hkv, D), _rand(rng, n, Hkv, D)
        out = attn(q, K, V, 1.0 / math.sqrt(D))
        for r in range(Hq):
            h = r * Hkv // Hq
            s = [sum(q[r, d] * K[t, h, d] for d in range(D)) / math.sqrt(D) for t in range(n)]
            w = [math.exp(x) for x in s]
            ref = [sum(w[t] * V[t, h, d] for t in range(n)) / sum(w) for d in range(D)]
            np.testing.assert_allclose(out[r], ref, rtol=0, atol=1e-12)


def check_identical_keys_mean(attn):
    """All keys equal -> uniform weights -> output is the mean of V."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D, n = 8, 2, 16, 37
    q = _rand(rng, Hq, D)
    K = np.repeat(_rand(rng, 1, Hkv, D), n, axis=0)
    V = _rand(rng, n, Hkv, D)
    out = attn(q, K, V, 0.25)
    for r in range(Hq):
        np.testing.assert_allclose(out[r], V[:, r // 4, :].mean(axis=0), rtol=0, atol=1e-12)


def check_single_token(attn):
    """ctx = 1 -> the output is V[0] exactly."""
    rng = np.random.default_rng(14)
    q, K, V = _rand(rng, 4, 8), _rand(rng, 1, 2, 8), _rand(rng, 1, 2, 8)
    out = attn(q, K, V, 0.3)
    for r in range(4):
        assert np.array_equal(out[r], V[0, r // 2])


def check_gqa_equals_mha(attn):
    """Grouped heads equal plain multi-head attention with each kv head
    repeated for its group (query heads [h*g, (h+1)*g) share kv head h)."""
    rng = np.random.default_rng(15)
    Hq, Hkv, D, n = 8, 2, 16, 21
    q, K, V = _rand(rng, Hq, D), _rand(rng, n, Hkv, D), _rand(rng, n, Hkv, D)
    a = attn(q, K, V, 0.25)
    b = attn(q, np.repeat(K, Hq // Hkv, axis=1), np.repeat(V, Hq // Hkv, axis=1), 0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    # and the grouping is contiguous: kv head 1 carries constant values
    V2 = V.copy()
    V2[:, 1, :] = 5.0
    c = attn(q, K, V2, 0.25)
    np.testing.assert_allclose(c[4:], 5.0, rtol=0, atol=1e-12)
    assert np.all(np.abs(c[:4] - 5.0) > 1e-3)


def check_large_logits(attn):
    """Huge scores: finite output equal to V at the arg-max token."""
    rng = np.random.default_rng(16)
    Hq, Hkv, D, n = 2, 1, 8, 50
    q, K, V = _rand(rng, Hq, D) * 1000.0, _rand(rng, n, Hkv, D), _rand(rng, n, Hkv, D)
    out = attn(q, K, V, 1.0 / math.sqrt(D))
    assert np.all(np.isfinite(out))
    for r in range(Hq):
        s = K[:, 0, :] @ q[r]
        top2 = np.sort(s)[-2:]
        assert (top2[1] - top2[0]) / math.sqrt(D) > 40.0, "seed gives well separated maxima"
        np.testing.assert_allclose(out[r], V[int(np.argmax(s)), 0], rtol=0, atol=1e-12)


def check_empty_context(attn):
    out = attn(np.ones((4, 8)), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), 0.5)
    assert out.shape == (4, 8) and np.all(out == 0.0)


ATTN_CHECKS = [check_golden_gqa, check_sdpa, check_one_block_bruteforce, check_identical_keys_mean,
               check_single_token, check_gqa_equals_mha, check_large_logits, check_empty_context]


def check_split_merge(split_k, lse_merge, attn):
    """Partition partials merged by log-sum-exp equal direct attention
    (float64, 1e-12), for partitions that split ragged, exactly, one token
    each, and not at all."""
    rng = np.random.default_rng(17)
    Hq, Hkv, D = 8, 2, 16
    for n, part in [(100, 32), (96, 32), (7, 1), (50, 512), (513, 512), (1, 4)]:
        q, K, V = _rand(rng, Hq, D), _rand(rng, n, Hkv, D) * 2.0, _rand(rng, n, Hkv, D)
        m, l, acc = split_k(q, K, V, 0.25, part)
        assert m.shape == (-(-n // part), Hq)
        out = lse_merge(m, l, acc)
        np.testing.assert_allclose(out, attn(q, K, V, 0.25), rtol=0, atol=1e-12)
    # one partition: the merge is acc / l and m is the plain maximum score
    q, K, V = _rand(rng, Hq, D), _rand(rng, 9, Hkv, D), _rand(rng, 9, Hkv, D)
    m, l, acc = split_k(q, K, V, 0.25, 16)
    s0 = 0.25 * (K[:, 0, :] @ q[0])
    assert m[0, 0] == s0.max()
    np.testing.assert_allclose(l[0, 0], np.exp(s0 - s0.max()).sum(), rtol=1e-14)
    np.testing.assert_allclose(lse_merge(m, l, acc), acc[0] / l[0][:, None], rtol=0, atol=1e-14)


# ---------------------------------------------------------- block manager
def check_bm_golden(BM, OutOfBlocks):
    """Hand-traced allocation sequence (tests/golden/block_manager_trace.json)."""
    g = load_golden("block_manager_trace.json")
    p = g["pool"]
    bm = BM(p["num_blocks"], p["block_size"], p["order"])
    for st in g["steps"]:
        op = st["op"]
        if op == "add_seq":
            if st.get("error") == "oom":
                before = (list(bm.free), list(bm.rc))
                try:
                    bm.add_seq(st["seq"], st["n"])
                    raise AssertionError("expected out of blocks")
                except OutOfBlocks:
                    pass
                assert (list(bm.free), list(bm.rc)) == before
            else:
                assert bm.add_seq(st["seq"], st["n"]) == st["slots"]
        elif op == "fork":
            bm.fork(st["parent"], st["child"])
        elif op == "append":
            slots, pairs = bm.append(st["seqs"])
            assert list(slots) == st["slots"]
            assert [list(x) for x in pairs] == st["pairs"]
            if "table11" in st:
                assert bm.table(11) == st["table11"]
        elif op == "free_seq":
            bm.free_seq(st["seq"])
        elif op == "export":
            tab, lens = bm.export(st["seqs"], st["stride"])
            assert tab.tolist() == st["tables"] and lens.tolist() == st["lens"]
        if "num_free" in st:
            assert bm.num_free() == st["num_free"], (op, bm.num_free())
        for b, c in st.get("refcounts", {}).items():
            assert bm.refcount(int(b)) == c
    f = g["final"]
    assert bm.num_free() == f["num_free"]
    assert list(reversed(bm.free)) == f["free_stack_top_first"]
    assert [bm.refcount(b) for b in range(p["num_blocks"])] == f["refcounts"]
    s = f["stats"]
    assert tuple(bm.stats()) == (s["free"], s["used"], s["shared"], s["cow_count"], s["waste_tokens"])


def bm_invariants(bm):
    """Invariants the pages fix: free + referenced = pool; no block both free
    and referenced; refcounts equal table references; blocks held by a
    sequence = ceil(len / BS) (waste at most one partial block)."""
    N = bm.N
    free = list(bm.free)
    assert len(set(free)) == len(free)
    refs = [0] * N
    for s, t in bm.tables.items():
        assert len(t) == -(-bm.lens[s] // bm.BS)
        for b in t:
            refs[b] += 1
    assert refs == [bm.refcount(b) for b in range(N)]
    for b in free:
        assert refs[b] == 0
    evictable = list(getattr(bm, "evictable", []))
    assert len(free) + len(evictable) + sum(1 for r in refs if r > 0) == N
    # cached blocks: the key map and the block map agree; an evictable block is
    # cached and unreferenced; a block on the free stack is not cached
    block_key = getattr(bm, "block_key", {})
    for b, key in block_key.items():
        assert bm.cache[key][1] == b
    assert len(block_key) == len(getattr(bm, "cache", {}))
    for b in evictable:
        assert refs[b] == 0 and b in block_key
    for b in free:
        assert b not in block_key
    # a swapped-out sequence holds no block and is not live
    assert not set(getattr(bm, "swapped", {})) & set(bm.tables)


# ------------------------------------------------------------------- cache
def check_layout_golden(Cache):
    """Hand-computed element offsets (tests/golden/layout_tiny.json)."""
    g = load_golden("layout_tiny.json")
    p = g["pool"]
    for c in g["cases"]:
        cm = Cache(p["num_blocks"], p["num_kv_heads"], p["head_dim"], p["block_size"], p["dtype"])
        k = np.zeros((1, p["num_kv_heads"], p["head_dim"]), np.float32)
        v = np.zeros_like(k)
        k[0, c["head"], c["d"]] = 3.0
        v[0, c["head"], c["d"]] = -2.0
        cm.write([c["slot"]], k, v)
        kb, vb = cm.pool_bits()
        kf, vf = kb.reshape(-1), vb.reshape(-1)
        assert int(np.flatnonzero(kf == 0x4040)[0]) == c["k_offset"]      # bf16 3.0
        assert int(np.flatnonzero(vf == 0xC000)[0]) == c["v_offset"]      # bf16 -2.0
        # the write touched exactly the token's own elements (2 heads x 16 dims)
        assert int(np.sum(kf != 0x7FC0)) == p["num_kv_heads"] * p["head_dim"]


def check_paged_equals_contiguous(Cache, dtype):
    """Scatter tokens through a shuffled slot list, gather them back through
    the table: bit-identical to the contiguous rows; negative slots skipped."""
    import workloads as W
    rng = np.random.default_rng(21)
    N, H, D, BS = 12, 3, 64, 8
    cm = Cache(N, H, D, BS, dtype)
    blocks = rng.permutation(N)[:5]
    n = 37
    slots = np.array([blocks[t // BS] * BS + t % BS for t in range(n)])
    k = W.round_to_dtype(rng.standard_normal((n, H, D)).astype(np.float32), dtype)
    v = W.round_to_dtype(rng.standard_normal((n, H, D)).astype(np.float32), dtype)
    order = rng.permutation(n)
    sl = slots[order].copy()
    sl[::5] = -1                          # skipped
    cm.write(sl, k[order], v[order])
    cm.write(slots[order][::5], k[order][::5], v[order][::5])
    K, V = cm.gather(list(blocks), n)
    assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, v.astype(np.float64))


def check_copy_blocks(Cache):
    """A copy moves the whole block (every head, padding included) and
    nothing else."""
    rng = np.random.default_rng(22)
    cm = Cache(6, 2, 16, 4, "f16")
    x = rng.standard_normal((3, 2, 16)).astype(np.float16).astype(np.float32)
    cm.write([4, 5, 6], x, -x)             # block 1, offsets 0..2 (offset 3 stays poison)
    k0, v0 = (a.copy() for a in cm.pool_bits())
    cm.copy_blocks([(1, 3)])
    k1, v1 = cm.pool_bits()
    assert np.array_equal(k1[3], k0[1]) and np.array_equal(v1[3], v0[1])
    others = [b for b in range(6) if b != 3]
    assert np.array_equal(k1[others], k0[others]) and np.array_equal(v1[others], v0[others])


def check_bm_swap(BM, OutOfBlocks, InvalidOp):
    """Preemption by swap, hand-traced on tiny pools (LIFO free stack, blocks
    released in logical order, fresh blocks taken in logical order)."""
    bm = BM(6, 4)
    assert bm.add_seq(0, 10)[:5] == [0, 1, 2, 3, 4]           # table [0, 1, 2]
    assert bm.swap_out(0) == [0, 1, 2]
    assert bm.num_free() == 6 and bm.swapped == {0: 10}
    for bad in (lambda: bm.add_seq(0, 1), lambda: bm.swap_out(0), lambda: bm.append([0])):
        try:
            bad()
            raise AssertionError("a swapped-out id must be rejected")
        except InvalidOp:
            pass
    bm.add_seq(1, 1)                                          # takes block 2 (top of the stack)
    try:
        bm.fork(1, 0)
        raise AssertionError("fork onto a swapped-out id must be rejected")
    except InvalidOp:
        pass
    assert bm.swap_in(0) == [1, 0, 3]                         # next three on the stack
    assert bm.lens[0] == 10 and bm.swapped == {}
    assert bm.tables[0] == [1, 0, 3]

    # a shared block stays resident for its other sharer; it comes back private
    bm = BM(5, 4)
    bm.add_seq(1, 8)                                          # [0, 1]
    bm.fork(1, 2)
    assert bm.swap_out(1) == [0, 1]
    assert [bm.refcount(b) for b in range(5)] == [1, 1, 0, 0, 0] and bm.num_free() == 3
    assert bm.swap_in(1) == [2, 3]
    assert [bm.refcount(b) for b in range(5)] == [1, 1, 1, 1, 0]
    assert bm.tables[2] == [0, 1]

    # all or nothing when the pool is short
    bm = BM(3, 4)
    bm.add_seq(1, 12)                                         # [0, 1, 2]
    bm.swap_out(1)                                            # stack bottom..top = 0, 1, 2
    bm.add_seq(2, 5)                                          # [2, 1]
    snap = (list(bm.free), [bm.refcount(b) for b in range(3)], dict(bm.swapped))
    try:
        bm.swap_in(1)
        raise AssertionError("swap_in must fail without three free blocks")
    except OutOfBlocks:
        pass
    assert snap == (list(bm.free), [bm.refcount(b) for b in range(3)], dict(bm.swapped))
    bm.free_seq(2)
    assert bm.swap_in(1) == [1, 2, 0]

    # an empty sequence swaps without blocks
    bm = BM(2, 4)
    bm.add_seq(5, 0)
    assert bm.swap_out(5) == [] and bm.swapped == {5: 0}
    assert bm.swap_in(5) == [] and bm.lens[5] == 0


def check_bm_prefix_cache(BM, OutOfBlocks, InvalidOp):
    """Prefix caching, hand-traced on an 8-block pool of 4-token blocks
    (identity order: the free stack hands out 0, 1, 2, ... first)."""
    bm = BM(8, 4)
    A = list(range(1, 11))                                    # tokens 1..10: two full blocks + 2
    slots, hit = bm.add_seq_cached(1, A)
    assert (slots, hit) == (list(range(10)), 0)               # blocks 0, 1, 2; blocks 0 and 1 cached
    slots, hit = bm.add_seq_cached(2, A[:8] + [20, 21, 22])   # same first 8 tokens
    assert hit == 8 and bm.tables[2] == [0, 1, 3] and slots[8:] == [12, 13, 14]
    assert [bm.refcount(b) for b in (0, 1, 2, 3)] == [2, 2, 1, 1]
    slots, hit = bm.add_seq_cached(3, A[:4])                  # one full block, holds the last token
    assert hit == 0 and bm.tables[3] == [4]                   # never reused; its key is taken already
    assert tuple(bm.cache_stats()) == (2, 0, 2, 4)
    try:
        bm.add_seq_cached(3, A)
        raise AssertionError("a live id must be rejected")
    except InvalidOp:
        pass

    bm.free_seq(1)                                            # block 2 -> free stack
    bm.free_seq(2)                                            # 3 -> free stack; 1, 0 evictable
    assert bm.num_free() == 7 and tuple(bm.cache_stats())[:2] == (2, 2)
    slots, hit = bm.add_seq_cached(4, A[:9])                  # revives 0 and 1 from the evictable list
    assert hit == 8 and bm.tables[4] == [0, 1, 3]
    bm.free_seq(4)                                            # 1, 0 evictable again (1 oldest)
    bm.add_seq(5, 24)                                         # 5 free + evicts block 1 (drops its key)
    assert bm.tables[5] == [3, 2, 5, 6, 7, 1]
    assert tuple(bm.cache_stats())[:2] == (1, 1)

    snap = ([bm.refcount(b) for b in range(8)], bm.num_free(), tuple(bm.cache_stats()))
    try:
        bm.add_seq_cached(6, A[:9])                           # would revive 0 and need two more
        raise AssertionError("expected OutOfBlocks")
    except OutOfBlocks:
        pass
    try:
        bm.add_seq_cached(6, A[:5])                           # the only evictable block is its own hit
        raise AssertionError("expected OutOfBlocks")
    except OutOfBlocks:
        pass
    assert snap == ([bm.refcount(b) for b in range(8)], bm.num_free(), tuple(bm.cache_stats()))
    bm.free_seq(5)                                            # stack bottom..top: 3 2 5 6 7 1
    slots, hit = bm.add_seq_cached(6, A[:9])
    assert hit == 4 and bm.tables[6] == [0, 1, 7]             # block 1 cached again under a new id
    slots, hit = bm.add_seq_cached(8, A[:8])                  # two full blocks: only the first is looked up
    assert hit == 4 and bm.tables[8] == [0, 6]
    assert tuple(bm.cache_stats()) == (2, 0, 2 + 2 + 1 + 1, 4 + 2 + 2 + 1)
    # a block's tokens alone do not make a hit: tokens 5..8 are cached only
    # after tokens 1..4
    _, hit = bm.add_seq_cached(10, A[4:8] + [0])
    assert hit == 0 and bm.tables[10] == [5, 2]
    assert tuple(bm.cache_stats()) == (3, 0, 6, 10)

    for seq in (6, 8, 3, 10):
        bm.free_seq(seq)
    assert tuple(bm.cache_stats())[:2] == (3, 3) and bm.num_free() == 8
    bm.cache_clear()
    assert tuple(bm.cache_stats())[:2] == (0, 0) and bm.num_free() == 8
    _, hit = bm.add_seq_cached(9, A)
    assert hit == 0


# ------------------------------------------------- accounting (waste, admission)
def check_admit_golden(admit):
    """Hand-worked admission cases (tests/golden/admit_hand.json): the ceiling
    exactly reached, one block over, the reserve pushing a request over, the
    empty request, and a length that is not a multiple of the block size."""
    g = load_golden("admit_hand.json")
    for free, tokens, bs, reserve, want, why in g["cases"]:
        assert admit(free, tokens, bs, reserve) is want, why


def check_slab_golden(Slab):
    """Hand-traced contiguous reservations (tests/golden/
    slab_fragmentation_hand.json): first fit, merging on release, and a
    refusal while the free total would cover the request."""
    g = load_golden("slab_fragmentation_hand.json")
    s = Slab(g["capacity"])
    ids, with_room = {}, []
    for op in g["ops"]:
        if op[0] == "reserve":
            name, n = op[1], op[2]
            ids[name] = len(ids)
            room = s.free_slots() >= n
            start = s.reserve(ids[name], n)
            assert start == g["starts"][name], (name, start)
            if start is None and room:
                with_room.append(name)
        else:
            s.release(ids[op[1]])
    assert with_room == g["refused_with_room"]
    assert [list(h) for h in s.holes] == g["final_holes"]


def check_slab_invariants(Slab):
    """Random reservations and releases: the free runs and the reserved runs
    tile the pool exactly, free runs are sorted and never touch, a request
    is refused only when no free run is long enough, and releasing
    everything leaves one run of the whole pool."""
    rng = np.random.default_rng(41)
    cap = 97
    s = Slab(cap)
    live = []
    for k in range(600):
        if live and rng.random() < 0.45:
            s.release(live.pop(int(rng.integers(len(live)))))
        else:
            n = int(rng.integers(1, 20))
            longest = max((h[1] for h in s.holes), default=0)
            first = next((h[0] for h in s.holes if h[1] >= n), None)
            start = s.reserve(k, n)
            assert start == first and (start is None) == (longest < n)
            if start is not None:
                live.append(k)
        cover = np.zeros(cap, np.int64)
        for st, n in s.runs.values():
            cover[st:st + n] += 1
        for st, n in s.holes:
            assert n > 0
            cover[st:st + n] += 1
        assert np.all(cover == 1)
        starts = [h[0] for h in s.holes]
        assert starts == sorted(starts)
        assert all(a[0] + a[1] < b[0] for a, b in zip(s.holes, s.holes[1:]))
        assert s.free_slots() == cap - sum(n for _, n in s.runs.values())
    for rid in list(live):
        s.release(rid)
    assert [list(h) for h in s.holes] == [[0, cap]]


def check_replay_golden(replay):
    """One trace replayed by hand against contiguous runs of the request's
    length, of the longest context, and blocks from a free list
    (tests/golden/admission_replay_hand.json)."""
    from fractions import Fraction
    g = load_golden("admission_replay_hand.json")
    ev = [tuple(e) for e in g["events"]]
    for pol, e in g["expected"].items():
        r = replay(ev, pol, g["capacity_tokens"], g["block_size"], g["max_len"])
        for k in ("admitted", "refused", "refused_with_room", "peak_live"):
            assert r[k] == e[k], (pol, k, r[k], e[k])
        for k in ("mean_live", "reserved_unused", "used_fraction"):
            assert abs(r[k] - float(Fraction(*e[k]))) < 1e-12, (pol, k, r[k], e[k])


def check_replay_invariants(replay):
    """What the pages fix about the three pools on a churning trace: blocks
    from a free list are refused only when too few are free (never with room
    to spare); a pool that holds every request at once refuses nothing; with
    every request of one length, contiguous runs of that length do not
    fragment either; reserving the longest context leaves most of each
    reservation unused when requests are short."""
    rng = np.random.default_rng(43)
    n = 400
    lens = rng.integers(1, 65, size=n)
    life = rng.integers(1, 60, size=n)
    ev, by = [], {}
    for i in range(n):
        by.setdefault(i + int(life[i]), []).append(i)
    for t in range(n):
        ev += [("depart", i) for i in by.get(t, [])]
        ev.append(("arrive", t, int(lens[t])))
    cap = 16 * 32 * 16
    paged = replay(ev, "paged", 900, 4, 64)
    assert paged["refused"] > 0 and paged["refused_with_room"] == 0
    exact = replay(ev, "slab_exact", 900, 4, 64)
    assert exact["refused_with_room"] > 0
    for pol in ("paged", "slab_exact"):
        assert replay(ev, pol, int(lens.sum()) + 64, 4, 64)["refused"] == 0
    same = [e if e[0] == "depart" else ("arrive", e[1], 8) for e in ev]
    assert replay(same, "slab_exact", 900, 4, 64)["refused_with_room"] == 0
    mx = replay(ev, "slab_max", cap, 4, 64)
    assert mx["reserved_unused"] > 0.4 and paged["reserved_unused"] < 0.1
