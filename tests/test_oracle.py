"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from oracle import attention as A
from oracle.block_manager import BlockManagerModel, InvalidOp, OutOfBlocks
from oracle.cache import PagedCacheModel

import oracle_pins as P
from scenarios import fork_workload


@pytest.mark.parametrize("check", P.ATTN_CHECKS, ids=lambda f: f.__name__)
def test_attention_pins(check):
    check(A.decode_attention)


@pytest.mark.parametrize("check", P.ATTN_CHECKS, ids=lambda f: f.__name__)
def test_split_attention_pins(check):
    """The split-K form passes the same pins for several partition sizes."""
    for part in (1, 3, 16, 512):
        check(lambda q, K, V, s: A.decode_attention_split(q, K, V, s, part))


def test_split_merge():
    P.check_split_merge(A.split_k, A.lse_merge, A.decode_attention)


def test_block_manager_golden():
    P.check_bm_golden(BlockManagerModel, OutOfBlocks)


def test_layout_golden():
    P.check_layout_golden(PagedCacheModel)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_paged_equals_contiguous(dtype):
    P.check_paged_equals_contiguous(PagedCacheModel, dtype)


def test_copy_blocks():
    P.check_copy_blocks(PagedCacheModel)


# ------------------------------------------------------ block manager model
def test_bm_errors_change_nothing():
    bm = BlockManagerModel(4, 4)
    bm.add_seq(1, 9)                       # 3 blocks
    snap = (list(bm.free), list(bm.rc), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))
    with pytest.raises(OutOfBlocks):
        bm.add_seq(2, 5)
    with pytest.raises(InvalidOp):
        bm.add_seq(1, 1)
    with pytest.raises(InvalidOp):
        bm.free_seq(7)
    with pytest.raises(InvalidOp):
        bm.fork(7, 8)
    with pytest.raises(InvalidOp):
        bm.append([1, 1])
    bm.add_seq(3, 4)                       # last free block
    bm.fork(3, 4)
    snap = (list(bm.free), list(bm.rc), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))
    with pytest.raises(OutOfBlocks):       # seq 1 needs no block, seq 3 needs one
        bm.append([1, 3])
    assert snap == (list(bm.free), list(bm.rc), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))


def test_bm_swap_pins():
    P.check_bm_swap(BlockManagerModel, OutOfBlocks, InvalidOp)


def test_bm_prefix_cache_pins():
    P.check_bm_prefix_cache(BlockManagerModel, OutOfBlocks, InvalidOp)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 5), st.integers(0, 7), st.integers(0, 40)), max_size=60),
       st.sampled_from([1, 2, 4]))
def test_prefix_cache_reuses_only_identical_prefixes(ops, bs):
    """Brute force over the whole history: a reused block was first filled
    by a sequence whose tokens up to that block's end equal the new prompt's
    (the K/V a block holds is a function of that prefix), and the reuse stops
    before the block of the last token."""
    bm = BlockManagerModel(20, bs, list(reversed(range(20))))
    filled = {}                  # block -> prefix of tokens it was filled under (None: uncached content)
    prompts = [[(3 * i) % 5 for i in range(40)], [(3 * i) % 5 for i in range(6)] + [4] * 34]
    for kind, seq, n in ops:
        try:
            if kind <= 2:
                toks = prompts[kind % 2][: n % 30]
                slots, hit = bm.add_seq_cached(seq, toks)
                assert hit % bs == 0 and (hit < len(toks) or len(toks) == 0)
                table = bm.table(seq)
                for i, b in enumerate(table):
                    pre = tuple(toks[: (i + 1) * bs])
                    if i < hit // bs:
                        assert filled[b] == pre
                    else:
                        filled[b] = pre if (i + 1) * bs <= len(toks) else None
            elif kind == 3:
                bm.free_seq(seq)
            elif kind == 4:
                bm.add_seq(seq, n % 20)
                for b in bm.table(seq):
                    filled[b] = None
            else:
                bm.append([seq])
                filled[bm.table(seq)[-1]] = None
        except (OutOfBlocks, InvalidOp):
            pass
        P.bm_invariants(bm)


def test_swap_round_trip_restores_the_sequence():
    """Swap a sequence out (blocks copied to host arrays), let another
    sequence take and overwrite its blocks, swap it back into fresh blocks:
    its gathered K/V and its decode output are unchanged."""
    rng = np.random.default_rng(3)
    H, D, BS, N = 2, 16, 4, 8
    cache = PagedCacheModel(N, H, D, BS, "bf16")
    bm = BlockManagerModel(N, BS, rng.permutation(N))
    k = W.round_to_dtype(rng.standard_normal((11, H, D), dtype=np.float32), "bf16")
    v = W.round_to_dtype(rng.standard_normal((11, H, D), dtype=np.float32), "bf16")
    cache.write(bm.add_seq(0, 11), k, v)
    q = rng.standard_normal((H, D))
    k0, v0 = cache.gather(bm.table(0), 11)
    ref = A.decode_attention(q, k0, v0, 0.25)
    blocks = bm.swap_out(0)
    host_k, host_v = cache.k[blocks].copy(), cache.v[blocks].copy()
    other = bm.add_seq(1, N * BS)                              # every block, overwritten
    cache.write(other, np.ones((N * BS, H, D), np.float32), -np.ones((N * BS, H, D), np.float32))
    bm.free_seq(1)
    fresh = bm.swap_in(0)
    assert fresh != blocks
    cache.k[fresh], cache.v[fresh] = host_k, host_v
    k1, v1 = cache.gather(bm.table(0), 11)
    assert np.array_equal(k1, k0) and np.array_equal(v1, v0)
    assert np.array_equal(A.decode_attention(q, k1, v1, 0.25), ref)


def test_bm_interchangeable_blocks_after_churn():
    """Every free block is interchangeable: after any churn an allocation of
    k blocks succeeds exactly when k <= num_free."""
    rng = np.random.default_rng(3)
    bm = BlockManagerModel(64, 16, rng.permutation(64))
    live = []
    for i in range(2000):
        if rng.random() < 0.55 and bm.num_free():
            n = int(rng.integers(1, 16 * bm.num_free() + 1))
            bm.add_seq(i, n)
            live.append(i)
        elif live:
            bm.free_seq(live.pop(int(rng.integers(len(live)))))
        P.bm_invariants(bm)
    free = bm.num_free()
    with pytest.raises(OutOfBlocks):
        bm.add_seq(10**6, 16 * free + 1)
    bm.add_seq(10**6, 16 * free)
    assert bm.num_free() == 0


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 6), st.integers(0, 7), st.integers(0, 40)), max_size=60),
       st.sampled_from([1, 4, 8]))
def test_bm_random_ops_keep_invariants(ops, bs):
    bm = BlockManagerModel(24, bs, list(reversed(range(24))))
    for kind, seq, n in ops:
        try:
            if kind == 0:
                bm.add_seq(seq, n % 20)
            elif kind == 1:
                bm.append([s for s in sorted(bm.tables) if (s + n) % 3 == 0])
            elif kind == 2:
                bm.fork(seq, (seq + n) % 8)
            elif kind == 3:
                bm.free_seq(seq)
            elif kind == 5:
                bm.swap_out(seq)
            elif kind == 6:
                bm.swap_in(seq)
            else:
                bm.append([seq])
        except (OutOfBlocks, InvalidOp):
            pass
        P.bm_invariants(bm)


# ----------------------------------------------------- scenario-level pins
def _tiny(**kw):
    return W.tiny(**kw)


def test_scenario_paged_equals_contiguous_attention():
    """Outputs over the pool equal attention over the workload's own
    contiguous rows (the gather is exact)."""
    w = _tiny(num_seqs=4, ctx=[1, 16, 17, 70], block_size=16, dtype="bf16", seed=1)
    r = oracle.run_scenario(w)
    d = r.decodes[-1]
    for j, s in enumerate(d.seqs):
        rows = w.row_of(s, np.arange(int(w.ctx[s])))
        ref = A.decode_attention(w.q_sets[0][s], w.k_rows[rows], w.v_rows[rows], w.cfg.scale)
        assert np.array_equal(d.out[j], ref)


def test_scenario_permutation_invariance():
    """Blocks may sit anywhere in any order: permuting physical blocks leaves
    the outputs bit-identical and changes the tables."""
    a = oracle.run_scenario(_tiny(ctx=[5, 40, 33], seed=2, permute=False))
    b = oracle.run_scenario(_tiny(ctx=[5, 40, 33], seed=2, permute=True))
    assert not np.array_equal(a.decodes[-1].tables, b.decodes[-1].tables)
    assert np.array_equal(a.decodes[-1].out, b.decodes[-1].out)


def _fork_workload(prefix, suffix, share: bool):
    return fork_workload(prefix, suffix, share)


def test_scenario_shared_equals_unshared():
    """Tables pointing at one physical prefix copy give the same outputs as
    private copies, bit for bit; the shared run uses fewer blocks."""
    for prefix in (16, 13):             # block-aligned prefix, and a partial shared block
        suffix = [1, 3, 9, 20]
        a = oracle.run_scenario(_fork_workload(prefix, suffix, share=True))
        b = oracle.run_scenario(_fork_workload(prefix, suffix, share=False))
        assert np.array_equal(a.decodes[-1].out, b.decodes[-1].out)
        assert a.bm.num_free() > b.bm.num_free()
        cows = sum(len(x["pairs"]) for x in a.appends)
        assert cows == (len(suffix) - 1 if prefix % 8 else 0)


def test_scenario_cow_isolation():
    """Copy-on-write gives the writer its own copy: the block the others still
    share is bit-identical before and after, and so are their outputs."""
    w = _fork_workload(13, [0, 0, 0], share=True)
    w.ops = w.ops[:4] + [("decode", [0, 1, 2], 0)]          # create, add, 2 forks, decode
    r0 = oracle.run_scenario(w)
    shared_last = r0.bm.table(0)[-1]
    k_before = r0.cache.k[shared_last].copy()
    v_before = r0.cache.v[shared_last].copy()
    w.ops = w.ops[:4] + [("append", [1]), ("decode", [0, 2], 0)]
    r1 = oracle.run_scenario(w)
    assert r1.appends[0]["pairs"] == [(shared_last, r1.bm.table(1)[-1])]
    assert np.array_equal(r1.cache.k[shared_last], k_before)
    assert np.array_equal(r1.cache.v[shared_last], v_before)
    assert np.array_equal(r1.decodes[-1].out, r0.decodes[-1].out[[0, 2]])
    assert r1.bm.refcount(shared_last) == 2


# ------------------------------------------------------ workload scripts
def test_c1_construction():
    w = W.build("c1_tiny_f32")
    r = oracle.run_scenario(w)
    assert r.bm.N - r.bm.num_free() == 29
    d = r.decodes[-1]
    assert d.ctx.tolist() == [17, 64, 100, 255]
    order = w.ops[0][2]
    # prefill takes order[0..27] by sequence then block; the decode step's
    # block for sequence 0 (position 16 starts a block) is order[28]
    assert d.tables[0, :2].tolist() == [order[0], order[28]]
    assert d.tables[3, :16].tolist() == list(order[12:28])


@pytest.mark.parametrize("name", ["c2_gqa_bf16_bs8", "c2_gqa_bf16", "c2_gqa_bf16_bs32", "c5_long_splitk"])
def test_uniform_constructions(name):
    w = W.build(name, values=False)
    r = oracle.run_scenario(w, outputs=False, cache=False)
    bs = w.cfg.block_size
    need = int(np.sum(-(-w.ctx // bs)))
    assert r.bm.N == int(np.ceil(1.2 * need)) and r.bm.N - r.bm.num_free() == need
    assert r.decodes[-1].ctx.tolist() == w.ctx.tolist()
    P.bm_invariants(r.bm)


def test_c3_churn_construction():
    w = W.build("c3_mha_f16_churn", values=False)
    assert w.ctx.min() >= 1 and w.ctx.max() <= 4096
    assert 380 < w.ctx.mean() < 650          # lognormal mean 512 before clipping
    r = oracle.run_scenario(w, outputs=False, cache=False)
    P.bm_invariants(r.bm)
    need = int(np.sum(-(-w.ctx // 16)))
    assert r.bm.N - r.bm.num_free() == need
    # the churn scattered the batch: tables are far from the identity layout
    t = r.decodes[-1].tables
    first = t[:, 0]
    assert np.mean(np.diff(first) == 1) < 0.5


@pytest.mark.parametrize("name", ["c4a_prefix_share", "c4b_prefix_cow"])
def test_c4_construction(name):
    w = W.build(name, values=False)
    r = oracle.run_scenario(w, outputs=False, cache=False)
    P.bm_invariants(r.bm)
    pairs = [p for a in r.appends for p in a["pairs"]]
    tabs = r.decodes[-1].tables
    if name == "c4a_prefix_share":
        assert pairs == []
        assert all(r.bm.refcount(int(b)) == 64 for b in tabs[0, :128])
    else:
        first = r.appends[0]
        assert len(first["pairs"]) == 63 and len(pairs) == 63
        src = {p[0] for p in first["pairs"]}
        assert len(src) == 1 and tabs[63, 127] == next(iter(src))       # last sharer in place
        assert all(r.bm.refcount(int(b)) == 64 for b in tabs[0, :127])
    assert r.decodes[-1].ctx.tolist() == w.ctx.tolist()


# ----------------------------------------------------------------- prefill
def _masked_prefill(Q, K, V, scale):
    """Independent formulation: the whole L x n score matrix per query head,
    an explicit causal mask, a row softmax and one product with V."""
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    L, Hq, D = Q.shape
    n, Hkv, _ = K.shape
    g = Hq // Hkv
    pos = n - L + np.arange(L)
    out = np.zeros_like(Q)
    for r in range(Hq):
        S = Q[:, r, :] @ K[:, r // g, :].T * scale            # [L, n]
        S[np.arange(n)[None, :] > pos[:, None]] = -np.inf
        P = np.exp(S - S.max(axis=1, keepdims=True))
        out[:, r, :] = (P / P.sum(axis=1, keepdims=True)) @ V[:, r // g, :]
    return out


@pytest.mark.parametrize("L,n,hq,hkv", [(1, 1, 2, 1), (5, 5, 4, 2), (3, 9, 8, 2), (7, 20, 4, 4)])
def test_prefill_oracle_matches_masked_matrix(L, n, hq, hkv):
    """Row by row decode over growing prefixes equals the masked score matrix
    (a chunk at the end of its context; the whole prompt when L = n)."""
    rng = np.random.default_rng([L, n, hq])
    D = 8
    Q = rng.standard_normal((L, hq, D))
    K = rng.standard_normal((n, hkv, D))
    V = rng.standard_normal((n, hkv, D))
    got = oracle.prefill_attention(Q, K, V, 0.35)
    assert np.allclose(got, _masked_prefill(Q, K, V, 0.35), rtol=0, atol=1e-12)


def test_prefill_first_token_sees_only_itself():
    """The first token of a fresh prompt attends to position 0 alone: its
    output is V[0] exactly, whatever the scores; the last row equals decode
    over the whole context."""
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((6, 4, 8)) * 50
    K = rng.standard_normal((6, 2, 8))
    V = rng.standard_normal((6, 2, 8))
    out = oracle.prefill_attention(Q, K, V, 1.0)
    assert np.array_equal(out[0], np.repeat(V[0], 2, axis=0))
    assert np.array_equal(out[-1], oracle.decode_attention(Q[-1], K, V, 1.0))
    with pytest.raises(ValueError):
        oracle.prefill_attention(Q, K[:3], V[:3], 1.0)
