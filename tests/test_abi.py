"""The C ABI without a GPU: symbols, the C++ block manager (bit-exact with the
oracle's model) and host-side argument validation."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from oracle.block_manager import BlockManagerModel, InvalidOp, OutOfBlocks

import oracle_pins as P

pa = pytest.importorskip("paged_kv_cache_332_amd", reason="libpa.so not built")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 20
    lib = ctypes.CDLL(pa.LIB_PATH)
    missing = [s for s in syms if not hasattr(lib, s)]
    assert not missing, missing
    assert pa.pa_version().startswith("pa ")


# ----------------------------------------------------------- block manager
class CppBM:
    """The C++ manager behind the model's interface, for the shared pins."""

    def __init__(self, num_blocks, block_size, order=None):
        self.N, self.BS = num_blocks, block_size
        self.m = pa.BlockManager(num_blocks, block_size, order)
        self._seqs = set()
        self._swapped = set()

    def _wrap(self, fn, *a):
        try:
            return fn(*a)
        except pa.OutOfBlocks as e:
            raise OutOfBlocks() from e
        except pa.PAError as e:
            raise InvalidOp(str(e)) from e

    def add_seq(self, seq, n):
        out = list(self._wrap(self.m.add_seq, seq, n))
        self._seqs.add(seq)
        return out

    def append(self, seqs):
        slots, pairs = self._wrap(self.m.append_slots, list(seqs))
        return list(slots), [tuple(p) for p in pairs.tolist()]

    def fork(self, parent, child):
        self._wrap(self.m.fork, parent, child)
        self._seqs.add(child)

    def free_seq(self, seq):
        self._wrap(self.m.free_seq, seq)
        self._seqs.discard(seq)

    def swap_out(self, seq):
        out = [int(b) for b in self._wrap(self.m.swap_out, seq)]
        self._seqs.discard(seq)
        self._swapped.add(seq)
        return out

    def swap_in(self, seq):
        out = [int(b) for b in self._wrap(self.m.swap_in, seq)]
        self._swapped.discard(seq)
        self._seqs.add(seq)
        return out

    @property
    def swapped(self):
        return {s: self.m.swapped_len(s) for s in self._swapped}

    def add_seq_cached(self, seq, tokens):
        slots, hit = self._wrap(self.m.add_seq_cached, seq, tokens)
        self._seqs.add(seq)
        return [int(x) for x in slots], hit

    def cache_stats(self):
        return self.m.cache_stats()

    def cache_clear(self):
        self.m.cache_clear()

    def export(self, seqs, stride):
        return self._wrap(self.m.export, list(seqs), stride)

    def num_free(self):
        return self.m.num_free()

    def refcount(self, b):
        return self.m.refcount(b)

    def table(self, seq):
        n = self.m.seq_len(seq)
        tab, _ = self.m.export([seq], max(1, -(-n // self.BS)))
        return [int(x) for x in tab[0] if x >= 0]

    def stats(self):
        return self.m.stats()

    @property
    def free(self):
        return list(reversed(self.m.free_list().tolist()))

    @property
    def rc(self):
        return [self.m.refcount(b) for b in range(self.N)]

    @property
    def tables(self):
        return {s: self.table(s) for s in self._seqs}

    @property
    def lens(self):
        return {s: self.m.seq_len(s) for s in self._seqs}


def test_cpp_block_manager_golden():
    P.check_bm_golden(CppBM, OutOfBlocks)


def test_cpp_block_manager_swap():
    P.check_bm_swap(CppBM, OutOfBlocks, InvalidOp)


def test_cpp_block_manager_prefix_cache():
    P.check_bm_prefix_cache(CppBM, OutOfBlocks, InvalidOp)


def _prompt(kind, n, bs):
    """Prompts from a few shared prefixes so that lookups hit, miss and
    diverge part-way (token ids 0..3 only)."""
    base = [(7 * i + kind) % 4 for i in range(64)]
    fork = n % 5
    return base[: max(0, n - fork)] + [(kind + j) % 4 for j in range(fork)]


@settings(max_examples=120, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 8), st.integers(0, 9), st.integers(0, 40)), max_size=60),
       st.sampled_from([1, 2, 4, 8]), st.integers(0, 2**31 - 1))
def test_cpp_matches_model_with_prefix_cache(ops, bs, seed):
    """Every operation, cached adds and evictions included, leaves the C++
    manager and the model in the same state with the same results."""
    order = list(np.random.default_rng(seed).permutation(16))
    cpp, model = CppBM(16, bs, order), BlockManagerModel(16, bs, order)
    for kind, seq, n in ops:
        results = []
        for bm in (cpp, model):
            try:
                if kind in (0, 7, 8):
                    r = bm.add_seq_cached(seq, _prompt(kind % 2, n % 30, bs))
                elif kind == 1:
                    r = bm.append([s for s in sorted(model.tables) if (s + n) % 3 == 0])
                elif kind == 2:
                    r = bm.fork(seq, (seq + n) % 10)
                elif kind == 3:
                    r = bm.free_seq(seq)
                elif kind == 4:
                    r = bm.add_seq(seq, n % 20)
                elif kind == 5:
                    r = bm.swap_out(seq)
                else:
                    r = bm.swap_in(seq) if n % 7 else bm.cache_clear()
                results.append(("ok", r))
            except OutOfBlocks:
                results.append(("oom", None))
            except InvalidOp:
                results.append(("invalid", None))
        assert results[0][0] == results[1][0], (kind, results)
        if results[0][0] == "ok" and results[0][1] is not None:
            a, b = results[0][1], results[1][1]
            if kind == 1:
                assert list(a[0]) == list(b[0]) and [tuple(x) for x in a[1]] == [tuple(x) for x in b[1]]
            elif kind in (0, 7, 8):
                assert list(a[0]) == list(b[0]) and a[1] == b[1]
            else:
                assert list(a) == list(b)
        _same_state(cpp, model)
        P.bm_invariants(model)


def test_cpp_create_rejects_bad_order():
    with pytest.raises(pa.PAError):
        pa.BlockManager(4, 16, [0, 1, 1, 2])
    with pytest.raises(pa.PAError):
        pa.BlockManager(4, 0)


def _same_state(cpp: CppBM, model: BlockManagerModel):
    assert cpp.free == model.free
    assert cpp.rc == model.rc
    assert cpp.tables == {s: t for s, t in model.tables.items()}
    assert cpp.lens == model.lens
    assert cpp.swapped == model.swapped
    assert tuple(cpp.cache_stats()) == tuple(model.cache_stats())
    assert cpp.num_free() == model.num_free()
    assert tuple(cpp.stats()) == tuple(model.stats())
    # the shared prefix the C++ manager keeps per sequence (and walks again
    # only after a sharing change) against its definition on the model's
    # state: leading table entries whose refcount is above one
    for s, t in model.tables.items():
        k = 0
        while k < len(t) and model.rc[t[k]] > 1:
            k += 1
        assert cpp.m.shared_blocks(s) == k, (s, t, cpp.m.shared_blocks(s), k)
    assert cpp.m.shared_blocks(10 ** 6) == -1


@settings(max_examples=80, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 6), st.integers(0, 7), st.integers(0, 40)), max_size=50),
       st.sampled_from([1, 4, 8, 16]), st.integers(0, 2**31 - 1))
def test_cpp_matches_model_on_random_ops(ops, bs, seed):
    order = list(np.random.default_rng(seed).permutation(20))
    cpp, model = CppBM(20, bs, order), BlockManagerModel(20, bs, order)
    for kind, seq, n in ops:
        results = []
        for bm in (cpp, model):
            try:
                if kind == 0:
                    r = bm.add_seq(seq, n % 24)
                elif kind == 1:
                    r = bm.append([s for s in sorted(model.tables) if (s + n) % 3 == 0])
                elif kind == 2:
                    r = bm.fork(seq, (seq + n) % 8)
                elif kind == 3:
                    r = bm.free_seq(seq)
                elif kind == 5:
                    r = bm.swap_out(seq)
                elif kind == 6:
                    r = bm.swap_in(seq)
                else:
                    r = bm.append([seq])
                results.append(("ok", r))
            except OutOfBlocks:
                results.append(("oom", None))
            except InvalidOp:
                results.append(("invalid", None))
        assert results[0][0] == results[1][0]
        if results[0][0] == "ok" and results[0][1] is not None:
            a, b = results[0][1], results[1][1]
            if kind in (1, 4):
                assert list(a[0]) == list(b[0]) and [tuple(x) for x in a[1]] == [tuple(x) for x in b[1]]
            else:
                assert list(a) == list(b)
        _same_state(cpp, model)


def _replay_cpp(w):
    """The construction script on the C++ manager (no device work)."""
    bm = None
    appends, decodes = [], []
    stride = oracle.scenario.table_stride(w)
    for op in w.ops:
        k = op[0]
        if k == "create":
            bm = pa.BlockManager(op[1], w.cfg.block_size, op[2])
        elif k == "add_seq":
            bm.add_seq(op[1], op[2])
        elif k == "fork":
            bm.fork(op[1], op[2])
        elif k == "free_seq":
            bm.free_seq(op[1])
        elif k == "append":
            slots, pairs = bm.append_slots(op[1])
            appends.append((list(slots), [tuple(p) for p in pairs.tolist()]))
        elif k == "decode":
            decodes.append(bm.export(op[1], stride))
    return bm, appends, decodes


@pytest.mark.parametrize("name", sorted(W.CONFIGS))
def test_cpp_matches_model_on_config_scripts(name):
    """Tables, context lengths, slots, copy pairs and refcounts of every
    configuration's construction script are bit-identical."""
    w = W.build(name, values=False)
    ref = oracle.run_scenario(w, outputs=False, cache=False)
    bm, appends, decodes = _replay_cpp(w)
    assert [(list(a["slots"]), [tuple(p) for p in a["pairs"]]) for a in ref.appends] == appends
    for d_ref, (tab, ctx) in zip(ref.decodes, decodes):
        assert np.array_equal(d_ref.tables, tab) and np.array_equal(d_ref.ctx, ctx)
    assert [bm.refcount(b) for b in range(ref.bm.N)] == ref.bm.rc
    assert bm.free_list().tolist() == list(reversed(ref.bm.free))


def test_check_tables():
    tab = np.array([[3, 1, -1], [0, -1, -1]], np.int32)
    pa.pa_check_tables(tab, np.array([20, 16]), 16, 4)
    with pytest.raises(pa.PAError, match="out of"):
        pa.pa_check_tables(tab, np.array([40, 16]), 16, 4)
    with pytest.raises(pa.PAError, match="stride"):
        pa.pa_check_tables(tab, np.array([49, 1]), 16, 4)
    with pytest.raises(pa.PAError, match="out of"):
        pa.pa_check_tables(tab, np.array([1, 1]), 16, 2)      # block 3 outside a 2-block pool


# --------------------------------------------- validation before any launch
def _decode_args(**over):
    a = dict(out=16, out_dtype=pa.PA_F32, q=16, k=16, v=16, kv_dtype=pa.PA_BF16, tables=16, stride=256,
             ctx=16, max_ctx=4096, B=64, Hq=32, Hkv=8, D=128, BS=16, N=1000, scale=0.1, part=0, ws=0,
             ws_bytes=0, stream=0, kernel=0)
    a.update(over)
    return [a[k] for k in ["out", "out_dtype", "q", "k", "v", "kv_dtype", "tables", "stride", "ctx", "max_ctx",
                           "B", "Hq", "Hkv", "D", "BS", "N", "scale", "part", "ws", "ws_bytes", "stream",
                           "kernel"]]


@pytest.mark.parametrize("over,status", [
    (dict(D=96), 4), (dict(BS=64), 4), (dict(Hq=12, Hkv=8), 1), (dict(Hq=24, Hkv=8), 4),
    (dict(out_dtype=pa.PA_F16), 1), (dict(stride=10), 1), (dict(part=100), 1), (dict(part=64, BS=32), 1),
    (dict(q=8), 1), (dict(kv_dtype=7), 1), (dict(kernel=pa.PA_KERNEL_MFMA, kv_dtype=pa.PA_F32), 4),
    (dict(N=0), 1), (dict(N=1 << 28, BS=16), 1), (dict(q=0), 1),
    (dict(ws=0, ws_bytes=0, part=512), 1),          # 4096 tokens need 8 partitions: workspace required
])
def test_decode_rejects_bad_arguments(over, status):
    assert pa.lib.pa_decode_variant(*_decode_args(**over)) == status
    assert pa.lib.pa_last_error()


def test_write_and_copy_reject_bad_arguments():
    lib = pa.lib
    assert lib.pa_write_kv(16, 16, 16, 16, 16, -1, 8, 128, 16, 100, 2, 0) == 1
    assert lib.pa_write_kv(16, 16, 16, 16, 16, 1, 8, 96, 16, 100, 2, 0) == 4
    assert lib.pa_write_kv(0, 16, 16, 16, 16, 1, 8, 128, 16, 100, 2, 0) == 1
    assert lib.pa_write_kv(16, 16, 16, 16, 16, 0, 8, 128, 16, 100, 2, 0) == 0     # no-op, no launch
    assert lib.pa_copy_blocks(16, 16, 16, -2, 8, 128, 16, 100, 2, 0) == 1
    assert lib.pa_copy_blocks(16, 16, 16, 0, 8, 128, 16, 100, 2, 0) == 0


def test_workspace_bytes():
    def r(x):
        return -(-x // 256) * 256
    # stream kernel: two partial records per worker; 256 compute units x one
    # 144 KiB workgroup of 4 waves
    workers = 256 * 4
    stream = r(workers * 2 * 4 * 2 * 4) + r(workers * 2 * 4 * 128 * 4)
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 512, 512) == stream
    # partition kernels: m, l and acc sections per (sequence, q head, partition)
    rows = 64 * 32 * 8
    part = 2 * r(rows * 4) + r(rows * 128 * 4)
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 4096, 512) == max(stream, part)
    # auto partition sizes never need more than the 256-token bound
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 4096, 0) >= max(stream, part)
    assert pa.pa_decode_workspace_bytes(64, 32, 7, 128, 4096, 0) == 0   # heads not a multiple


def test_rebalance_feedback():
    """Host feedback of the stream kernel's workgroup shares: equal finish
    times keep equal weights; the workgroups of a die class (index modulo 8)
    that finish late lose share together and early ones gain; single slow
    workgroups only move their class; counter wrap-around between stamps is
    harmless; the result stays within its bounds."""
    from paged_kv_cache_332_amd.engine import rebalance
    g = 32
    w = np.full(g, 1024, dtype=np.int32)

    def stamps(finish, base=1000):
        t = np.zeros((g, 4, 2), dtype=np.int64)
        t[:, :, 0] = base
        t[:, :, 1] = base + np.asarray(finish)[:, None]
        return ((t + (1 << 31)) % (1 << 32) - (1 << 31)).astype(np.int32).ravel()

    assert (rebalance(w, stamps(np.full(g, 500))) == 1024).all()
    fin = np.full(g, 500)
    fin[3::8] = 1000          # class 3 slow
    fin[7::8] = 250           # class 7 fast
    r = rebalance(w, stamps(fin))
    assert (r[3::8] == r[3]).all() and (r[7::8] == r[7]).all()
    assert r[3] < r[0] < r[7] and abs(r.mean() - 1024) < 2
    # the same finish times across the 32-bit wrap of the counter
    assert (rebalance(w, stamps(fin, base=(1 << 32) - 300)) == r).all()
    # one slow workgroup moves only its class, by a quarter of the effect
    fin = np.full(g, 500)
    fin[5] = 900
    r = rebalance(w, stamps(fin))
    assert (r[5::8] == r[5]).all() and r[5] < r[0] and (r[np.arange(g) % 8 != 5] == r[0]).all()
    # bounds
    fin = np.full(g, 10)
    fin[0::8] = 10 ** 7
    r = rebalance(w, stamps(fin), rate=1.0)
    assert r.min() >= 64 and r.max() <= 16384 and r[0] == 64
    # several steps: the class finish times are averaged before one update,
    # so a die that was slow in one step and fast in the next keeps its share
    from paged_kv_cache_332_amd.engine import class_finish, rebalance_classes
    slow, fast = np.full(g, 500), np.full(g, 500)
    slow[2::8], fast[2::8] = 700, 300
    mean = (class_finish(stamps(slow), g) + class_finish(stamps(fast), g)) / 2
    assert np.allclose(mean, 500) and (rebalance_classes(w, mean) == 1024).all()
    assert (rebalance_classes(w, class_finish(stamps(slow), g)) == rebalance(w, stamps(slow))).all()


@settings(max_examples=60, deadline=None)
@given(ctx=st.lists(st.integers(0, 700), min_size=1, max_size=12), hkv=st.sampled_from([1, 2, 8]),
       grid=st.integers(1, 12), weighted=st.booleans(), seed=st.integers(0, 2 ** 16))
def test_stream_plan_matches_brute_force(ctx, hkv, grid, weighted, seed):
    """The host's split of the (sequence, kv head, 16-token tile) list over
    the stream kernel's waves: workgroup shares follow the weights, every
    tile has exactly one wave, and the cut items and their waves agree with
    the owner of every tile found by brute force."""
    import paged_kv_cache_332_amd as pa
    tiles = [(c + 15) // 16 for c in ctx]
    pre = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    wts = rng.integers(-3, 70000, size=grid).astype(np.int32) if weighted else None
    starts, entries, wave_list = pa.pa_stream_plan(pre, hkv, grid, wts)
    total = hkv * int(pre[-1])
    nw = 4 * grid
    # shares: workgroup b holds [T P_b / P, T P_(b+1) / P), quartered
    wc = np.ones(grid, dtype=np.int64) if wts is None else np.clip(wts.astype(np.int64), 1, 1 << 16)
    P = np.concatenate([[0], np.cumsum(wc)])
    for b in range(grid):
        a0, a1 = total * P[b] // P[-1], total * P[b + 1] // P[-1]
        assert [int(x) for x in starts[4 * b: 4 * b + 4]] == [a0 + (a1 - a0) * k // 4 for k in range(4)]
    assert starts[nw] == total and (np.diff(starts) >= 0).all()
    owner = np.searchsorted(starts[:nw], np.arange(total), side="right") - 1
    expect = []
    for s, nt in enumerate(tiles):
        for h in range(hkv):
            if nt == 0:
                continue
            gs = hkv * int(pre[s]) + h * nt
            own = sorted(set(owner[gs: gs + nt].tolist()))
            if len(own) > 1:
                expect.append((2 * (s * hkv + h) + int(starts[own[0]] < gs), own))
    assert len(entries) == len(expect)
    off = 0
    for k, (code, own) in enumerate(expect):
        code_k, cnt, off_k = (int(x) for x in entries[k, :3])
        assert (code_k, cnt, off_k) == (code, len(own), off)
        assert wave_list[off: off + cnt].tolist() == own
        inline = (own + [0, 0, 0])[:4]
        assert entries[k, 3:7].tolist() == inline and entries[k, 7] == 0
        off += cnt
    assert off == len(wave_list)


def test_stream_plan_rejects_bad_input():
    import paged_kv_cache_332_amd as pa
    with pytest.raises(pa.PAError):
        pa.pa_stream_plan(np.array([0, 5, 3], dtype=np.int32), 2, 4)      # decreasing prefix
    with pytest.raises(pa.PAError):
        pa.pa_stream_plan(np.array([0, 5], dtype=np.int32), 2, 2000)      # grid beyond the limit


def _prefill_args(**over):
    a = dict(out=16, out_dtype=pa.PA_F32, q=16, k=16, v=16, kv_dtype=pa.PA_BF16, tables=16, stride=256,
             qs=16, ctx=16, max_q=512, max_ctx=4096, B=64, Hq=32, Hkv=8, D=128, BS=16, N=1000, scale=0.1,
             ws=None, ws_bytes=0, stream=0)
    a.update(over)
    return [a[k] for k in ["out", "out_dtype", "q", "k", "v", "kv_dtype", "tables", "stride", "qs", "ctx",
                           "max_q", "max_ctx", "B", "Hq", "Hkv", "D", "BS", "N", "scale", "ws", "ws_bytes", "stream"]]


@pytest.mark.parametrize("over,status", [
    (dict(kv_dtype=pa.PA_F32), 4), (dict(D=96), 4), (dict(Hq=24, Hkv=8), 4), (dict(Hq=12, Hkv=8), 1),
    (dict(out_dtype=pa.PA_F16), 1), (dict(max_q=5000), 1), (dict(stride=10), 1), (dict(q=8), 1),
    (dict(qs=0), 1), (dict(B=10000), 4),
    (dict(max_q=16, B=8, ws=16, ws_bytes=100), 1),      # short chunks of 8 sequences split: workspace too small
    (dict(max_q=16, B=8, ws=8, ws_bytes=1 << 30), 1),   # workspace not 16-byte aligned
])
def test_prefill_rejects_bad_arguments(over, status):
    """Host validation of pa_prefill, before any launch."""
    assert pa.lib.pa_prefill(*_prefill_args(**over)) == status
    assert pa.lib.pa_last_error()


def test_prefill_workspace_bytes():
    """The context split is asked for only where few workgroups would run
    (fewer than two per compute unit; one per sequence, kv head and query
    block), and holds at least two pieces' partial states for every query row
    it covers."""
    Hq, Hkv, D = 32, 8, 128
    assert pa.pa_prefill_workspace_bytes(512, 4160, 64, Hq, Hkv, D) == 0      # 5632 workgroups
    assert pa.pa_prefill_workspace_bytes(16, 4160, 64, Hq, Hkv, D) == 0       # 512 workgroups
    short = pa.pa_prefill_workspace_bytes(16, 131072, 8, Hq, Hkv, D)         # 64 workgroups
    assert short >= 2 * 8 * 16 * Hq * (D + 2) * 4
    # a longer bound never needs less; a context of one piece has nothing to split
    assert pa.pa_prefill_workspace_bytes(16, 262144, 8, Hq, Hkv, D) >= short
    assert pa.pa_prefill_workspace_bytes(16, 512, 8, Hq, Hkv, D) == 0
    # shapes pa_prefill rejects need none
    assert pa.pa_prefill_workspace_bytes(16, 131072, 8, 24, Hkv, D) == 0
    assert pa.pa_prefill_workspace_bytes(0, 131072, 8, Hq, Hkv, D) == 0


@pytest.mark.parametrize("hq,hkv,maxq,b,want", [
    (32, 8, 512, 64, 3),      # 5632 workgroups; the last of 11 blocks of 48 tokens holds 32: 16 of 528 rows empty
    (32, 8, 128, 64, 3),      # 1536 workgroups, 16 of 144 rows empty
    (32, 8, 64, 64, 2),       # a third of the last three-block rows empty
    (32, 8, 16, 64, 1),       # 512 workgroups at two blocks
    (64, 8, 512, 8, 3),       # group 8: 24-token blocks, 1408 workgroups
    (64, 8, 128, 8, 2),       # 384 workgroups at three blocks, 512 at two
    (32, 8, 32, 64, 2),       # 512 workgroups at two blocks, none empty
    (32, 8, 48, 64, 1),       # a quarter of the last two-block rows empty
    (32, 8, 512, 8, 2),       # 704 at three blocks, 1024 at two
    (24, 8, 512, 64, 0),      # group 3: rejected
])
def test_prefill_column_blocks(hq, hkv, maxq, b, want):
    """The prefill's workgroup size per launch shape (the benchmark counts
    streamed bytes with it)."""
    assert pa.pa_prefill_column_blocks(hq, hkv, maxq, b) == want


def _swap_args(**over):
    a = dict(k=16, v=16, hk=16, hv=16, blocks=16, n=4, to_host=1, Hkv=8, D=128, BS=16, N=1000, dtype=pa.PA_BF16,
             stream=0)
    a.update(over)
    return [a[k] for k in ["k", "v", "hk", "hv", "blocks", "n", "to_host", "Hkv", "D", "BS", "N", "dtype", "stream"]]


@pytest.mark.parametrize("over,status", [
    (dict(to_host=2), 1), (dict(n=-1), 1), (dict(D=96), 4), (dict(BS=12), 4), (dict(N=0), 1), (dict(dtype=7), 1),
    (dict(hk=0), 1), (dict(hv=8), 1),
    (dict(), 1),              # pointers the device cannot address (no device here)
    (dict(n=0, hk=0), 0),     # nothing to move
])
def test_swap_blocks_rejects_bad_arguments(over, status):
    """Host validation of pa_swap_blocks, before any launch."""
    assert pa.lib.pa_swap_blocks(*_swap_args(**over)) == status
    if status:
        assert pa.lib.pa_last_error()


def test_shared_blocks_follow_forks_copies_and_frees():
    """Hand-traced sharing changes (block size 4, a 10-token prompt in blocks
    0..2, the last one partly filled): the leading shared blocks of every
    table after forks, a copy-on-write by one of three sharers (the partly
    filled block stays shared by the other two), the last sharer's in-place
    write, and frees that leave a single holder."""
    bm = pa.BlockManager(16, 4)
    bm.add_seq(0, 10)
    assert bm.shared_blocks(0) == 0
    bm.fork(0, 1)
    bm.fork(0, 2)
    assert [bm.shared_blocks(s) for s in (0, 1, 2)] == [3, 3, 3]
    _, pairs = bm.append_slots([1])           # copies block 2; two sharers remain
    assert len(pairs) == 1
    assert [bm.shared_blocks(s) for s in (0, 1, 2)] == [3, 2, 3]
    _, pairs = bm.append_slots([0])           # copies again; sequence 2 now holds block 2 alone
    assert len(pairs) == 1
    assert [bm.shared_blocks(s) for s in (0, 1, 2)] == [2, 2, 2]
    _, pairs = bm.append_slots([2])           # the last holder writes in place
    assert len(pairs) == 0
    assert [bm.shared_blocks(s) for s in (0, 1, 2)] == [2, 2, 2]
    bm.free_seq(1)
    assert [bm.shared_blocks(s) for s in (0, 2)] == [2, 2]
    bm.free_seq(2)
    assert bm.shared_blocks(0) == 0
    assert bm.shared_blocks(2) == -1


def _aligned(nbytes, align=256):
    """A host buffer whose address is a multiple of `align` (stands in for a
    device pointer: the call below is rejected before anything reads it)."""
    raw = np.zeros(nbytes + align, np.uint8)
    off = (-raw.ctypes.data) % align
    return raw, raw.ctypes.data + off


@pytest.mark.parametrize("bad", ["null k_new", "misaligned v_new"])
def test_rejected_step_leaves_the_manager_unchanged(bad):
    """pa_step validates every argument before the manager appends: a
    rejected call (here the new tokens' rows) returns INVALID and leaves
    lengths, tables, refcounts and counters exactly as they were."""
    bs, hkv, hq, d, stride = 16, 2, 8, 64, 8
    bm = pa.BlockManager(40, bs)
    for s, n in enumerate([16, 5, 33]):
        bm.add_seq(s, n)
    bm.fork(0, 3)
    seqs = np.array([0, 1, 2, 3], np.int64)
    before = (bm.stats(), bm.export(list(seqs), stride), [bm.refcount(b) for b in range(40)])
    words = pa.step_record_words(len(seqs), stride, hkv)
    stage_h = np.zeros(words, np.int32)
    keep = []
    ptrs = {}
    for name, nbytes in (("stage_dev", 4 * words), ("k", 40 * hkv * d * bs * 2), ("v", 40 * hkv * d * bs * 2),
                         ("q", 4 * hq * d * 2), ("out", 4 * hq * d * 4), ("kn", 4 * hkv * d * 2),
                         ("vn", 4 * hkv * d * 2), ("ws", 1 << 24)):
        raw, p = _aligned(nbytes)
        keep.append(raw)
        ptrs[name] = p
    kn, vn = (None, ptrs["vn"]) if bad == "null k_new" else (ptrs["kn"], ptrs["vn"] + 2)
    st = pa.lib.pa_step(bm._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(seqs),
                        stage_h.ctypes.data, ptrs["stage_dev"], words, stride, ptrs["k"], ptrs["v"], kn, vn,
                        ptrs["q"], ptrs["out"], 0, 2, hq, hkv, d, bs, 40, 0.125, 0, ptrs["ws"], 1 << 24, 0, None,
                        None, None, None, None, 0, None)
    assert st == 1, pa.lib.pa_last_error()
    assert "k_new" in pa.lib.pa_last_error().decode()
    after = (bm.stats(), bm.export(list(seqs), stride), [bm.refcount(b) for b in range(40)])
    assert after[0] == before[0] and after[2] == before[2]
    assert np.array_equal(after[1][0], before[1][0]) and np.array_equal(after[1][1], before[1][1])


@settings(max_examples=30, deadline=None)
@given(st.integers(1, 300), st.sampled_from([1, 3, 8]), st.integers(0, 2 ** 32 - 1), st.integers(0, 2 ** 31 - 1))
def test_native_class_finish_matches_numpy(grid, classes, base, seed):
    """pa_stream_class_finish (the engine's per-step load-balance feedback)
    equals the engine's numpy definition, also when the 32-bit counter wraps
    inside the pass."""
    from paged_kv_cache_332_amd.engine import class_finish
    rng = np.random.default_rng(seed)
    start = base + rng.integers(0, 50, size=4 * grid)
    end = start + rng.integers(0, 10000, size=4 * grid)
    stamps = np.empty(8 * grid, np.int64)
    stamps[0::2], stamps[1::2] = start, end
    stamps32 = ((stamps + (1 << 31)) % (1 << 32) - (1 << 31)).astype(np.int32)
    out = np.zeros(classes)
    pa.stream_class_finish(stamps32.ctypes.data, grid, classes, out)
    np.testing.assert_allclose(out, class_finish(stamps32, grid, classes), rtol=0, atol=1e-9)
