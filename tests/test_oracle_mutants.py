"""Planted mistakes in the oracle must fail at least one pin.

Each mutant is the oracle module's own source with one plausible slip
(a dropped term, a wrong sign or index, a transposed operand, a different
free-list order ...), loaded as a separate module on the CPU.  The pins of
tests/oracle_pins.py run against it and at least one must fail; this shows
the pins would catch that kind of mistake in the real oracle.
"""
import importlib.util
import os
import types

import pytest

import oracle_pins as P

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _mutant(module: str, old: str, new: str, count: int = 1, pre: str = None, post: str = None,
            env: dict = None) -> types.ModuleType:
    with open(os.path.join(ORACLE_DIR, module + ".py")) as f:
        src = f.read()
    assert src.count(old) >= count, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    if pre is not None:
        assert pre in src
        src = src.replace(pre, post)
    mod = types.ModuleType(f"oracle_mutant_{module}")
    mod.__dict__.update(env or {})
    exec(compile(src, f"<mutant {module}>", "exec"), mod.__dict__)
    return mod


def _fails(checks) -> bool:
    for c in checks:
        try:
            c()
        except Exception:
            return True
    return False


ATTN_MUTANTS = [
    ("scale squared", "s[r] = (K[:, h, :] @ q[r]) * scale", "s[r] = (K[:, h, :] @ q[r]) * scale * scale"),
    ("no scale", "s[r] = (K[:, h, :] @ q[r]) * scale", "s[r] = (K[:, h, :] @ q[r])"),
    ("negated score", "s[r] = (K[:, h, :] @ q[r]) * scale", "s[r] = -(K[:, h, :] @ q[r]) * scale"),
    ("interleaved head map in scores", "        h = r // g\n", "        h = r % Hkv\n"),
    ("interleaved head map in values", "out[r] = (p @ V[:, r // g, :]) / p.sum()", "out[r] = (p @ V[:, r % Hkv, :]) / p.sum()"),
    ("no max subtraction", "p = np.exp(s[r] - s[r].max())", "p = np.exp(s[r])"),
    ("no normalisation", "out[r] = (p @ V[:, r // g, :]) / p.sum()", "out[r] = (p @ V[:, r // g, :])"),
    ("drops last token", "    s = _scores(q, K, scale)\n    for r in range(Hq):\n        p = np.exp(s[r] - s[r].max())\n        out[r] = (p @ V[:, r // g, :]) / p.sum()",
     "    s = _scores(q, K, scale)[:, : max(1, n - 1)]\n    for r in range(Hq):\n        p = np.exp(s[r] - s[r].max())\n        out[r] = (p @ V[: max(1, n - 1), r // g, :]) / p.sum()"),
    ("uses K as V", "out[r] = (p @ V[:, r // g, :]) / p.sum()", "out[r] = (p @ K[:, r // g, :]) / p.sum()"),
]


@pytest.mark.parametrize("name,old,new", ATTN_MUTANTS, ids=[m[0] for m in ATTN_MUTANTS])
def test_attention_mutant_is_caught(name, old, new):
    m = _mutant("attention", old, new)
    assert _fails([lambda c=c: c(m.decode_attention) for c in P.ATTN_CHECKS]), name


SPLIT_MUTANTS = [
    ("merge forgets rescale of l", "L = (np.asarray(l) * w).sum(axis=0)", "L = np.asarray(l).sum(axis=0)"),
    ("merge rescale sign", "w = np.exp(m - M[None, :])", "w = np.exp(M[None, :] - m)"),
    ("partition drops a token", "lo, hi = p * part, min(n, (p + 1) * part)", "lo, hi = p * part, min(n, (p + 1) * part - 1)"),
    ("partition max not subtracted", "e = np.exp(sp - m[p, r])", "e = np.exp(sp)"),
    ("partial acc uses K", "acc[p, r] = e @ V[lo:hi, r // g, :]", "acc[p, r] = e @ K[lo:hi, r // g, :]"),
]


@pytest.mark.parametrize("name,old,new", SPLIT_MUTANTS, ids=[m[0] for m in SPLIT_MUTANTS])
def test_split_mutant_is_caught(name, old, new):
    m = _mutant("attention", old, new)
    checks = [lambda: P.check_split_merge(m.split_k, m.lse_merge, m.decode_attention)]
    checks += [lambda c=c: c(lambda q, K, V, s: m.decode_attention_split(q, K, V, s, 16))
               for c in P.ATTN_CHECKS]
    assert _fails(checks), name


BM_MUTANTS = [
    ("FIFO free list", "self.free: List[int] = list(reversed(order))", "self.free: List[int] = list(order)"),
    ("copy even when unshared", "elif self.rc[t[-1]] > 1:", "elif self.rc[t[-1]] > 0:"),
    ("never copy-on-write", "elif self.rc[t[-1]] > 1:", "elif False:"),
    ("free in reverse order", "        for b in table:\n            self.rc[b] -= 1", "        for b in reversed(table):\n            self.rc[b] -= 1"),
    ("slot off by one", "return t[pos // self.BS] * self.BS + pos % self.BS", "return t[pos // self.BS] * self.BS + (pos + 1) % self.BS"),
    ("block on full, not on first write", "            if pos % self.BS == 0:\n                t.append", "            if pos % self.BS == 1:\n                t.append"),
    ("fork forgets refcount", "        for b in self.tables[child]:\n            self.rc[b] += 1", "        pass"),
    ("no all-or-nothing", "        if need > self.num_free():\n            raise OutOfBlocks()\n        self.tables[seq]", "        self.tables[seq]"),
]


@pytest.mark.parametrize("name,old,new", BM_MUTANTS, ids=[m[0] for m in BM_MUTANTS])
def test_block_manager_mutant_is_caught(name, old, new):
    m = _mutant("block_manager", old, new)
    assert _fails([lambda: P.check_bm_golden(m.BlockManagerModel, m.OutOfBlocks)]), name


SWAP_MUTANTS = [
    ("swap_out keeps its blocks", "        self.swapped[seq] = self.lens[seq]\n        self.free_seq(seq)",
     "        self.swapped[seq] = self.lens[seq]\n        del self.tables[seq], self.lens[seq]"),
    ("swapped id reused by add_seq", "if seq in self.tables or seq in self.swapped or n < 0:",
     "if seq in self.tables or n < 0:"),
    ("swap_in loses a token", "        n = self.swapped[seq]\n", "        n = max(self.swapped[seq] - 1, 0)\n"),
    ("swap_in takes blocks in reverse", "        self.tables[seq] = [self._pop() for _ in range(need)]\n        self.lens[seq] = n\n        return list",
     "        self.tables[seq] = [self._pop() for _ in range(need)][::-1]\n        self.lens[seq] = n\n        return list"),
    ("swap_in not all-or-nothing", "            raise OutOfBlocks()\n        del self.swapped[seq]",
     "            need = len(self.free)\n        del self.swapped[seq]"),
]


@pytest.mark.parametrize("name,old,new", SWAP_MUTANTS, ids=[m[0] for m in SWAP_MUTANTS])
def test_swap_mutant_is_caught(name, old, new):
    m = _mutant("block_manager", old, new)
    assert _fails([lambda: P.check_bm_swap(m.BlockManagerModel, m.OutOfBlocks, m.InvalidOp)]), name


PREFIX_MUTANTS = [
    ("key without parent", "key = (parent, tuple(tokens[i * BS:(i + 1) * BS]))", "key = (0, tuple(tokens[i * BS:(i + 1) * BS]))"),
    ("reuses the last token's block", "lookable = (n - 1) // BS if n else 0", "lookable = n // BS"),
    ("evicts the newest first", "b = self.evictable.pop(0)", "b = self.evictable.pop()"),
    ("prefix start evicted first", "self.evictable.extend(reversed(cached))", "self.evictable.extend(cached)"),
    ("evicted key kept", "del self.cache[self.block_key.pop(b)]", "self.block_key.pop(b)"),
    ("revived hits counted as free", "if nb - len(hits) > self.num_free() - revived:", "if nb - len(hits) > self.num_free():"),
    ("hits not counted", "        self.hit_blocks += len(hits)\n", ""),
    ("cached blocks freed", "                if b in self.block_key:", "                if False:"),
]


@pytest.mark.parametrize("name,old,new", PREFIX_MUTANTS, ids=[m[0] for m in PREFIX_MUTANTS])
def test_prefix_cache_mutant_is_caught(name, old, new):
    m = _mutant("block_manager", old, new)
    assert _fails([lambda: P.check_bm_prefix_cache(m.BlockManagerModel, m.OutOfBlocks, m.InvalidOp)]), name


CACHE_MUTANTS = [
    ("V stored token-major", "self.v[blk, :, :, off] = vb", "self.v.reshape(self.N, self.H, self.BS, self.D)[blk, :, off, :] = vb"),
    ("K chunk transposed", "kx = kb.reshape(T, self.H, self.D // self.X, self.X)",
     "kx = kb.reshape(T, self.H, self.X, self.D // self.X).transpose(0, 1, 3, 2)"),
    ("copy skips V", "            self.v[dst] = self.v[src]\n", "            pass\n"),
    ("negative slot not skipped", "keep = slots >= 0", "keep = slots >= -(1 << 60)"),
]


@pytest.mark.parametrize("name,old,new", CACHE_MUTANTS, ids=[m[0] for m in CACHE_MUTANTS])
def test_cache_mutant_is_caught(name, old, new):
    m = _mutant("cache", old, new)
    checks = [lambda: P.check_layout_golden(m.PagedCacheModel),
              lambda: P.check_copy_blocks(m.PagedCacheModel)]
    checks += [lambda d=d: P.check_paged_equals_contiguous(m.PagedCacheModel, d) for d in ("bf16", "f32")]
    assert _fails(checks), name


ACCOUNTING_MUTANTS = [
    ("admit with strict inequality", "return need + reserve_blocks <= free_blocks", "return need + reserve_blocks < free_blocks"),
    ("admit ignores the reserve", "return need + reserve_blocks <= free_blocks", "return need <= free_blocks"),
    ("admit rounds blocks down", "    need = -(-num_tokens // block_size)\n    return", "    need = num_tokens // block_size\n    return"),
    ("slab best fit", "for i, (start, length) in enumerate(self.holes):",
     "for i, (start, length) in sorted(enumerate(self.holes), key=lambda e: e[1][1]):"),
    ("slab needs a longer run", "            if length >= n:\n", "            if length > n:\n"),
    ("slab never merges right", "if i + 1 < len(holes) and holes[i][0] + holes[i][1] == holes[i + 1][0]:", "if False:"),
    ("slab never merges left", "if i > 0 and holes[i - 1][0] + holes[i - 1][1] == holes[i][0]:", "if False:"),
    ("room judged by the longest run", "room = slab.free_slots() >= ask", "room = slab.largest_hole() >= ask"),
    ("longest-context pool reserves the length", "ask = max_len if policy == \"slab_max\" else n", "ask = n"),
    ("paged replay keeps a block back", "ok = admit(bm.num_free(), n, block_size, 0)", "ok = admit(bm.num_free(), n, block_size, 1)"),
    ("refused request counted live", "            refused += 1\n", "            refused += 1\n            live[rid] = n\n"),
]


def _accounting_checks(m):
    return [lambda: P.check_admit_golden(m.admit), lambda: P.check_slab_golden(m.SlabAllocator),
            lambda: P.check_slab_invariants(m.SlabAllocator), lambda: P.check_replay_golden(m.replay_admissions),
            lambda: P.check_replay_invariants(m.replay_admissions)]


def _accounting_mutant(old, new):
    # the module imports the block-manager model relatively; the mutant gets
    # the real one
    import oracle.block_manager as bmm
    return _mutant("accounting", old, new, pre="from .block_manager import BlockManagerModel",
                   post="BlockManagerModel = __bm.BlockManagerModel", env={"__bm": bmm})


@pytest.mark.parametrize("name,old,new", ACCOUNTING_MUTANTS, ids=[m[0] for m in ACCOUNTING_MUTANTS])
def test_accounting_mutant_is_caught(name, old, new):
    m = _accounting_mutant(old, new)
    assert _fails(_accounting_checks(m)), name


def test_unmutated_accounting_passes_every_pin():
    m = _accounting_mutant("from typing import", "from typing import")
    for c in _accounting_checks(m):
        c()


@pytest.mark.parametrize("module", ["attention", "block_manager", "cache"])
def test_unmutated_copy_passes_every_pin(module):
    """The harness itself: the oracle's source loaded the same way, with no
    mistake planted, passes every pin (so a caught mutant is the mistake)."""
    m = _mutant(module, "import numpy as np", "import numpy as np")
    if module == "attention":
        for c in P.ATTN_CHECKS:
            c(m.decode_attention)
        P.check_split_merge(m.split_k, m.lse_merge, m.decode_attention)
    elif module == "block_manager":
        P.check_bm_golden(m.BlockManagerModel, m.OutOfBlocks)
        P.check_bm_swap(m.BlockManagerModel, m.OutOfBlocks, m.InvalidOp)
        P.check_bm_prefix_cache(m.BlockManagerModel, m.OutOfBlocks, m.InvalidOp)
    else:
        P.check_layout_golden(m.PagedCacheModel)
        P.check_copy_blocks(m.PagedCacheModel)
        for d in ("bf16", "f16", "f32"):
            P.check_paged_equals_contiguous(m.PagedCacheModel, d)
