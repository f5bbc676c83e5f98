"""Preemption by swap on an MI355X: pa_bm_swap_out / pa_swap_blocks copy a
sequence's blocks to pinned host memory, other work reuses and overwrites the
blocks, pa_bm_swap_in / pa_swap_blocks bring them back into fresh blocks.  The
restored pool bytes must equal the originals bit for bit, and decode over the
restored sequence must give the same output as before the swap, bit for bit
(the decode plan depends on context lengths only, not on block ids)."""
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def _bits(t):
    """Raw bits (the pool's unwritten slots hold NaN poison, so compare bits)."""
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def _same(a, b):
    return torch.equal(_bits(a.to(b.device)), _bits(b))


def _blocks_of(pool, ids):
    return pool[torch.as_tensor(ids, dtype=torch.long, device=pool.device)].reshape(len(ids), -1)


def _decode(pa, eng, q_dev, seqs, hq, d):
    out = eng.decode(seqs, q_dev).clone()
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype,bs,list_on_device", [("bf16", 16, False), ("f16", 32, True), ("f32", 8, False)])
def test_swap_round_trip(dtype, bs, list_on_device):
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    ctx = [300, 17, 1, 129]
    hq, hkv, d = 16, 4, 128
    say("swap round trip", dtype, bs, "device list" if list_on_device else "pinned list")
    # room for the victim's blocks twice over (held by the new sequence and swapped back in)
    need = sum(-(-(c + 1) // bs) for c in ctx)
    w = W.tiny(num_seqs=len(ctx), dtype=dtype, seed=7, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs, num_blocks=2 * need + 8)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    seqs = list(range(len(ctx)))
    rng = np.random.default_rng(9)
    q = W.round_to_dtype(rng.standard_normal((len(ctx), hq, d), dtype=np.float32), dtype)
    q_dev = torch.from_numpy(q).to("cuda").to(runner.TORCH_DTYPE[dtype])
    before = _decode(pa, eng, q_dev, seqs, hq, d)
    torch.cuda.synchronize()

    victim = 0
    old = eng.bm.swap_out(victim)
    assert len(old) == -(-ctx[victim] // bs) and eng.bm.swapped_len(victim) == ctx[victim]
    k_ref, v_ref = _blocks_of(eng.k_cache, old).clone(), _blocks_of(eng.v_cache, old).clone()
    tdt = eng.k_cache.dtype
    host_k = torch.full(k_ref.shape, 7, dtype=tdt).pin_memory()
    host_v = torch.full(v_ref.shape, 7, dtype=tdt).pin_memory()

    def ids(blocks):
        t = torch.from_numpy(np.asarray(blocks, np.int32))
        return t.to("cuda") if list_on_device else t.pin_memory()

    out_ids = ids(old)
    pa.pa_swap_blocks(eng.k_cache, eng.v_cache, host_k, host_v, out_ids, to_host=True)
    # the blocks are reused at once: a new sequence takes them and the pool is overwritten
    taken = eng.bm.add_seq(99, len(old) * bs)
    reused = sorted({int(s) // bs for s in taken})
    assert set(reused) == set(int(b) for b in old)
    idx = torch.as_tensor(reused, dtype=torch.long, device="cuda")
    eng.k_cache[idx] = torch.randn(eng.k_cache[idx].shape, device="cuda").to(tdt)
    eng.v_cache[idx] = torch.randn(eng.v_cache[idx].shape, device="cuda").to(tdt)
    torch.cuda.synchronize()
    assert _same(host_k, k_ref) and _same(host_v, v_ref)

    # bring it back while the other sequence still holds the old blocks
    new = eng.bm.swap_in(victim)
    assert not set(int(b) for b in new) & set(reused)
    in_ids = ids(new)
    pa.pa_swap_blocks(eng.k_cache, eng.v_cache, host_k, host_v, in_ids, to_host=False)
    torch.cuda.synchronize()
    assert _same(_blocks_of(eng.k_cache, new), k_ref)
    assert _same(_blocks_of(eng.v_cache, new), v_ref)
    after = _decode(pa, eng, q_dev, seqs, hq, d)
    torch.cuda.synchronize()
    assert _same(after, before)
    eng.bm.free_seq(99)


def test_swap_skips_ids_outside_the_pool():
    """An id outside [0, num_blocks) moves nothing; the others move."""
    import paged_kv_cache_332_amd as pa
    k = torch.randn((6, 2, 8, 16, 8), device="cuda").to(torch.bfloat16)
    v = torch.randn((6, 2, 64, 16), device="cuda").to(torch.bfloat16)
    host_k = torch.zeros((3, 2 * 64 * 16), dtype=torch.bfloat16).pin_memory()
    host_v = torch.zeros((3, 2 * 64 * 16), dtype=torch.bfloat16).pin_memory()
    ids = torch.tensor([4, 6, -1], dtype=torch.int32).pin_memory()
    pa.pa_swap_blocks(k, v, host_k, host_v, ids, to_host=True)
    torch.cuda.synchronize()
    assert torch.equal(host_k[0].to("cuda"), k[4].reshape(-1)) and torch.equal(host_v[0].to("cuda"), v[4].reshape(-1))
    assert not host_k[1:].any() and not host_v[1:].any()
    k0 = k.clone()
    ids_in = torch.tensor([7, 2, 1], dtype=torch.int32).pin_memory()
    pa.pa_swap_blocks(k, v, host_k, host_v, ids_in, to_host=False)
    torch.cuda.synchronize()
    assert not k[2].any() and not k[1].any()
    assert torch.equal(k[0], k0[0]) and torch.equal(k[3:], k0[3:])


def test_swap_rejects_pageable_host_memory():
    import paged_kv_cache_332_amd as pa
    k = torch.zeros((4, 2, 8, 16, 8), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((4, 2, 64, 16), dtype=torch.bfloat16, device="cuda")
    host = torch.zeros((1, 2 * 64 * 16), dtype=torch.bfloat16)            # pageable
    ids = torch.tensor([1], dtype=torch.int32).pin_memory()
    with pytest.raises(pa.PAError):
        pa.pa_swap_blocks(k, v, host, host.pin_memory(), ids, to_host=True)


def test_preempt_by_recompute():
    """The other way back from preemption: the sequence is released
    (pa_bm_free_seq), its blocks are reused and overwritten, and it is
    re-admitted later (pa_bm_admit) with its K/V rows written again through
    the new slots (the rows a model recomputes when it prefills the prompt
    again): decode over it gives the same bits as before the eviction."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    ctx = [300, 17, 129]
    hq, hkv, d, bs = 16, 4, 128, 16
    need = sum(-(-(c + 1) // bs) for c in ctx)
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=11, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs, num_blocks=2 * need + 8)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    seqs = list(range(len(ctx)))
    rng = np.random.default_rng(12)
    q = W.round_to_dtype(rng.standard_normal((len(ctx), hq, d), dtype=np.float32), "bf16")
    q_dev = torch.from_numpy(q).to("cuda").to(torch.bfloat16)
    before = _decode(pa, eng, q_dev, seqs, hq, d)
    victim = 0
    old = [int(b) for b in eng.bm.export([victim], eng.stride)[0][0] if b >= 0]
    eng.bm.free_seq(victim)
    # the released blocks are reused at once and overwritten
    taken = eng.bm.add_seq(99, len(old) * bs)
    idx = torch.as_tensor(sorted({int(s) // bs for s in taken}), dtype=torch.long, device="cuda")
    eng.k_cache[idx] = torch.randn(eng.k_cache[idx].shape, device="cuda").to(torch.bfloat16)
    eng.v_cache[idx] = torch.randn(eng.v_cache[idx].shape, device="cuda").to(torch.bfloat16)
    # re-admission with headroom, then the recomputed rows go back through the slots
    slots = eng.bm.admit(victim, ctx[victim], reserve_blocks=1)
    rows = w.row_of(victim, np.arange(ctx[victim]))
    k = torch.from_numpy(w.k_rows[rows].astype(np.float32)).to("cuda").to(torch.bfloat16)
    v = torch.from_numpy(w.v_rows[rows].astype(np.float32)).to("cuda").to(torch.bfloat16)
    pa.pa_write_kv(eng.k_cache, eng.v_cache, k, v, torch.from_numpy(np.ascontiguousarray(slots)).to("cuda"))
    torch.cuda.synchronize()
    after = _decode(pa, eng, q_dev, seqs, hq, d)
    assert _same(after, before)
    eng.bm.free_seq(99)
