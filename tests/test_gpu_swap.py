"""Preemption by swap on an MI355X: pa_bm_swap_out / pa_swap_blocks copy a
sequence's blocks to pinned host memory, other work reuses and overwrites the
blocks, pa_bm_swap_in / pa_swap_blocks bring them back into fresh blocks.
Each step is mirrored on the oracle's block-manager and cache models: block
ids, host copies and pool bytes must be bit-exact with the models, and decode
over the restored sequence within tolerance of the float64 oracle (and, as
the decode plan depends on context lengths only, bit-identical to the decode
before the swap)."""
import sys

import numpy as np
import pytest
import torch

import oracle
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


TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def _pool_np(t):
    """Raw bits of a device pool as the oracle's cache model stores them."""
    b = _bits(t).cpu().numpy()
    return b.view(np.uint32) if t.element_size() == 4 else b.view(np.uint16)


def _oracle_side(w):
    """The oracle's block-manager and cache models after the workload's
    construction (no attention yet)."""
    ref = oracle.run_scenario(w, outputs=False)
    return ref.bm, ref.cache


def _check_against_oracle(eng, bm_model, cm, q, seqs, out, dtype, scale, label):
    """Pools bit for bit against the cache model, and decode rows against
    float64 attention over K/V the model gathers through its own tables."""
    assert np.array_equal(_pool_np(eng.k_cache), cm.k), f"{label}: K pool bits differ from the oracle"
    assert np.array_equal(_pool_np(eng.v_cache), cm.v), f"{label}: V pool bits differ from the oracle"
    got = out.double().cpu().numpy()
    errs = []
    for j, s in enumerate(seqs):
        K, V = cm.gather(bm_model.table(s), bm_model.length(s))
        want = oracle.decode_attention(q[j], K, V, scale)
        err = float(np.max(np.abs(got[j] - want)))
        errs.append(err)
        assert err <= TOL[dtype] and err <= 1e-4 * float(np.max(np.abs(want))) + 1e-8, (label, s, err)
    return max(errs)


@pytest.mark.parametrize("dtype,bs,list_on_device", [("bf16", 16, False), ("f16", 32, True), ("f32", 8, False)])
def test_swap_round_trip(dtype, bs, list_on_device):
    """Swap a sequence out (its blocks released, their bytes copied to
    pinned host memory), let a new sequence take and overwrite the blocks,
    swap it back into fresh blocks.  Every step is mirrored on the oracle's
    block-manager and cache models ("Paged Attention: Virtual Memory for the
    KV Cache", §What it does not fix): block ids, the host copies and both
    pools are bit-exact with the models; decode over the restored sequence
    is within tolerance of the oracle and bit-identical to the decode before
    the swap."""
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
    bm_model, cm = _oracle_side(w)
    tdt = runner.TORCH_DTYPE[dtype]
    seqs = list(range(len(ctx)))
    rng = np.random.default_rng(9)
    q = W.round_to_dtype(rng.standard_normal((len(ctx), hq, d), dtype=np.float32), dtype)
    q_dev = torch.from_numpy(q).to("cuda").to(tdt)
    before = _decode(pa, eng, q_dev, seqs, hq, d)
    _check_against_oracle(eng, bm_model, cm, q, seqs, before, dtype, w.cfg.scale, "before")

    victim = 0
    old = eng.bm.swap_out(victim)
    assert list(old) == bm_model.swap_out(victim)
    assert eng.bm.swapped_len(victim) == bm_model.swapped_len(victim) == ctx[victim]
    host_k = torch.full((len(old), cm.k[0].size), 7, dtype=tdt).pin_memory()
    host_v = torch.full((len(old), cm.v[0].size), 7, dtype=tdt).pin_memory()
    host_model_k, host_model_v = cm.k[list(old)].reshape(len(old), -1).copy(), cm.v[list(old)].reshape(len(old), -1).copy()

    def ids(blocks):
        t = torch.from_numpy(np.asarray(blocks, np.int32))
        return t.to("cuda") if list_on_device else t.pin_memory()

    pa.pa_swap_blocks(eng.k_cache, eng.v_cache, host_k, host_v, ids(old), to_host=True)
    # the blocks are reused at once: a new sequence takes them and its rows
    # are written over them, on the device and in the model alike
    n99 = len(old) * bs
    taken = eng.bm.add_seq(99, n99)
    assert list(taken) == bm_model.add_seq(99, n99)
    assert {int(s) // bs for s in taken} == set(int(b) for b in old)
    k99 = W.round_to_dtype(rng.standard_normal((n99, hkv, d), dtype=np.float32), dtype)
    v99 = W.round_to_dtype(rng.standard_normal((n99, hkv, d), dtype=np.float32), dtype)
    pa.pa_write_kv(eng.k_cache, eng.v_cache, torch.from_numpy(k99).to("cuda").to(tdt),
                   torch.from_numpy(v99).to("cuda").to(tdt),
                   torch.from_numpy(np.ascontiguousarray(taken, dtype=np.int32)).to("cuda"))
    cm.write(taken, k99, v99)
    torch.cuda.synchronize()
    hb = lambda t: _bits(t).numpy().view(np.uint32 if t.element_size() == 4 else np.uint16)
    assert np.array_equal(hb(host_k), host_model_k) and np.array_equal(hb(host_v), host_model_v)

    # bring it back while the other sequence still holds the old blocks
    new = eng.bm.swap_in(victim)
    assert list(new) == bm_model.swap_in(victim)
    assert not set(int(b) for b in new) & set(int(b) for b in old)
    pa.pa_swap_blocks(eng.k_cache, eng.v_cache, host_k, host_v, ids(new), to_host=False)
    cm.k[list(new)] = host_model_k.reshape(cm.k[list(new)].shape)
    cm.v[list(new)] = host_model_v.reshape(cm.v[list(new)].shape)
    torch.cuda.synchronize()
    after = _decode(pa, eng, q_dev, seqs, hq, d)
    err = _check_against_oracle(eng, bm_model, cm, q, seqs, after, dtype, w.cfg.scale, "after swap-in")
    say("swap round trip", dtype, "max abs error after swap-in", err)
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
    again).  Mirrored on the oracle's models: slots and both pools bit-exact,
    decode within tolerance of the oracle and bit-identical to the decode
    before the eviction."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    from oracle import accounting
    ctx = [300, 17, 129]
    hq, hkv, d, bs = 16, 4, 128, 16
    need = sum(-(-(c + 1) // bs) for c in ctx)
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=11, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs, num_blocks=2 * need + 8)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    bm_model, cm = _oracle_side(w)
    seqs = list(range(len(ctx)))
    rng = np.random.default_rng(12)
    q = W.round_to_dtype(rng.standard_normal((len(ctx), hq, d), dtype=np.float32), "bf16")
    q_dev = torch.from_numpy(q).to("cuda").to(torch.bfloat16)
    before = _decode(pa, eng, q_dev, seqs, hq, d)
    _check_against_oracle(eng, bm_model, cm, q, seqs, before, "bf16", w.cfg.scale, "before")
    victim = 0
    eng.bm.free_seq(victim)
    bm_model.free_seq(victim)
    # the released blocks are reused at once and overwritten
    n99 = -(-ctx[victim] // bs) * bs
    taken = eng.bm.add_seq(99, n99)
    assert list(taken) == bm_model.add_seq(99, n99)
    k99 = W.round_to_dtype(rng.standard_normal((n99, hkv, d), dtype=np.float32), "bf16")
    v99 = W.round_to_dtype(rng.standard_normal((n99, hkv, d), dtype=np.float32), "bf16")
    pa.pa_write_kv(eng.k_cache, eng.v_cache, torch.from_numpy(k99).to("cuda").to(torch.bfloat16),
                   torch.from_numpy(v99).to("cuda").to(torch.bfloat16),
                   torch.from_numpy(np.ascontiguousarray(taken, dtype=np.int32)).to("cuda"))
    cm.write(taken, k99, v99)
    # re-admission with headroom, then the recomputed rows go back through the slots
    assert accounting.admit(bm_model.num_free(), ctx[victim], bs, 1)
    slots = eng.bm.admit(victim, ctx[victim], reserve_blocks=1)
    assert list(slots) == bm_model.add_seq(victim, ctx[victim])
    rows = w.row_of(victim, np.arange(ctx[victim]))
    k = torch.from_numpy(w.k_rows[rows].astype(np.float32)).to("cuda").to(torch.bfloat16)
    v = torch.from_numpy(w.v_rows[rows].astype(np.float32)).to("cuda").to(torch.bfloat16)
    pa.pa_write_kv(eng.k_cache, eng.v_cache, k, v, torch.from_numpy(np.ascontiguousarray(slots)).to("cuda"))
    cm.write(slots, w.k_rows[rows], w.v_rows[rows])
    torch.cuda.synchronize()
    after = _decode(pa, eng, q_dev, seqs, hq, d)
    err = _check_against_oracle(eng, bm_model, cm, q, seqs, after, "bf16", w.cfg.scale, "after re-admission")
    say("recompute: max abs error after re-admission", err)
    assert _same(after, before)
    eng.bm.free_seq(99)
