"""HIP path against the CPU oracle on an MI355X.

Integer results (slots, copy pairs, tables, context lengths, the K/V pool
bytes) must be bit-identical; decode outputs (fp32) must be within 2e-3 of the
float64 oracle for 16-bit caches and 1e-5 for fp32 caches.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
# A second bound, relative to the output's scale: max|err| <= REL * max|ref|.
# The kernels keep about 16 significant bits of each softmax weight (a 16-bit
# high part plus its rounded remainder, error <= 2^-17 relative) and sum in
# fp32, so the error tracks the output's own magnitude (measured ratios
# 1e-6 .. 6e-6).  Over long contexts the outputs shrink (about 0.01 at 80k
# tokens with K scaled 0.5) and the absolute bound alone would pass a dropped
# 16-token tile or 512-token partition (output shifts of 1e-4 .. 1.2e-3); the
# relative bound fails those by two orders of magnitude.
REL = 1e-4


def _pa():
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    return pa, runner


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def pool_bits(t: torch.Tensor) -> np.ndarray:
    if t.element_size() == 2:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def check_run(w, dev, ref, tol=None, pools=True, label="", rel=REL):
    """Compare a device replay with the oracle's replay of the same script."""
    tol = TOL[w.cfg.dtype] if tol is None else tol
    assert len(dev.appends) == len(ref.appends)
    for a, b in zip(dev.appends, ref.appends):
        assert list(a["slots"]) == list(b["slots"]), label
        assert a["pairs"] == [tuple(p) for p in b["pairs"]], label
    assert len(dev.decodes) == len(ref.decodes)
    errs = []
    for d, r in zip(dev.decodes, ref.decodes):
        assert np.array_equal(d.tables, r.tables) and np.array_equal(d.ctx, r.ctx), label
        out = d.out.float().cpu().numpy().astype(np.float64)
        rows = r.computed
        assert np.all(np.isfinite(out[rows])), label
        err = float(np.max(np.abs(out[rows] - r.out[rows]))) if rows else 0.0
        scale = float(np.max(np.abs(r.out[rows]))) if rows else 0.0
        errs.append(err)
        assert err <= tol, f"{label}: max abs error {err:.3e} > {tol}"
        assert err <= rel * scale + 1e-8, f"{label}: max abs error {err:.3e} > {rel} x max|ref| {scale:.3e}"
    if pools:
        kb, vb = ref.cache.pool_bits()
        assert np.array_equal(pool_bits(dev.engine.k_cache), kb), f"{label}: K pool bytes differ"
        assert np.array_equal(pool_bits(dev.engine.v_cache), vb), f"{label}: V pool bytes differ"
    return errs


def _kernels():
    import paged_kv_cache_332_amd as pa
    return {"valu": pa.PA_KERNEL_VALU, "mfma": pa.PA_KERNEL_MFMA, "stream": pa.PA_KERNEL_STREAM,
            "auto": pa.PA_KERNEL_AUTO}


class _Lazy(dict):
    def __missing__(self, k):
        self.update(_kernels())
        return dict.__getitem__(self, k)


KERNELS = _Lazy()


# ------------------------------------------------------------ small cases
SMALL = []
for dtype in ("f32", "f16", "bf16"):
    for d in (64, 128):
        for bs in (8, 16, 32):
            for g in (1, 4, 8):
                kernels = ["valu"] + (["mfma"] if dtype != "f32" and g > 1 else []) + \
                    (["stream"] if dtype != "f32" else [])
                for kern in kernels:
                    SMALL.append((dtype, d, bs, g, kern))


@pytest.mark.parametrize("dtype,d,bs,g,kern", SMALL, ids=lambda *a: None)
def test_small_shapes(dtype, d, bs, g, kern):
    """Ragged contexts (one token, a block minus one, exact blocks, several
    partitions with a ragged tail) with split-K at a small partition size."""
    pa, runner = _pa()
    hkv = 2
    ctx = [1, bs - 1, bs, bs + 1, 3 * bs, 700, 129]
    w = W.tiny(num_seqs=len(ctx), num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d, block_size=bs,
               dtype=dtype, ctx=ctx, seed=bs + d + g)
    part = max(128, 4 * bs)
    say("small", dtype, d, bs, g, kern, "part", part)
    ref = oracle.run_scenario(w)
    dev = runner.run_script(w, partition_size=part, kernel=KERNELS[kern])
    check_run(w, dev, ref, label=f"{dtype}/D{d}/BS{bs}/g{g}/{kern}")


@pytest.mark.parametrize("part", [64, 128, 256, 512, 1024, 0])
@pytest.mark.parametrize("kern", ["valu", "mfma", "stream"])
def test_partition_sizes(part, kern):
    """Every partition size gives the oracle's result (one partition, many,
    and the merge of ragged ones)."""
    pa, runner = _pa()
    if part and part % (4 * 16):
        pytest.skip("partition must hold 4 blocks")
    w = W.tiny(num_seqs=5, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
               ctx=[1, 63, 64, 1000, 2049], seed=3)
    say("partition", part, kern)
    ref = oracle.run_scenario(w)
    dev = runner.run_script(w, partition_size=part, kernel=KERNELS[kern])
    check_run(w, dev, ref, label=f"part{part}/{kern}")


# --------------------------------------------------------- full configs
@functools.lru_cache(maxsize=1)
def _config(name):
    say("generating", name)
    w = W.build(name)
    say("oracle", name)
    ref = oracle.run_scenario(w)
    return w, ref


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c1_tiny_f32", "c2_gqa_bf16", "c2_gqa_bf16_bs8", "c2_gqa_bf16_bs32",
                                  "c4a_prefix_share", "c4b_prefix_cow", "c3_mha_f16_churn", "c5_long_splitk"])
def test_config_parity(name):
    """The five configurations at full size, in the launch configuration the
    benchmark times (engine steps: one packed host-to-device copy, copy-on-
    write copies, KV write, decode pass and merge): every output row and every
    pool byte."""
    pa, runner = _pa()
    w, ref = _config(name)
    say("device replay", name)
    dev = runner.run_script(w, partition_size=w.cfg.partition_size, use_step=True)
    errs = check_run(w, dev, ref, label=name)
    say(name, "max abs errors", errs)
    if name == "c4a_prefix_share":
        assert all(len(a["pairs"]) == 0 for a in dev.appends)
    if name == "c4b_prefix_cow":
        assert len(dev.appends[0]["pairs"]) == 63
    del dev
    torch.cuda.empty_cache()



@pytest.mark.timeout(600)
def test_fp16_output_is_rounded_fp32():
    """The fp16 output is the fp32 output rounded to nearest even, bit for
    bit, on the fp16 MHA configuration's last decode (256 sequences, 40
    heads: about a thousand items cut between waves and merged, where a
    multiply fused into the fp16 conversion would round the exact product
    once and land on the other side of some ties)."""
    pa, runner = _pa()
    w = W.build("c3_mha_f16_churn")
    say("fp16 output")
    dev = runner.run_script(w)
    eng = dev.engine
    dec = dev.decodes[-1]
    q = dev.q_dev[dec.q_index][torch.tensor(dec.seqs, device="cuda")].contiguous()
    tab = torch.from_numpy(np.ascontiguousarray(dec.tables)).to("cuda")
    ctx = torch.from_numpy(np.asarray(dec.ctx, np.int32)).to("cuda")
    n, hq, d = q.shape
    out32 = torch.empty((n, hq, d), dtype=torch.float32, device="cuda")
    out16 = torch.empty((n, hq, d), dtype=torch.float16, device="cuda")
    for out in (out32, out16):
        ws = eng.workspace(n, hq, int(max(dec.ctx)))
        pa.pa_decode(out, q, eng.k_cache, eng.v_cache, tab, ctx, int(max(dec.ctx)), 1.0 / d ** 0.5,
                     workspace=ws if ws.numel() else None)
    torch.cuda.synchronize()
    diff = int((out32.to(torch.float16).view(torch.int16) != out16.view(torch.int16)).sum())
    say("fp16 output elements off the rounded fp32 one:", diff)
    assert diff == 0
    del dev
    torch.cuda.empty_cache()

@pytest.mark.timeout(600)
def test_half_precision_output_is_rounded_fp32():
    """The bf16 output is the fp32 output rounded to nearest even (torch's
    conversion), bit for bit, on the batch-64 GQA configuration."""
    pa, runner = _pa()
    w, ref = _config("c2_gqa_bf16")
    say("bf16 output")
    dev = runner.run_script(w, out_dtype=torch.bfloat16)
    eng = dev.engine
    q = dev.q_dev[0]
    seqs = list(range(w.cfg.num_seqs))
    out32 = eng.decode(seqs, q, out_dtype=torch.float32)
    out16 = dev.decodes[-1].out
    torch.cuda.synchronize()
    assert torch.equal(out32.to(torch.bfloat16).view(torch.int16), out16.view(torch.int16))
    err = float((out16.double().cpu() - torch.from_numpy(ref.decodes[-1].out)).abs().max())
    say("bf16 output max abs error", err)


# ------------------------------------------------ invariants on the device
def test_permutation_invariance_bitwise():
    """Blocks may sit anywhere in any order: outputs are bit-identical when the
    physical blocks are permuted (the reduction order follows logical
    position only)."""
    pa, runner = _pa()
    outs = []
    for permute in (False, True):
        w = W.tiny(num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                   ctx=[5, 300, 77, 1030], seed=9, permute=permute)
        for kern in (pa.PA_KERNEL_VALU, pa.PA_KERNEL_MFMA, pa.PA_KERNEL_STREAM):
            say("permutation", permute, kern)
            dev = runner.run_script(w, partition_size=256, kernel=kern)
            outs.append((permute, kern, dev.decodes[-1].out.cpu(), dev.decodes[-1].tables))
    for kern in (pa.PA_KERNEL_VALU, pa.PA_KERNEL_MFMA, pa.PA_KERNEL_STREAM):
        a = [o for o in outs if o[1] == kern and not o[0]][0]
        b = [o for o in outs if o[1] == kern and o[0]][0]
        assert not np.array_equal(a[3], b[3])
        assert torch.equal(a[2], b[2])


def test_shared_equals_unshared_bitwise():
    """Sequences whose tables point at one physical prefix give the same
    outputs, bit for bit, as sequences holding private copies."""
    pa, runner = _pa()
    from scenarios import fork_workload
    for prefix in (16, 13):
        res = []
        for share in (True, False):
            w = fork_workload(prefix, [1, 3, 9, 20], share, block_size=8, num_kv_heads=2, num_q_heads=8,
                              head_dim=128)
            say("sharing", prefix, share)
            dev = runner.run_script(w, partition_size=128)
            res.append(dev.decodes[-1].out.cpu())
            if share:
                ref = oracle.run_scenario(w)
                check_run(w, dev, ref, label=f"shared prefix {prefix}")
        assert torch.equal(res[0], res[1])


def test_cow_isolation():
    """After a sharer copies the partial block it writes, the block the others
    still share keeps its bytes and their outputs are unchanged, bit for bit."""
    pa, runner = _pa()
    from scenarios import fork_workload
    w = fork_workload(13, [0, 0, 0], True, block_size=8, num_kv_heads=2, num_q_heads=8, head_dim=128)
    w.ops = w.ops[:4] + [("decode", [0, 1, 2], 0)]
    say("cow isolation: before")
    d0 = runner.run_script(w, partition_size=128)
    last = d0.engine.bm.export([0], 2)[0][0][1]
    kb0 = pool_bits(d0.engine.k_cache)[last].copy()
    vb0 = pool_bits(d0.engine.v_cache)[last].copy()
    w.ops = w.ops[:4] + [("append", [1]), ("decode", [0, 2], 0)]
    say("cow isolation: after")
    d1 = runner.run_script(w, partition_size=128)
    assert d1.appends[0]["pairs"] == [(int(last), int(d1.engine.bm.export([1], 2)[0][0][1]))]
    assert np.array_equal(pool_bits(d1.engine.k_cache)[last], kb0)
    assert np.array_equal(pool_bits(d1.engine.v_cache)[last], vb0)
    assert torch.equal(d1.decodes[-1].out.cpu(), d0.decodes[-1].out.cpu()[[0, 2]])
    ref = oracle.run_scenario(w)
    check_run(w, d1, ref, label="cow")


def test_zero_context_gives_zero_rows():
    pa, runner = _pa()
    from paged_kv_cache_332_amd.engine import PagedKVEngine
    say("zero context")
    eng = PagedKVEngine(16, 2, 128, 16, torch.bfloat16, max_seqs=3, max_context=64)
    rows = torch.randn(40, 2, 128, device="cuda").to(torch.bfloat16)
    eng.add_seq(0, None, None, 0)
    eng.add_seq(1, rows, rows, 40)
    eng.add_seq(2, None, None, 0)
    q = torch.randn(3, 8, 128, device="cuda").to(torch.bfloat16)
    for kern in (pa.PA_KERNEL_VALU, pa.PA_KERNEL_MFMA, pa.PA_KERNEL_STREAM):
        out = eng.decode([0, 1, 2], q, kernel=kern)
        torch.cuda.synchronize()
        assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
        assert torch.all(torch.isfinite(out[1])) and torch.any(out[1] != 0)


def test_write_kv_skips_negative_slots():
    pa, runner = _pa()
    say("negative slots")
    k, v = pa.alloc_cache(4, 2, 64, 8, torch.float16)
    before_k, before_v = pool_bits(k), pool_bits(v)
    x = torch.randn(3, 2, 64, device="cuda").to(torch.float16)
    slots = torch.tensor([-1, 9, -5], dtype=torch.int32, device="cuda")
    pa.pa_write_kv(k, v, x, x, slots)
    torch.cuda.synchronize()
    after_k, after_v = pool_bits(k), pool_bits(v)
    changed = np.argwhere(after_k != before_k)
    assert set(changed[:, 0].tolist()) == {1} and set(changed[:, 3].tolist()) == {1}
    cm = oracle.PagedCacheModel(4, 2, 64, 8, "f16")
    cm.write([-1, 9, -5], x.float().cpu().numpy(), x.float().cpu().numpy())
    assert np.array_equal(after_k, cm.k) and np.array_equal(after_v, cm.v)


def test_large_logits_stay_finite():
    """Scores far apart (query x 64): the running-maximum softmax neither
    overflows nor loses the dominant token."""
    pa, runner = _pa()
    w = W.tiny(num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
               ctx=[40, 600, 1500], seed=4)
    w.q_sets = [W.round_to_dtype(w.q_sets[0] * 64.0, "bf16")]
    ref = oracle.run_scenario(w)
    for kern in (pa.PA_KERNEL_VALU, pa.PA_KERNEL_MFMA, pa.PA_KERNEL_STREAM):
        say("large logits", kern)
        dev = runner.run_script(w, partition_size=256, kernel=kern)
        check_run(w, dev, ref, label=f"large logits {kern}")


@pytest.mark.parametrize("case", ["tiny_ctx", "many_seqs", "one_seq", "mixed_zero"])
def test_stream_work_split(case):
    """The stream kernel splits the tile list of all (sequence, kv head)
    items evenly over its waves: fewer tiles than waves, many one-token
    sequences, one long sequence cut over many waves, empty sequences mixed
    in.  Every output row matches the oracle; a second call on the same
    workspace (counters left at zero) gives bit-identical results."""
    pa, runner = _pa()
    if case == "tiny_ctx":
        kw = dict(ctx=[1, 2, 3, 5, 8, 13, 21], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16)
    elif case == "many_seqs":
        kw = dict(ctx=list(np.random.default_rng(11).integers(1, 40, size=300)), num_q_heads=4, num_kv_heads=4,
                  head_dim=64, block_size=8)
    elif case == "one_seq":
        kw = dict(ctx=[70000], num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=32)
    else:
        kw = dict(ctx=[0, 600, 0, 0, 33, 4000, 0], num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16)
    w = W.tiny(num_seqs=len(kw["ctx"]), dtype="bf16", seed=21, **kw)
    if case == "mixed_zero":
        # empty sequences are added with no tokens, skip the append and are decoded
        ctx = [int(x) for x in kw["ctx"]]
        w.ops = [w.ops[0]] + [("add_seq", i, max(n - 1, 0), True) for i, n in enumerate(ctx)] + \
            [("append", [i for i, n in enumerate(ctx) if n > 0]), ("decode", list(range(len(ctx))), 0)]
    say("stream split", case)
    ref = oracle.run_scenario(w)
    dev = runner.run_script(w, kernel=pa.PA_KERNEL_STREAM)
    check_run(w, dev, ref, label=f"stream {case}")
    eng = dev.engine
    seqs = dev.decodes[-1].seqs
    q = dev.q_dev[dev.decodes[-1].q_index][torch.tensor(seqs, device="cuda")].contiguous()
    again = eng.decode(seqs, q, kernel=pa.PA_KERNEL_STREAM)
    torch.cuda.synchronize()
    assert torch.equal(again, dev.decodes[-1].out)


@pytest.mark.parametrize("case", ["random", "one_heavy", "alternating"])
def test_stream_weights(case):
    """The stream kernel's workgroup weights change only how the tile list is
    split: random weights over the whole valid range, one workgroup holding
    nearly all the work (most workgroups empty) and alternating light and
    heavy ones all match the oracle through the fused step, and the kernel
    writes a start and end stamp for every wave."""
    pa, runner = _pa()
    ctx = [3000, 17, 900, 4100, 1, 250, 1024, 2000]
    hq, hkv, d = 32, 8, 128
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=23, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv,
               head_dim=d, block_size=16)
    g = pa.pa_decode_stream_grid(len(ctx), hq, hkv, d)
    assert g > 0

    def set_weights(eng):
        wt = eng.weights(len(ctx), hq)
        assert wt is not None and wt.shape == (g,)
        if case == "random":
            wt[:] = np.random.default_rng(5).integers(1, 65537, size=g)
        elif case == "one_heavy":
            wt[:] = 1
            wt[g // 3] = 65536
        else:
            wt[:] = np.where(np.arange(g) % 2 == 0, 1, 1000)

    say("stream weights", case, "grid", g)
    ref = oracle.run_scenario(w)
    dev = runner.run_script(w, use_step=True, kernel=pa.PA_KERNEL_STREAM, on_engine=set_weights)
    check_run(w, dev, ref, label=f"weights {case}")
    eng = dev.engine
    st = eng._ring[(eng._ri - 1) % len(eng._ring)]
    t = st.times[: 8 * g].numpy().astype(np.int64).reshape(g, 4, 2)
    span = (t[:, :, 1] - t[:, :, 0] + (1 << 31)) % (1 << 32) - (1 << 31)
    assert (span >= 0).all() and span.max() > 0


@pytest.mark.parametrize("kern", ["auto", "mfma"])
def test_step_layer_reuses_the_record(kern):
    """A second layer run on the last step's record (pa_step_layer: its own
    pools, new tokens and queries; the same slots, tables and split): with a
    copy of the first layer's pools it reproduces the first layer's output
    bit for bit, and with every value of V negated (pool and new token) it
    gives the negated output, so it reads its own pools (to 1e-6: the matrix
    cores' accumulation need not round symmetrically about zero).  The first
    layer matches the oracle."""
    pa, runner = _pa()
    ctx = [700, 33, 1500, 16, 2049, 5]
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=31, ctx=ctx, num_q_heads=16, num_kv_heads=4, head_dim=128,
               block_size=16)
    say("step layer", kern)
    ref = oracle.run_scenario(w)
    dev = runner.run_script(w, use_step=True, kernel=KERNELS[kern])
    check_run(w, dev, ref, label=f"layer 0 {kern}")
    eng = dev.engine
    seqs = dev.decodes[-1].seqs
    a = dev.appends[-1]
    rows = np.array([w.row_of(s, np.array([p]))[0] for s, p in zip(a["seqs"], a["pos"])], dtype=np.int64)
    idx = torch.from_numpy(rows).to("cuda")
    k_new, v_new = dev.k_dev[idx].contiguous(), dev.v_dev[idx].contiguous()
    q = dev.q_dev[dev.decodes[-1].q_index][torch.tensor(seqs, device="cuda")].contiguous()
    out0 = dev.decodes[-1].out
    kb, vb = eng.k_cache.clone(), eng.v_cache.clone()
    out1 = torch.empty_like(out0)
    eng.step_layer(kb, vb, k_new, v_new, q, out1)
    vn = -eng.v_cache
    out2 = torch.empty_like(out0)
    eng.step_layer(eng.k_cache.clone(), vn, k_new, (-v_new).contiguous(), q, out2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out0)
    err = float((out2 + out0).abs().max())
    say("negated V: max |out2 + out0|", err)
    assert err <= 1e-6 and float(out0.abs().max()) > 0.1
    assert torch.equal(kb.view(torch.int16), eng.k_cache.view(torch.int16))


@pytest.mark.parametrize("prefix,bs", [(13, 8), (40, 16), (64, 32)])
def test_step_marks_shared_prefix_blocks(prefix, bs):
    """Forked sequences decoded through pa_step (the path that tells the pass
    which leading blocks other sequences share, so that their loads stay
    cached): the step record's counts equal the oracle model's (blocks with
    refcount above one at the front of each table, after the step's
    copy-on-write), and the outputs equal those of unshared copies bit for
    bit and the oracle within tolerance."""
    pa, runner = _pa()
    from scenarios import fork_workload
    res = []
    for share in (True, False):
        w = fork_workload(prefix, [3, 3, 3, 3], share, block_size=bs, num_kv_heads=2, num_q_heads=8,
                          head_dim=128)
        say("step over shared prefix", prefix, bs, share)
        dev = runner.run_script(w, use_step=True)
        res.append(dev.decodes[-1].out.cpu())
        ref = oracle.run_scenario(w)
        check_run(w, dev, ref, label=f"step prefix {prefix} share {share}")
        eng = dev.engine
        st = eng._ring[(eng._ri - 1) % len(eng._ring)]
        n = len(ref.decodes[-1].seqs)
        at = 4 * n + n * eng.stride + n + 1
        got = st.h[at: at + n].numpy()
        want = []
        for s in ref.decodes[-1].seqs:
            t = ref.bm.table(s)[: -(-ref.bm.length(s) // bs)]
            k = 0
            while k < len(t) and ref.bm.refcount(t[k]) > 1:
                k += 1
            want.append(k)
        assert list(got) == want, (list(got), want)
        assert (max(want) > 0) == share
    assert torch.equal(res[0], res[1])


@pytest.mark.parametrize("n,kern", [(1024, "stream"), (1100, "auto")])
def test_largest_batches(n, kern):
    """The stream kernel's largest batch (1024 sequences, every length and
    prefix sum held in LDS) and one sequence more under automatic selection,
    which then runs the per-partition kernel: short ragged contexts, every
    output row against the oracle."""
    pa, runner = _pa()
    ctx = list(np.random.default_rng(n).integers(1, 24, size=n))
    w = W.tiny(num_seqs=n, ctx=ctx, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=8, dtype="bf16",
               seed=3)
    say("largest batch", n, kern)
    ref = oracle.run_scenario(w)
    k = pa.PA_KERNEL_STREAM if kern == "stream" else pa.PA_KERNEL_AUTO
    dev = runner.run_script(w, kernel=k)
    check_run(w, dev, ref, label=f"batch {n} {kern}")
    if kern == "stream":
        with pytest.raises(pa.PAError):
            w2 = W.tiny(num_seqs=n + 1, ctx=ctx + [5], num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=8,
                        dtype="bf16", seed=3)
            runner.run_script(w2, kernel=pa.PA_KERNEL_STREAM)


# ------------------------------------------- every tile counted exactly once
def _position_coded(name=None, ctx=None, hq=64, hkv=8, d=128, bs=32, seed=0):
    """A workload whose keys are identical within each kv head and whose
    values encode each token's position: V[t][h][c] = (t + 5h + c) mod 128 -
    64.  Every score of a (sequence, head) is the same number, so every
    kernel's softmax weight is exactly 2^0 = 1 and the output is the mean of V
    over the context (the oracle's identical-keys closed form).  The values
    are small integers, so every partial sum is an integer below 2^24 and
    exact in fp32 whatever the order: the kernels' only rounding is the final
    division (<= 2 ulp of |out| <= 64, under 2e-5).  A tile dropped or counted
    twice moves some output element by at least 16 x 63.5 / ctx (6.8e-3 at
    131072 tokens), one token past the context by at least 4.8e-4."""
    if name is not None:
        w = W.build(name, values=False)
        hq, hkv, d = w.cfg.num_q_heads, w.cfg.num_kv_heads, w.cfg.head_dim
    else:
        w = W.tiny(num_seqs=len(ctx), num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, dtype="bf16",
                   ctx=ctx, seed=seed)
    rng = np.random.default_rng([901, seed])
    R = int(np.sum(w.ctx))
    kvec = W.round_to_dtype(rng.standard_normal((1, hkv, d), dtype=np.float32), "bf16")
    w.k_rows = np.broadcast_to(kvec, (R, hkv, d))
    pos = np.concatenate([np.arange(int(n), dtype=np.int64) for n in w.ctx])
    v = np.empty((R, hkv, d), np.float32)
    code = 5 * np.arange(hkv)[None, :, None] + np.arange(d)[None, None, :]
    for i in range(0, R, 1 << 16):
        v[i:i + (1 << 16)] = (pos[i:i + (1 << 16), None, None] + code) % 128 - 64
    w.v_rows = v
    w.q_sets = [W.round_to_dtype(rng.standard_normal((len(w.ctx), hq, d), dtype=np.float32), "bf16")]
    return w


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", ["c5_long_splitk", "mixed_bs16", "mixed_bs8"])
def test_every_tile_counted_once(case):
    """Position-coded values with identical keys (see _position_coded) at the
    long-context configuration's full size (8 sequences of 32k..131k tokens,
    64 query / 8 kv heads, block size 32, 512-token partitions) and on ragged
    mixes at block sizes 16 and 8: the fused step (stream kernel with the
    host plan), pa_decode's stream kernel without a plan, and the 512-token
    partition kernels (matrix-core and vector) with their log-sum-exp merge
    each give the oracle's result within 1e-4, so no tile is dropped, doubled
    or read past the context on any decode path."""
    pa, runner = _pa()
    if case == "c5_long_splitk":
        w = _position_coded("c5_long_splitk")
    elif case == "mixed_bs16":
        w = _position_coded(ctx=[70000, 1, 17, 40000, 33, 2049, 512, 511], hq=32, hkv=8, bs=16, seed=1)
    else:
        w = _position_coded(ctx=[20000, 9, 3000, 1, 15000, 16], hq=16, hkv=4, d=64, bs=8, seed=2)
    say("position coded", case, "contexts", [int(x) for x in w.ctx])
    scale = w.cfg.scale
    want = []
    q = w.q_sets[0]
    for i, n in enumerate(w.ctx):
        rows = w.row_of(i, np.arange(int(n)))
        want.append(oracle.decode_attention(q[i], w.k_rows[rows], w.v_rows[rows], scale))
    want = np.stack(want)
    dev = runner.run_script(w, partition_size=512, use_step=True)
    eng = dev.engine
    seqs = dev.decodes[-1].seqs
    qd = dev.q_dev[0][torch.tensor(seqs, device="cuda")].contiguous()
    outs = {"step stream": dev.decodes[-1].out}
    for label, kern in (("stream", pa.PA_KERNEL_STREAM), ("mfma 512", pa.PA_KERNEL_MFMA),
                        ("valu 512", pa.PA_KERNEL_VALU)):
        outs[label] = eng.decode(seqs, qd, partition_size=512, kernel=kern)
    torch.cuda.synchronize()
    for label, o in outs.items():
        err = float(np.max(np.abs(o.double().cpu().numpy() - want)))
        say("position coded", case, label, "max abs error", err)
        assert err <= 1e-4, f"{case} {label}: max abs error {err:.3e}"
    del dev, eng
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kern", ["mfma", "valu"])
def test_long_context_partition_kernels(kern):
    """The long-context configuration at full size through the 512-token
    partition kernels and the log-sum-exp merge (pa_decode with an explicit
    kernel, on the pools the fused step built): every output row within the
    absolute and the relative bound of the oracle."""
    pa, runner = _pa()
    w, ref = _config("c5_long_splitk")
    say("c5 partition kernels", kern)
    dev = runner.run_script(w, partition_size=512, use_step=True)
    eng = dev.engine
    d = dev.decodes[-1]
    q = dev.q_dev[d.q_index][torch.tensor(d.seqs, device="cuda")].contiguous()
    out = eng.decode(d.seqs, q, partition_size=512, kernel=KERNELS[kern])
    torch.cuda.synchronize()
    r = ref.decodes[-1]
    got = out.double().cpu().numpy()
    err = float(np.max(np.abs(got[r.computed] - r.out[r.computed])))
    scale = float(np.max(np.abs(r.out[r.computed])))
    say("c5", kern, "max abs error", err, "max|ref|", scale)
    assert err <= TOL["bf16"] and err <= REL * scale
    del dev, eng
    torch.cuda.empty_cache()


def test_weights_change_only_rounding():
    """The stream kernel's workgroup weights move the cuts between waves,
    hence the summation and merge order: outputs under very different
    weights (the engine's initial per-die shares, random, a ramp) agree to
    rounding (far inside the oracle tolerance), and the same weights give
    the same bits again."""
    pa, runner = _pa()
    ctx = [3000, 17, 900, 4100, 1, 250, 1024, 2000, 33, 700]
    hq, hkv, d = 32, 8, 128
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=29, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=16)
    g = pa.pa_decode_stream_grid(len(ctx), hq, hkv, d)
    ref = oracle.run_scenario(w)

    def run(kind):
        def set_weights(eng):
            wt = eng.weights(len(ctx), hq)
            if kind == "random":
                wt[:] = np.random.default_rng(8).integers(1, 65537, size=g)
            elif kind == "ramp":
                wt[:] = 1 + 64 * np.arange(g)
        dev = runner.run_script(w, use_step=True, kernel=pa.PA_KERNEL_STREAM, on_engine=set_weights)
        check_run(w, dev, ref, label=f"weights {kind}")
        return dev.decodes[-1].out.cpu()

    outs = {k: run(k) for k in ("initial", "random", "ramp", "initial again")}
    assert torch.equal(outs["initial"], outs["initial again"])
    top = float(outs["initial"].abs().max())
    for k in ("random", "ramp"):
        diff = float((outs[k] - outs["initial"]).abs().max())
        say("weights", k, "max |difference| to the initial shares", diff, "max|out|", top)
        assert diff <= 1e-5 * top        # measured 7e-7 x max|out|
