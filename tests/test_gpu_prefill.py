"""Paged prefill (pa_prefill) against the CPU oracle on an MI355X: chunks of
new tokens attend causally over their sequences' paged context.  Outputs
(fp32) must be within 2e-3 of the float64 oracle for 16-bit caches."""
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


# dtype, head_dim, block size, q heads, kv heads, context lengths, chunk lengths
CASES = {
    "gqa4_bf16_bs16": ("bf16", 128, 16, 32, 8, [300, 17, 1, 2049, 64], [300, 5, 1, 100, 64]),
    "mha_f16_bs8": ("f16", 64, 8, 8, 8, [40, 129, 7], [40, 33, 7]),
    "gqa8_bf16_bs32": ("bf16", 128, 32, 64, 8, [1000, 260], [250, 1]),
    "gqa16_bf16_d64": ("bf16", 64, 16, 16, 1, [77, 33], [77, 20]),
    "gqa2_f16_bs16": ("f16", 128, 16, 8, 4, [513, 1], [512, 1]),
    "long_context_bf16": ("bf16", 128, 16, 32, 8, [9000, 300], [64, 300]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_matches_oracle(case):
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    dtype, d, bs, hq, hkv, ctx, chunk = CASES[case]
    say("prefill", case)
    w = W.tiny(num_seqs=len(ctx), dtype=dtype, seed=41, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    seqs = list(range(len(ctx)))
    tab, ctx_now = eng.bm.export(seqs, eng.stride)
    assert list(ctx_now) == list(ctx)
    rng = np.random.default_rng([41, len(ctx)])
    T = int(sum(chunk))
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), dtype)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    tdt = runner.TORCH_DTYPE[dtype]
    q_dev = torch.from_numpy(q).to("cuda").to(tdt)
    out = torch.full((T, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1.0 / d ** 0.5
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"),
                  torch.from_numpy(qs).to("cuda"), torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"),
                  max(chunk), max(ctx), scale)
    # half-precision output: the fp32 result rounded to the cache dtype
    out_h = torch.empty((T, hq, d), dtype=tdt, device="cuda")
    pa.pa_prefill(out_h, q_dev, eng.k_cache, eng.v_cache, torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"),
                  torch.from_numpy(qs).to("cuda"), torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"),
                  max(chunk), max(ctx), scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = 0.0
    for i, (n, L) in enumerate(zip(ctx, chunk)):
        rows = w.row_of(i, np.arange(n))
        ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[rows], w.v_rows[rows], scale)
        err = max(err, float(np.max(np.abs(got[qs[i]: qs[i + 1]] - ref))))
    say(case, "max abs error", err)
    assert err <= 2e-3
    assert torch.equal(out_h, out.to(tdt))


def test_prefill_of_one_token_is_decode():
    """A one-token chunk is a decode step: pa_prefill agrees with the oracle's
    decode over the whole context, and so does pa_decode on the same row."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    ctx = [1, 300, 4000]
    w = W.tiny(num_seqs=3, dtype="bf16", seed=5, ctx=ctx, num_q_heads=32, num_kv_heads=8, head_dim=128,
               block_size=16)
    dev = runner.run_script(w)
    eng = dev.engine
    dec = dev.decodes[-1]
    q_dev = dev.q_dev[dec.q_index][torch.tensor(dec.seqs, device="cuda")].contiguous()
    out = torch.empty((3, 32, 128), dtype=torch.float32, device="cuda")
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, torch.from_numpy(np.ascontiguousarray(dec.tables)).to("cuda"),
                  torch.arange(4, dtype=torch.int32, device="cuda"),
                  torch.from_numpy(np.asarray(dec.ctx, np.int32)).to("cuda"), 1, max(ctx), 1.0 / 128 ** 0.5)
    torch.cuda.synchronize()
    ref = oracle.run_scenario(w).decodes[-1].out
    assert float(np.max(np.abs(out.cpu().numpy() - ref))) <= 2e-3
    assert float(torch.max(torch.abs(out - dec.out))) <= 2e-3


def test_prefill_rejects_bad_arguments():
    import paged_kv_cache_332_amd as pa
    k = torch.zeros((4, 2, 8, 16, 8), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((4, 2, 64, 16), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((3, 8, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((3, 8, 64), dtype=torch.float32, device="cuda")
    tab = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    qs = torch.tensor([0, 3], dtype=torch.int32, device="cuda")
    cl = torch.tensor([3], dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PAError):
        pa.pa_prefill(out, q, k, v, tab, qs, cl, 5, 3, 0.1)       # chunk longer than the context bound
    with pytest.raises(pa.PAError):
        pa.pa_prefill(out, q, k, v, tab, qs, cl, 3, 100, 0.1)     # table stride too short for the bound
    with pytest.raises(pa.PAError):
        pa.pa_prefill(out, q, k.float(), v.float(), tab, qs, cl, 3, 3, 0.1)  # fp32 cache


# dtype, head_dim, block size, q heads, kv heads, sequences, chunk, context range: batches large
# enough for two column blocks per wave, three for the *_three_blocks cases (the same sequence
# alone takes one)
WIDE = {
    # (8 sequences: 1024 workgroups with two column blocks, 704 with three)
    "gqa4_bf16_bs16": ("bf16", 128, 16, 32, 8, 8, 512, (520, 1400)),
    "gqa4_bf16_bs16_three_blocks": ("bf16", 128, 16, 32, 8, 32, 768, (770, 1200)),
    "mha_f16_bs8_d64_three_blocks": ("f16", 64, 8, 16, 16, 16, 3072, (3072, 3400)),
    "mha_f16_bs8_d64": ("f16", 64, 8, 16, 16, 8, 1024, (1030, 1500)),
    "gqa8_bf16_bs32": ("bf16", 128, 32, 64, 8, 8, 256, (300, 2000)),
    "gqa16_bf16_d64": ("bf16", 64, 16, 16, 1, 8, 1024, (1024, 1300)),
    # bf16 with three column blocks converts the values to fp16: every block
    # size, both head dims and groups 1, 4, 8 and 16 (batches of >= 4096
    # workgroups)
    "gqa4_bf16_bs8_three_blocks": ("bf16", 128, 8, 32, 8, 32, 768, (770, 1000)),
    "gqa4_bf16_bs32_three_blocks": ("bf16", 128, 32, 32, 8, 32, 768, (770, 1000)),
    "gqa4_bf16_d64_three_blocks": ("bf16", 64, 16, 16, 4, 32, 1536, (1536, 1700)),
    "gqa8_bf16_three_blocks": ("bf16", 128, 16, 64, 8, 16, 768, (768, 900)),
    "gqa16_bf16_d64_three_blocks": ("bf16", 64, 16, 16, 1, 16, 3072, (3072, 3200)),
    "mha_bf16_d64_three_blocks": ("bf16", 64, 16, 16, 16, 16, 3072, (3072, 3200)),
    # contexts past 512 tiles: the block ids are staged again inside the
    # conversion pipeline
    "gqa4_bf16_long_three_blocks": ("bf16", 128, 16, 32, 8, 8, 3072, (8400, 9200)),
}


@pytest.mark.parametrize("case", list(WIDE))
def test_prefill_wide_workgroups_match_narrow(case):
    """A batch large enough for two or three column blocks per wave gives,
    for every sequence, the same bits as that sequence prefilled alone (one
    column block per wave): both take the same tiles in the same order per
    column.  The exception is bf16 with three column blocks, whose P V runs
    as one fp16 product against values converted to fp16 (one column block
    splits P into two bf16 products): there the two agree to 2e-3.
    Sampled rows also match the oracle's decode at their positions."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    dtype, d, bs, hq, hkv, B, L, (lo, hi) = WIDE[case]
    rng = np.random.default_rng([77, len(case)])
    ctx = [int(x) for x in rng.integers(lo, hi, B)]
    chunk = [L] * B
    say("prefill wide vs narrow", case)
    w = W.tiny(num_seqs=B, dtype=dtype, seed=78, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, ctx_now = eng.bm.export(list(range(B)), eng.stride)
    T = sum(chunk)
    tdt = runner.TORCH_DTYPE[dtype]
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), dtype)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev = torch.from_numpy(q).to("cuda").to(tdt)
    scale = 1.0 / d ** 0.5
    out = torch.full((T, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"),
                  torch.from_numpy(qs).to("cuda"), torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"),
                  L, max(ctx), scale)
    for i in range(B):
        one = torch.full((chunk[i], hq, d), float("nan"), dtype=torch.float32, device="cuda")
        pa.pa_prefill(one, q_dev[qs[i]: qs[i + 1]].contiguous(), eng.k_cache, eng.v_cache,
                      torch.from_numpy(np.ascontiguousarray(tab[i: i + 1])).to("cuda"),
                      torch.tensor([0, chunk[i]], dtype=torch.int32, device="cuda"),
                      torch.tensor([ctx[i]], dtype=torch.int32, device="cuda"), chunk[i], ctx[i], scale)
        torch.cuda.synchronize()
        if dtype == "bf16" and case.endswith("three_blocks"):
            assert float(torch.max(torch.abs(one - out[qs[i]: qs[i + 1]]))) <= 2e-3, i
        else:
            assert torch.equal(one.view(torch.int32), out[qs[i]: qs[i + 1]].view(torch.int32)), i
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = 0.0
    for i in range(0, B, 3):
        rows = w.row_of(i, np.arange(ctx[i]))
        K, V = w.k_rows[rows], w.v_rows[rows]
        for t in sorted({0, 1, 15, 16, 63, L // 2, L - 1}):
            pos = ctx[i] - chunk[i] + t
            ref = oracle.decode_attention(q[qs[i] + t], K[: pos + 1], V[: pos + 1], scale)
            err = max(err, float(np.max(np.abs(got[qs[i] + t] - ref))))
    say(case, "wide prefill sampled max abs error", err)
    assert err <= 2e-3


def test_prefill_empty_chunks_and_no_rows():
    """Sequences with an empty chunk (no query rows) next to ones with rows,
    and a call with no rows at all: only the real rows are written (the
    rest of the output keeps its NaN fill), and they match the oracle."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    ctx = [40, 1, 300, 17]
    chunk = [0, 1, 0, 17]
    hq, hkv, d, bs = 8, 2, 64, 16
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=61, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    rng = np.random.default_rng(62)
    T = sum(chunk)
    q = W.round_to_dtype(rng.standard_normal((T + 3, hq, d), dtype=np.float32), "bf16")
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev = torch.from_numpy(q).to("cuda").to(torch.bfloat16)
    out = torch.full((T + 3, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    args = (torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"), torch.from_numpy(qs).to("cuda"),
            torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"))
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, *args, max(chunk), max(ctx), 1.0 / d ** 0.5)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i, (n, L) in enumerate(zip(ctx, chunk)):
        if L == 0:
            continue
        rows = w.row_of(i, np.arange(n))
        ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[rows], w.v_rows[rows], 1.0 / d ** 0.5)
        assert float(np.max(np.abs(got[qs[i]: qs[i + 1]] - ref))) <= 2e-3
    assert np.isnan(got[T:]).all()                       # rows past the last chunk untouched
    # no rows at all: nothing is launched and nothing changes
    before = out.clone()
    zero = torch.zeros(len(ctx) + 1, dtype=torch.int32, device="cuda")
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, args[0], zero, args[2], 0, max(ctx), 1.0 / d ** 0.5)
    torch.cuda.synchronize()
    assert torch.equal(out.isnan(), before.isnan()) and torch.equal(out.nan_to_num(), before.nan_to_num())


# scales that take the kernel's other branches: a negative one (the sign of q
# is flipped so that the factor inside the exponent is positive), zero (every
# weight equal) and a large one (peaked rows whose reference maximum is
# raised many times along the context)
SCALES = {"negative": -0.125, "zero": 0.0, "large": 2.0}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("which", list(SCALES))
def test_prefill_scale_sign_zero_and_large(dtype, which):
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    scale = SCALES[which]
    ctx, chunk = [700, 40, 1], [300, 40, 1]
    hq, hkv, d, bs = 16, 4, 128, 16
    say("prefill scale", which, dtype)
    w = W.tiny(num_seqs=len(ctx), dtype=dtype, seed=91, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    rng = np.random.default_rng([92, len(which)])
    T = sum(chunk)
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), dtype)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev = torch.from_numpy(q).to("cuda").to(runner.TORCH_DTYPE[dtype])
    out = torch.full((T, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"),
                  torch.from_numpy(qs).to("cuda"), torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"),
                  max(chunk), max(ctx), scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = 0.0
    for i, n in enumerate(ctx):
        rows = w.row_of(i, np.arange(n))
        ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[rows], w.v_rows[rows], scale)
        err = max(err, float(np.max(np.abs(got[qs[i]: qs[i + 1]] - ref))))
    say(which, dtype, "max abs error", err)
    assert err <= 2e-3


def test_prefill_values_far_from_one():
    """bf16 values far from the unit range (all of them: the prefill keeps
    P V in 16-bit products, whose range must not limit them).  Sequences
    with huge values (2^40), tiny ones (2^-30), a switch from tiny to huge
    along the context, leading zero values, and one outlier of 2^30 in one
    half of the dims of one kv head: every output row is within 2e-3 of the
    oracle relative to the largest value its row sees in the same kv head
    and half of the dims."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    ctx, chunk = [700, 500, 900, 300, 200], [300, 200, 400, 300, 50]
    hq, hkv, d, bs = 16, 4, 128, 16
    say("prefill values far from one")
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=95, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    # powers of two keep every bf16 value exact
    w.v_rows[w.row_of(0, np.arange(700))] *= 2.0 ** 40
    w.v_rows[w.row_of(1, np.arange(500))] *= 2.0 ** -30
    w.v_rows[w.row_of(2, np.arange(450))] *= 2.0 ** -30
    w.v_rows[w.row_of(2, np.arange(450, 900))] *= 2.0 ** 20
    w.v_rows[w.row_of(3, np.arange(100))] = 0.0
    w.v_rows[w.row_of(4, np.array([150])), 0, :4] = 2.0 ** 30
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    rng = np.random.default_rng(96)
    T = sum(chunk)
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), "bf16")
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    out = torch.full((T, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_prefill(out, torch.from_numpy(q).to("cuda").to(torch.bfloat16), eng.k_cache, eng.v_cache,
                  torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"), torch.from_numpy(qs).to("cuda"),
                  torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"), max(chunk), max(ctx), 1.0 / d ** 0.5)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    G = hq // hkv
    worst = 0.0
    for i, (n, L) in enumerate(zip(ctx, chunk)):
        V = w.v_rows[w.row_of(i, np.arange(n))].astype(np.float64)
        ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[w.row_of(i, np.arange(n))], V, 1.0 / d ** 0.5)
        # largest magnitude seen by row t, per kv head and half of the dims
        half_max = np.abs(V).reshape(n, hkv, 2, d // 2).max(axis=3)          # [n, hkv, 2]
        seen = np.maximum.accumulate(half_max, axis=0)[n - L:]               # [L, hkv, 2]
        bound = np.repeat(np.repeat(seen, G, axis=1), d // 2, axis=2)        # [L, hq, d]
        rel = np.abs(got[qs[i]: qs[i + 1]] - ref) / np.maximum(bound, 1e-300)
        say("sequence", i, "max error relative to the values seen", float(rel.max()))
        worst = max(worst, float(rel.max()))
    assert worst <= 2e-3


# ------------------------------------------------------------ context split
def _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, split, out_dtype=torch.float32):
    """pa_prefill of the chunks, with the workspace its context split asks for
    (split=True; the shape must ask for one) or without (one piece each)."""
    T, hq, d = q_dev.shape
    ws = None
    if split:
        nbytes = pa.pa_prefill_workspace_bytes(max(chunk), max(ctx), len(ctx), hq, eng.H, d)
        assert nbytes > 0, "this shape does not split"
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((T, hq, d), float("nan"), dtype=out_dtype, device="cuda")
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"),
                  torch.from_numpy(np.asarray(qs, np.int32)).to("cuda"),
                  torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"), max(chunk), max(ctx), scale, workspace=ws)
    return out


# launches of fewer than 512 workgroups (two per compute unit), which split:
# dtype, head_dim, block size, q heads, kv heads, context lengths, chunk lengths
SPLIT_RANDOM = {
    "gqa4_bf16_bs16": ("bf16", 128, 16, 8, 2, [300, 17, 1, 2049, 64], [300, 5, 1, 100, 64]),
    "gqa8_bf16_bs32": ("bf16", 128, 32, 32, 4, [1000, 260], [250, 1]),
    "long_context_bf16": ("bf16", 128, 16, 32, 8, [9000, 300], [64, 300]),
    "mha_f16_d64_bs8": ("f16", 64, 8, 8, 8, [3000, 129, 7, 1500], [40, 33, 7, 1]),
    "gqa16_bf16_d64": ("bf16", 64, 16, 16, 1, [2000, 33], [77, 20]),
}


@pytest.mark.parametrize("case", list(SPLIT_RANDOM))
def test_prefill_context_split_matches_oracle(case):
    """With a workspace, launches of few workgroups split each sequence's
    prefix into pieces of at least 32 tiles and merge them by log-sum-exp
    (these cases cut their longer contexts into 2 to 7 pieces): within 2e-3 of
    the oracle, and the 16-bit output is the fp32 one rounded."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    dtype, d, bs, hq, hkv, ctx, chunk = SPLIT_RANDOM[case]
    say("prefill split", case)
    w = W.tiny(num_seqs=len(ctx), dtype=dtype, seed=41, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    rng = np.random.default_rng([41, len(ctx)])
    T = int(sum(chunk))
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), dtype)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    tdt = runner.TORCH_DTYPE[dtype]
    q_dev = torch.from_numpy(q).to("cuda").to(tdt)
    scale = 1.0 / d ** 0.5
    out = _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, True)
    out_h = _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, True, out_dtype=tdt)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = 0.0
    for i, n in enumerate(ctx):
        rows = w.row_of(i, np.arange(n))
        ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[rows], w.v_rows[rows], scale)
        err = max(err, float(np.max(np.abs(got[qs[i]: qs[i + 1]] - ref))))
    say(case, "split: max abs error", err)
    assert err <= 2e-3
    assert torch.equal(out_h, out.to(tdt))



# every chunk within one query block of its (sequence, kv head) (4 CB (16 /
# group) tokens with one column block): the launches whose tiles are each
# read by one workgroup, with streaming loads, in one piece and split
# (these batches have fewer than 512 workgroups):
# dtype, head_dim, block size, q heads, kv heads, context lengths, chunk lengths
ONE_BLOCK = {
    "gqa8_bf16_bs32": ("bf16", 128, 32, 64, 8, [3000, 40, 8, 700], [8, 3, 8, 1]),
    "gqa4_bf16_bs8": ("bf16", 128, 8, 32, 8, [2500, 16, 900], [16, 16, 7]),
    "mha_f16_bs16": ("f16", 128, 16, 16, 16, [2100, 64, 333], [64, 50, 1]),
    "gqa16_bf16_d64": ("bf16", 64, 16, 16, 1, [5000, 4, 77], [4, 4, 2]),
}


@pytest.mark.parametrize("case", list(ONE_BLOCK))
def test_prefill_one_query_block_matches_oracle(case):
    """Chunks that fit one query block, over block sizes 8, 16 and 32 and
    groups 1, 4, 8 and 16: in one piece and split, within 2e-3 of the
    oracle, and the 16-bit output is the fp32 one rounded."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    dtype, d, bs, hq, hkv, ctx, chunk = ONE_BLOCK[case]
    g = hq // hkv
    assert max(chunk) <= 4 * (16 // g) and pa.pa_prefill_column_blocks(hq, hkv, max(chunk), len(ctx)) == 1
    say("prefill one query block", case)
    w = W.tiny(num_seqs=len(ctx), dtype=dtype, seed=43, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    rng = np.random.default_rng([43, len(ctx)])
    T = int(sum(chunk))
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), dtype)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    tdt = runner.TORCH_DTYPE[dtype]
    q_dev = torch.from_numpy(q).to("cuda").to(tdt)
    scale = 1.0 / d ** 0.5
    for split in (False, True):
        out = _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, split)
        out_h = _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, split, out_dtype=tdt)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        err = 0.0
        for i, n in enumerate(ctx):
            rows = w.row_of(i, np.arange(n))
            ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[rows], w.v_rows[rows], scale)
            err = max(err, float(np.max(np.abs(got[qs[i]: qs[i + 1]] - ref))))
        say(case, "split" if split else "one piece", "max abs error", err)
        assert err <= 2e-3
        assert torch.equal(out_h, out.to(tdt))

# contexts, chunks, q heads, kv heads, head dim, block size, dtype
SPLIT_CODED = {
    # chunks of at most 16 tokens: one query block per (sequence, kv head),
    # pieces of 32 tiles, up to 18 of them
    "short_bf16_bs16": ([9000, 17, 2049, 300, 4097, 1, 4112, 4111], [16, 5, 16, 16, 1, 1, 16, 16], 32, 8, 128, 16,
                        "bf16"),
    # longer chunks beside short ones: pieces of 114 tiles, the chunk's
    # query blocks in the last piece
    "mixed_bf16_bs16": ([9000, 17, 2049, 300, 4097, 1], [16, 5, 100, 300, 16, 1], 16, 4, 128, 16, "bf16"),
    "short_f16_d64_bs8": ([6000, 257, 1, 3001], [8, 8, 1, 3], 16, 4, 64, 8, "f16"),
    "short_bf16_g16_bs32": ([5000, 640, 33], [1, 16, 16], 16, 1, 128, 32, "bf16"),
}


@pytest.mark.parametrize("case", list(SPLIT_CODED))
def test_prefill_context_split_counts_every_tile_once(case):
    """Keys identical within each kv head and position-coded values
    V[t][h][c] = (t + 5h + c) mod 128 - 64: every weight is exactly 2^0, so
    each query token's output is the mean of V over its prefix, and every
    partial sum is an integer exact in fp32 in any order (pieces and merge
    included: every piece has the same reference, so the merge scales by 1).
    Split and unsplit launches both give the oracle's result within 1e-4; a
    tile dropped or counted twice moves an output by at least 16 x 63.5 /
    9000 = 0.11, one token past a prefix by at least 63.5 / 9000 = 7e-3."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    ctx, chunk, hq, hkv, d, bs, dtype = SPLIT_CODED[case]
    say("prefill split position coded", case)
    w = W.tiny(num_seqs=len(ctx), dtype=dtype, seed=43, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    rng = np.random.default_rng([902, len(ctx)])
    R = int(np.sum(w.ctx))
    kvec = W.round_to_dtype(rng.standard_normal((1, hkv, d), dtype=np.float32), dtype)
    w.k_rows = np.broadcast_to(kvec, (R, hkv, d))
    pos = np.concatenate([np.arange(int(n), dtype=np.int64) for n in w.ctx])
    code = 5 * np.arange(hkv)[None, :, None] + np.arange(d)[None, None, :]
    w.v_rows = ((pos[:, None, None] + code) % 128 - 64).astype(np.float32)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    T = int(sum(chunk))
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), dtype)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev = torch.from_numpy(q).to("cuda").to(runner.TORCH_DTYPE[dtype])
    scale = 1.0 / d ** 0.5
    outs = {"split": _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, True),
            "one piece": _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, False)}
    torch.cuda.synchronize()
    want = np.concatenate([
        oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[w.row_of(i, np.arange(n))],
                                 w.v_rows[w.row_of(i, np.arange(n))], scale)
        for i, n in enumerate(ctx)])
    for label, o in outs.items():
        err = float(np.max(np.abs(o.double().cpu().numpy() - want)))
        say(case, label, "max abs error", err)
        assert err <= 1e-4, f"{case} {label}: max abs error {err:.3e}"


@pytest.mark.parametrize("case", ["ties", "over_rank_limit"])
def test_prefill_sequence_order(case):
    """Workgroups take sequences in order of decreasing context (ranked in
    the kernel, ties by index) up to 256 sequences, in index order beyond:
    every sequence's rows written (the output starts as NaN) and within 2e-3
    of the oracle, with many equal lengths and with 300 sequences."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    rng = np.random.default_rng([44, len(case)])
    if case == "ties":
        ctx = [int(x) for x in rng.choice([33, 200, 517], size=40)]
    else:
        ctx = [int(x) for x in rng.integers(1, 80, size=300)]
    chunk = [int(min(c, x)) for c, x in zip(ctx, rng.integers(1, 40, size=len(ctx)))]
    hq, hkv, d, bs, dtype = 8, 2, 64, 16, "bf16"
    say("prefill order", case, len(ctx), "sequences")
    w = W.tiny(num_seqs=len(ctx), dtype=dtype, seed=45, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    T = int(sum(chunk))
    q = W.round_to_dtype(rng.standard_normal((T, hq, d), dtype=np.float32), dtype)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev = torch.from_numpy(q).to("cuda").to(runner.TORCH_DTYPE[dtype])
    scale = 1.0 / d ** 0.5
    out = _prefill_run(pa, eng, q_dev, tab, qs, ctx, chunk, scale, False)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert np.all(np.isfinite(got))
    err = 0.0
    for i, n in enumerate(ctx):
        rows = w.row_of(i, np.arange(n))
        ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[rows], w.v_rows[rows], scale)
        err = max(err, float(np.max(np.abs(got[qs[i]: qs[i + 1]] - ref))))
    say(case, "max abs error", err)
    assert err <= 2e-3


def test_prefill_context_split_with_empty_chunks():
    """A split launch (workspace given, few workgroups) with empty chunks
    next to split ones: the empty ones write nothing (their workgroups and
    the merge skip them, the output keeps its NaN fill past the rows), the
    others, cut into 2 to 6 pieces, match the oracle."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    ctx = [2000, 1, 3000, 17, 1200, 2600]
    chunk = [0, 1, 0, 17, 5, 16]
    hq, hkv, d, bs = 8, 2, 64, 16
    say("prefill split with empty chunks")
    w = W.tiny(num_seqs=len(ctx), dtype="bf16", seed=63, ctx=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
               block_size=bs)
    dev = runner.run_script(w, decode=False)
    eng = dev.engine
    tab, _ = eng.bm.export(list(range(len(ctx))), eng.stride)
    rng = np.random.default_rng(64)
    T = sum(chunk)
    q = W.round_to_dtype(rng.standard_normal((T + 3, hq, d), dtype=np.float32), "bf16")
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev = torch.from_numpy(q).to("cuda").to(torch.bfloat16)
    nbytes = pa.pa_prefill_workspace_bytes(max(chunk), max(ctx), len(ctx), hq, hkv, d)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((T + 3, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_prefill(out, q_dev, eng.k_cache, eng.v_cache, torch.from_numpy(np.ascontiguousarray(tab)).to("cuda"),
                  torch.from_numpy(qs).to("cuda"), torch.from_numpy(np.asarray(ctx, np.int32)).to("cuda"),
                  max(chunk), max(ctx), 1.0 / d ** 0.5, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i, (n, L) in enumerate(zip(ctx, chunk)):
        if L == 0:
            continue
        rows = w.row_of(i, np.arange(n))
        ref = oracle.prefill_attention(q[qs[i]: qs[i + 1]], w.k_rows[rows], w.v_rows[rows], 1.0 / d ** 0.5)
        assert float(np.max(np.abs(got[qs[i]: qs[i + 1]] - ref))) <= 2e-3, i
    assert np.isnan(got[T:]).all()
