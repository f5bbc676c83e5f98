"""pa_decode_noalloc (the decode entry point that allocates nothing: its
workspace is the library's static device scratch) against pa_decode with a
workspace the caller allocates, through the C ABI: two calls in a row, the
second with a smaller input, each bit-identical to pa_decode and within
tolerance of the float64 oracle; a call that needs more workspace than the
scratch holds is refused before anything runs."""
import os
import re
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def scratch_bytes() -> int:
    m = re.search(r"#define PA_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def _case(w, kernel_note):
    """One decode of workload w through both entry points on the same pools
    and tables; returns the max abs error against the oracle."""
    import paged_kv_cache_332_amd as pa
    from paged_kv_cache_332_amd import runner
    say("no-alloc decode", kernel_note, "contexts", [int(x) for x in w.ctx])
    ref = oracle.run_scenario(w)
    dev = runner.run_script(w)
    eng = dev.engine
    d = dev.decodes[-1]
    seqs = d.seqs
    q = dev.q_dev[d.q_index][torch.tensor(seqs, device="cuda")].contiguous()
    tab = torch.from_numpy(np.ascontiguousarray(d.tables)).to("cuda")
    ctx = torch.from_numpy(np.ascontiguousarray(d.ctx, dtype=np.int32)).to("cuda")
    max_ctx = int(d.ctx.max())
    part = w.cfg.partition_size
    need = pa.pa_decode_workspace_bytes(len(seqs), q.shape[1], eng.H, eng.D, max_ctx, part)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    with_ws = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    no_ws = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_decode(with_ws, q, eng.k_cache, eng.v_cache, tab, ctx, max_ctx, w.cfg.scale, part, ws)
    pa.pa_decode_noalloc(no_ws, q, eng.k_cache, eng.v_cache, tab, ctx, max_ctx, w.cfg.scale, part)
    torch.cuda.synchronize()
    assert torch.equal(no_ws, with_ws), "pa_decode_noalloc differs from pa_decode"
    r = ref.decodes[-1]
    err = float(np.max(np.abs(no_ws.double().cpu().numpy()[r.computed] - r.out[r.computed])))
    tol = 1e-5 if w.cfg.dtype == "f32" else 2e-3
    assert err <= tol, err
    return err


def test_noalloc_matches_pa_decode_twice():
    """A batch-64 grouped-query bf16 decode (stream kernel, its per-wave
    records in the scratch), then a smaller fp32 one whose sequences span
    several 128-token partitions (vector kernel, its partials in the same
    scratch, which still holds the first call's bytes)."""
    big = W.tiny(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                 ctx=list(np.random.default_rng(5).integers(128, 4097, size=64)), seed=51)
    e1 = _case(big, "bf16 batch 64")
    small = W.tiny(num_seqs=5, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=8, dtype="f32",
                   ctx=[1, 9, 300, 1000, 129], seed=52)
    small.cfg = W.Config(small.cfg.name, 0, 5, 8, 2, 64, 8, "f32", partition_size=128)
    e2 = _case(small, "f32 batch 5")
    say("no-alloc decode max abs errors", e1, e2)


def test_noalloc_refuses_more_than_its_scratch():
    """fp32 with 64-token partitions over 256 sequences of up to 4096 tokens
    needs 256 x 40 x 64 x 130 x 4 bytes (340 MB) of partials: refused with a
    message naming the scratch, before any launch."""
    import paged_kv_cache_332_amd as pa
    k, v = pa.alloc_cache(8, 40, 128, 16, torch.float32)
    q = torch.zeros((256, 40, 128), dtype=torch.float32, device="cuda")
    out = torch.zeros_like(q)
    tab = torch.zeros((256, 256), dtype=torch.int32, device="cuda")
    ctx = torch.ones(256, dtype=torch.int32, device="cuda")
    need = 256 * 40 * 64 * (128 + 2) * 4
    assert need > scratch_bytes()
    with pytest.raises(pa.PAError, match="static scratch"):
        pa.pa_decode_noalloc(out, q, k, v, tab, ctx, 4096, 0.088, 64)
    torch.cuda.synchronize()
    assert not out.any()
