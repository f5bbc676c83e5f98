"""Small hand-built scripts shared by the oracle tests and the GPU tests."""
import numpy as np

import workloads as W


def fork_workload(prefix, suffix, share: bool, block_size=8, num_kv_heads=2, num_q_heads=4,
                  head_dim=64, dtype="bf16", seed=5):
    """Sequences with a common prefix, either forked from sequence 0 (shared
    blocks, copy-on-write on divergence) or added as independent copies; then
    each appends its suffix tokens step by step and all are decoded."""
    base = W.tiny(num_seqs=len(suffix), ctx=[prefix + s for s in suffix], block_size=block_size,
                  num_kv_heads=num_kv_heads, num_q_heads=num_q_heads, head_dim=head_dim, dtype=dtype,
                  seed=seed)
    B = len(suffix)
    row_start = base.row_start.copy()
    w = W.Workload(base.cfg, base.ctx, base.k_rows, base.v_rows, base.q_sets, [],
                   4 * int(base.num_blocks) + 64, row_start, 0)

    def row_of(seq, positions):
        positions = np.asarray(positions, dtype=np.int64)
        # every sequence reads sequence 0's rows for the prefix
        return np.where(positions < prefix, positions, row_start[seq] + positions)
    w.row_of = row_of
    ops = [("create", w.num_blocks, None)]
    if share:
        ops.append(("add_seq", 0, prefix, True))
        ops += [("fork", 0, i) for i in range(1, B)]
    else:
        ops += [("add_seq", i, prefix, True) for i in range(B)]
    done = [0] * B
    while any(done[i] < suffix[i] for i in range(B)):
        step = [i for i in range(B) if done[i] < suffix[i]]
        ops.append(("append", step))
        for i in step:
            done[i] += 1
    ops.append(("decode", list(range(B)), 0))
    w.ops = ops
    return w
