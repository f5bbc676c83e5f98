"""The waste and admission table of the accounting model — TEST
INFRASTRUCTURE ONLY: ``python -m oracle.waste_table`` prints one JSON line.

The 13B-like MHA configuration's traffic (``workloads.admission_trace``:
lognormal lengths, about 256 requests live) replayed against that
configuration's own pool (its blocks x block size token slots) three ways:
contiguous runs of the longest context (4096), contiguous runs of each
request's own length, and blocks from a shared free list.  Plus the pages'
worked internal-waste figure (4096-token reservations holding 512-token
requests).  Calls only this package and the seeded inputs.
"""
from __future__ import annotations

import json

import workloads as W

from . import accounting as A


def table() -> dict:
    w = W.build("c3_mha_f16_churn", values=False)
    bs = w.cfg.block_size
    cap = w.num_blocks * bs
    ev, lengths = W.admission_trace()
    rows = {p: A.replay_admissions(ev, p, cap, bs, 4096) for p in ("slab_max", "slab_exact", "paged")}
    for r in rows.values():
        for k in ("mean_live", "reserved_unused", "used_fraction"):
            r[k] = round(r[k], 4)
    return {"trace": {"requests": int(len(lengths)), "mean_length": round(float(lengths.mean()), 1),
                      "pool_tokens": cap, "block_size": bs, "max_len": 4096},
            "policies": rows,
            "worked_example": {"max_len": 4096, "mean_len": 512,
                               "unused_fraction": A.reserve_max_waste([512], 4096)}}


if __name__ == "__main__":
    print(json.dumps(table()))
