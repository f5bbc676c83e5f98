"""CPU oracle for paged-attention decode — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here, and this package imports nothing from
the product.  The only module both sides share is ``workloads`` (seeded
inputs, no method arithmetic).

What it computes, and from which passage:

* ``attention``  — plain softmax attention of one query per head over the
  logically contiguous sequence, in float64.  The pages say the paged kernel
  follows the block table and reads the logical sequence as if it were laid
  out end to end ("Paged Attention: Virtual Memory for the KV Cache", §The fix
  borrowed from operating systems; glossary "What is Paged Attention?"), so the
  result is exactly textbook attention over the gathered sequence; the pages
  print no formula, so the plainest reading (scaled dot product, scale
  1/sqrt(head_dim), max-subtracted softmax) is used.  ``split_k`` /
  ``lse_merge`` are the same result computed over fixed token partitions and
  recombined by log-sum-exp.  ``prefill_attention`` is the step before decode:
  each new token of a chunk attends to its context up to its own position
  (causal, the plain reading: the pages give no formula).
* ``block_manager`` — a model of the block allocator the pages describe: a
  shared pool of interchangeable fixed-size blocks handed out one at a time on
  demand and returned when a request finishes, tables of block references,
  sharing by reference and copy-on-write on divergence ("Paged Attention:
  Virtual Memory for the KV Cache", §The fix…, §Sharing comes almost for free;
  "Paged Attention as a Memory Manager", §How the Kernel Executes Paged
  Attention).  The pages leave the free-list order and tie-breaks open; the
  fixed policy is written out in that module.
* ``cache`` — the byte image of the K and V pools under the library's block
  layout, written token by token through slots and copied block by block.
* ``scenario`` — runs a workload's construction script through the model and
  the cache and returns every integer result and the expected outputs.
* ``accounting`` — the unused fraction of a cache reserved for the longest
  context per request against the last-block slack of blocks taken on demand,
  and the headroom admission test ("Paged Attention as a Memory Manager",
  §The KV-Cache Fragmentation Problem; "Paged Attention: Virtual Memory for the
  KV Cache", §The fix borrowed from operating systems, §What it buys in
  practice).

Every function is pinned by tests in ``tests/test_oracle*.py`` against closed
forms, a library routine (torch's scaled_dot_product_attention in float64),
hand-traced fixtures under ``tests/golden/`` and invariants the pages fix.
"""
from . import accounting, attention, block_manager, cache, scenario  # noqa: F401
from .attention import decode_attention, prefill_attention, split_k, lse_merge, decode_attention_split  # noqa: F401
from .block_manager import BlockManagerModel, OutOfBlocks, InvalidOp  # noqa: F401
from .cache import PagedCacheModel  # noqa: F401
from .scenario import run_scenario, ScenarioResult  # noqa: F401
