"""CPU oracle for the Hybrid HiSparse sparse-MLA decode step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the GPU path is checked against.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does, and it shares no code with the HIP library (its only common input
is the seeded generator in ``synth``).

Everything is numpy in float64.  Each function states the passage of the
pages it follows:

* "Hybrid HiSparse for GLM 5.3" (Part 1), sections "Using sparsity when it is
  needed" (indexer top-K, HiSparse offload, IndexShare) and "How it works"
  (three residency states, fused top-K resolver, one pool and one tensor,
  HMA row ids gathered with a single stride).
* Part 2 (PCP/DCP/P-D for GLM-5.3), section "Why not TP or DP?" (the indexer
  scores every earlier token and keeps 2,048; 64 heads share the latent),
  the "Try it" section (short prompts stay on the sparse-MLA MQA kernel),
  and footnote 1 (656-byte FP8 rows; QK over 576 dims, PV over 512).
* Part 1, "How it works", the paragraphs after the three residency states: the
  write side of the host pool (completed pages copied to host memory, then
  giving up their GPU blocks without a second copy), and hot pages leased from
  the shared block pool and given back.
* Part 1, "Composing with the rest of vLLM": per-step resolver plans that can
  be replayed and share the request's hot state (speculative decoding).

Where the pages are silent the reading taken is stated at the function.
Parity status: every function below is pinned by tests under
``tests/test_oracle_*.py`` (closed forms, invariants, brute force, library
special cases).  Absolute attention and score values at full scale have no
worked example on the pages; those are pinned only through the checks listed
in the tests.
"""
from .hisparse_oracle import (  # noqa: F401
    BLOCK,
    HotPool,
    HotState,
    attention,
    bf16_decode,
    decode_latent_rows,
    dequant_idx_keys,
    e4m3_decode,
    E4M3_VALUES,
    indexer_scores,
    materialize_pages,
    release_hot,
    release_pages,
    resolve,
    topk_select,
)
