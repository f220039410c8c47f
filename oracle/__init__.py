"""Plain, slow fp64 CPU oracle for the sparse paged decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import or run it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or constants) and never imports it.

Pages cited in this package:

* [P1] "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
  Hierarchy" (thelatestinai.com/papers/2610.13708) -- the card whose abstract
  describes MOIRA: the coverage rule and self-planning attention.
* [P2] "HiSparse: Scaling Sparse Attention Decoding with Hierarchical KV Cache"
  (scholarbro.com/p/47450) -- abstract: host-resident KV with a fixed-size GPU
  cache, LRU replacement, outputs unchanged by placement.
* [P3] "Unifying Sparse Attention with Hierarchical Memory for Scalable
  Long-Context LLM Serving" (thelatestinai.com/papers/2604.26837) -- SPIN
  abstract and the RaBitQCache card (adaptive top-p retrieval).
"""

from .sparse_oracle import (  # noqa: F401
    PAGE,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    summaries,
    bound,
    page_logits,
    head_mass,
    group_mass,
    coverage_cut,
    topk_cut,
    select_unit,
    attend_tokens,
    attend_pages,
    merge_partials,
    dense_unit,
    list_accepted,
)
from .lru import (LRUState, pooled_unit, resolve_pooled_step, resolve_step,  # noqa: F401
                  textbook_bucketed_trace, textbook_lru_trace)
