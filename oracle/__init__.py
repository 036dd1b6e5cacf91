"""CPU oracle for Kara's decode-time KV-cache compression step.

TEST INFRASTRUCTURE ONLY.  This package is the independent, plain and slow
definition that the HIP path is checked against.  Only the test suite, the
smoke check in ``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``decode_kv_cache_kara_amd``)
never imports, calls or links anything here, and nothing here imports the
product path: the two share no code.

Sources (cited by page title and section):

* "Technical Summary: Kara - Sliding-Window KV Cache Compression for Efficient
  Serving of Reasoning LLMs" (gist.science), section "Methodology: Kara",
  items 1-3.  Cited below as [Summary, Methodology n].
* "Kara - Sliding-Window KV Cache Compression for Efficient Serving of
  Reasoning LLMs under Memory Constraints" (the paper's front matter as shown
  by docshare.wps.com): Abstract, section 1 Introduction, Fig. 1 and Fig. 2
  captions.  Cited below as [Paper, ...].

Every floating-point step runs in float64 unless a function states that it
reproduces a float32 decision rule.  Functions whose result has no pin other
than this module's own reading of the pages are marked "parity unpinned".
"""

from .kara_oracle import (  # noqa: F401
    window_scores,
    topk_candidates,
    token2chunk,
    select_retained,
    FifoPool,
    plan_compaction,
    apply_compaction,
    window_keys,
    compress,
    logical_tokens,
    schedule_step,
)
