"""Plain fp64 CPU oracle for the head-scale KV-pruning hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
or its Python binding; the one thing both sides take from elsewhere is the
seeded input data (``workloads``), which holds none of the method's
arithmetic.

Sources (the web pages the method is described on):
  * HeatKV project page, "HeatKV: Head-tuned KV-cache Compression for Visual
    Autoregressive Modeling" (arm-research.github.io/heatkv): Abstract,
    Method steps 1-5, Results (Table 1 excerpt).
  * Pith review page of arXiv 2605.14877 (the same paper): captions of
    Figures 2-4 and the Appendix A signature of Algorithm 2.

Modules:
  numerics   bf16 bit patterns -> fp64 values
  attention  block-causal multi-scale attention over kept segments; S-CAS
  schedule   S-CAS table + budget -> static keep-mask (per-scale orderings,
             shared prefix, sink scales kept)
  cache      ragged cache layout, expected compacted contents, cache-size
             accounting
  calibration  streamed S-CAS over many batches; ranking stability between
             two calibration subsets
  progressive  growing pruning sets (lazy prefix lengths N_k), cache size
             after every layer, expiry steps and the cache contents they imply
  policies   condensed + local scale-window schedule (a second generator of
             expiry steps)
  quant      (scale-block, channel) group-wise 4-bit storage of the cache and
             attention over the dequantized segments

Every function is written for readability, not speed.  Where the pages leave
a step open, the reading taken is stated in the function's docstring.
"""
from . import numerics, attention, schedule, cache, calibration, progressive, policies, quant  # noqa: F401
