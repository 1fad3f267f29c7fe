"""fp64 CPU oracle for masked attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg call it.  It
shares no code with the GPU path (no kernels, headers, helpers or tables); the
only common module is ``synthetic`` (seeded inputs and mask parameters).

Sources, cited by page title and section:

* "Long-Context Attention Benchmark" review (xllm-io), section 3 "mask
  taxonomy": the fourteen mask families (names only; the readings used are
  listed in ``oracle.masks``).
* "FlashAttention vs. RingAttention" (dtcms), FlashAttention-1 "problem and
  bottleneck": the definition softmax(Q K^T / sqrt(d_k)) V; FlashAttention-2
  "core optimisations": one merged softmax statistic (the log-sum-exp) and the
  dQ dependency dQ_i = sum_j dS_ij K_j.

Modules:
  masks       vectorised mask predicates, one per family (numpy)
  attention   fp64 forward / backward materialising full score rows
  bruteforce  pure-Python loops with math.fsum, for tiny cases (a second,
              independent implementation used to pin the two above)
"""
from . import masks, attention, bruteforce  # noqa: F401
