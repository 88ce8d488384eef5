"""Oracle for the split-K decode GEMM: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the HIP
path (``split_reduction_amd``), and neither side imports the other.

What it computes (the pages are the vLLM API documentation pages listed below):

* ``formats``: the number formats the path reads and writes -- bf16 with
  round-to-nearest-even, OCP E4M3FN, E2M1 and E8M0 (MXFP4), and MXFP8 (E4M3
  elements with E8M0 block scales), each written from the format's own
  definition, not from a bit trick.
* ``gemm``: the plain fp64 definition ``C[t, n] = sum_k X[t, k] * W[n, k]`` and
  its MXFP4 and MXFP8 forms on decoded weights, a pure-Python brute force for tiny shapes,
  the acceptance bound, and the fixed-order fp32 butterfly of a wave reduction.

Pages cited in this package:

* ``vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk``
  (the split-K GEMM ``SplitKGemm``),
* ``vllm.models.muse_spark.amd.mono.kernels.dev`` (MXFP4 decode, bf16 pairs),
* ``vllm.models.deepseek_v41.amd.mono.common.ops`` (E4M3 packing, butterflies).

Every function here is pinned by ``tests/test_oracle_*.py`` to something other
than itself (closed forms, exhaustive tables, library routines, brute force,
hand-worked fixtures under ``tests/golden/``).
"""

from . import formats, gemm  # noqa: F401
