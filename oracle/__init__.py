"""CPU oracle for the FP8 W8A8 block-scaled linear path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, links or calls anything under ``oracle/``; only the
tests, the smoke check and the CPU-baseline leg of the benchmark do.  The
oracle shares no code, table or constant generator with the GPU path.

Every function is written to be checked against the pages by eye: plain
numpy, fp64 where the pages do not fix a precision, fp32 where the method
itself is defined in fp32 (the activation/weight scale and the quotient).

Sources (cited by page title and section):
  * "[vLLM] FP8" (blog.secrett2633.cloud/opensource/vllm/fp8): the block
    quantization rules, the scaling-strategy list and the format table in
    the paper summary.
  * "FP8 Quantization" (zzong2006.github.io): sections B, C, D.1, D.2.
  * "fp8-serving-slower-than-bf16" (hrletsgo.me): hardware-generation and
    arithmetic-intensity sections.
  * "FP8 and FP4: Throughput Needs Scaling" (llm-engineer.pages.dev): the
    E4M3/E5M2 card and the kernel-caveat card.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against printed constants, closed forms, invariants and exact brute force.
No function is "parity unpinned".
"""

from . import e4m3, quant, gemm, tolerance  # noqa: F401
