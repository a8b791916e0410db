"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds no arithmetic of the quantization method or the GEMM: it only draws
random numbers and rounds them to the bf16 input dtype.
"""

from .synth import *  # noqa: F401,F403
