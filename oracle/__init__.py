"""CPU oracle for the KronQ per-layer quantization path (test infrastructure).

This package is test infrastructure, not part of the product. Only the test
suite, the smoke check of the build entry point and the CPU-baseline leg of
the benchmark may import it. It shares no code with the GPU library or its
Python binding: it reads only the seeded inputs from ``kq_synth``.
"""
from .kronq import *  # noqa: F401,F403
