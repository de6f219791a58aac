"""CPU float64 oracle for GQA / GQE (test infrastructure only).

Imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg; the HIP library and its Python binding never import it.
"""
from .gqa_oracle import *  # noqa: F401,F403
from .gqa_oracle import __all__  # noqa: F401
