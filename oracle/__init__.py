"""CPU oracle for the AlexNet forward pass and training step -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  It is a plain, slow, obviously-correct implementation: the
per-layer arithmetic lives in ``alexnet_oracle.cpp`` (direct loops, float64),
and ``alexnet.py`` composes those layers in the order the pages give.  It
shares no code with the HIP library and never calls it.

Parity status: every function is pinned by a CPU test in tests/test_oracle_*.py.
The Philox4x32-10 generator and the dropout-mask rule are pinned word for word
against PyTorch's independent source-level engine (tests/test_oracle_philox.py).
"""
from .lib import *  # noqa: F401,F403
from . import alexnet  # noqa: F401
