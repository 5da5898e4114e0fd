"""CPU oracle for the W8A8 INT8 linear layer (test infrastructure only).

Imported only by tests/, the package smoke check and the benchmark's
CPU-baseline leg. The GPU library never imports or calls anything here.
"""
from .w8a8_oracle import *  # noqa: F401,F403
from . import w8a8_oracle  # noqa: F401
