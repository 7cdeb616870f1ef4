"""CPU oracle package -- TEST INFRASTRUCTURE ONLY (see nf4_oracle's header).

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from . import nf4_oracle  # noqa: F401
