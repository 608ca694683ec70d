"""Oracle for the Compass/Cohere2 parallel decoder layer.

TEST INFRASTRUCTURE ONLY: plain float64 (numpy) definitions used to check the
HIP library. Only tests, the smoke check and the bench's CPU-baseline leg may
import this package; the product path never does.
"""
from . import compass_oracle  # noqa: F401
