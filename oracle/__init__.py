"""CPU fp64 oracle for MLA absorbed decode -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and this package imports nothing
from the product path.
"""
from .mla_oracle import *  # noqa: F401,F403
