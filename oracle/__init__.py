"""CPU oracle of the R-KV compression step — TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP product path never imports or calls it.
"""
from . import rkv_oracle, brute  # noqa: F401
