"""Seeded synthetic workloads for paged single-token decode attention.

This package is the one piece of code shared by the fp64 oracle side (tests,
CPU baseline) and the HIP side (tests, benchmark).  It draws inputs only:
context lengths, the physical-page permutation, q/K/V values and their
storage encodings.  It holds none of the attention arithmetic.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .make import Case, make_case, logical_kv  # noqa: F401
