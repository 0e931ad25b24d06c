"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This package holds no step of the compression method: it only draws correlated,
outlier-heavy key/value vectors, queries and attention-mass profiles with the
shapes of the workloads the method is measured on.  Both the HIP library and the
oracle receive these arrays as plain inputs.
"""
from .kv import *  # noqa: F401,F403
from .configs import CONFIGS, Config  # noqa: F401
