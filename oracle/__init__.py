"""fp64 CPU oracle for MLRA / absorbed-MLA decode attention.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never does. See ``mlra_oracle`` for the
definition it computes and the passages it follows.
"""
from .mlra_oracle import *  # noqa: F401,F403
from .mlra_oracle import __all__  # noqa: F401
