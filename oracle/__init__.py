"""fp64 CPU oracle for MLRA / absorbed-MLA decode attention and the GQA comparator.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never does. See ``mlra_oracle`` and
``gqa_oracle`` for the definitions they compute and the passages they follow.
"""
from .mlra_oracle import *  # noqa: F401,F403
from .mlra_oracle import __all__  # noqa: F401
from .gqa_oracle import *  # noqa: F401,F403
from . import gqa_oracle as _g
__all__ = list(__all__) + list(_g.__all__)
