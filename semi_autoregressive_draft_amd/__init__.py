"""DSpark semi-autoregressive draft-proposal hot path for AMD Instinct MI355X.

The compute lives in libdspark.so (hand-written gfx950 HIP kernels behind a C
ABI declared in include/dspark.h); ``binding`` exposes its entry points under
the same names, and ``path.DraftPath`` sequences them for one batch of blocks.
"""
from . import binding  # noqa: F401

__version__ = "0.1.0"
