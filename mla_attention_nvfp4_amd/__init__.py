"""NVFP4 MLA attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmla_nvfp4.so`` (C ABI in
``include/mla_nvfp4.h``); ``ops`` re-exports its thin Python binding.  The
library is loaded on first use, and every call fails loudly if it is not
built.
"""
from . import _lib as ops  # noqa: F401
from ._lib import MlaError  # noqa: F401
