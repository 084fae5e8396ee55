"""SAS gated block-sparse attention for AMD MI355X (gfx950).

The compute lives in ``libsas.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/sas.h``); this package is its thin Python binding.  The
library is loaded on first use and every entry point raises if it has not
been built - there is no fallback implementation.
"""
from .api import *  # noqa: F401,F403
from .api import __all__  # noqa: F401
