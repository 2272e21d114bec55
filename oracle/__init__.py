"""CPU oracle package — test infrastructure only (tests, smoke check, benchmark CPU baseline).

The product path never imports it.  See ``oracle.mxfp4_moe``.
"""
from . import mxfp4_moe  # noqa: F401
