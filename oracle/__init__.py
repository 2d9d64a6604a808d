"""CPU oracle for the MXFP8 training hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (``quantize_grouped_gemm_amd``) never imports, links or runs
it, and this package imports nothing from the product path.

Everything here is plain numpy evaluated in float64 (exact where the method
is exact), written from the definitions so that it can be checked by eye.
"""

from .mx import *  # noqa: F401,F403
