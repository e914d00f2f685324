"""CPU oracle for the differential-attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's ``smoke()`` entry and the ``cpu_baseline`` leg of
``bench.py`` may import anything from here.  The product path (the HIP library and its
Python binding) never imports, calls or links this package, and this package imports
nothing from the product.

Contents
--------
``diffattn_oracle``  plain numpy float64 implementation of the method's definition
``bruteforce``       an independent pure-Python (lists + ``math.exp``) version for tiny inputs
``compare``          the parity metrics and tolerances the tests apply
``diffattn_backward`` float64 gradients of the V1 layout (chain rule on the definition)

Every function here is pinned by ``tests/test_oracle_pins.py`` against values the source
pages print, closed forms, special cases that reduce to library routines and brute force.
The output *values* at the large benchmark shapes are parity unpinned by the pages (they
print none); they are covered only through this pinned oracle.
"""

from .diffattn_oracle import (  # noqa: F401
    lambda_init,
    lambda_value,
    softmax_rows,
    diff_maps,
    diff_core_rows,
    branch_rows,
    rms_norm_rows,
    diff_attn_v1,
    diff_attn_v1_layers,
    diff_attn_v2,
    diff_decode_v2,
    diff_decode_v1,
)
from .diffattn_backward import diff_attn_v1_backward  # noqa: F401,E402
