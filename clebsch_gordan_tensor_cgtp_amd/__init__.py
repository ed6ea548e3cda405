"""MI355X-native Clebsch-Gordan tensor-product (CGTP) convolution.

The compute path is libcgtp.so (HIP kernels for gfx950 behind the C ABI in
include/cgtp.h); ``Plan`` in ``ops`` is its thin torch-facing binding.  The
library is loaded on first use of ``Plan`` and its absence raises.
"""


def __getattr__(name):
    if name in ("Plan",):
        from .ops import Plan
        return Plan
    raise AttributeError(name)
