"""MI355X-native ring attention: one device's share of context-parallel attention.

The hot path lives in libra.so (hand-written gfx950 HIP kernels behind the C ABI
of include/ra.h); this package is its ctypes binding (``_lib``), the host-side
ring driver (``ring``), rank layouts (``layout``), workloads (``configs``) and
work accounting (``sizing``).
"""

from . import configs, layout, sizing  # noqa: F401
from ._lib import (  # noqa: F401
    RaError,
    load,
    ra_factored_spatial,
    ra_factored_temporal,
    ra_finalize,
    ra_kv_pass,
    ra_merge_lse,
    ra_step,
)

__version__ = "0.1.0"
