"""MI355X (gfx950) AirCache visual KV-cache compression pass.

The pass runs in hand-written HIP kernels behind a C ABI (include/aircache.h);
this package holds the HIP sources, their build script and a thin binding that
uses PyTorch only for device memory and streams.
"""
from .api import AirCache, PlanOutputs, make_desc  # noqa: F401
