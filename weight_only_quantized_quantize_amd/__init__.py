"""Weight-only quantised decode linears (INT8 per-tensor and outlier-aware INT4)
for AMD MI355X: hand-written HIP kernels for gfx950 behind a C ABI (libwoq.so),
with this package as its thin Python binding."""
from . import woq  # noqa: F401
