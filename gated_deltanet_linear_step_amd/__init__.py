"""MI355X (gfx950) gated delta-rule step: HIP kernels behind a C ABI (libgdn.so).

The ops live in ``gated_deltanet_linear_step_amd.ops`` (a thin ctypes binding over
the C ABI in ``include/gdn.h``); importing this package does not load the
library -- the first op call does, and it raises if the library is missing.
"""
