"""libecho: Echo's error-compensated low-bit all-reduce hot path on MI355X.

The arithmetic runs in hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/echo.h`` (``libecho.so``).  ``error_feedback_quant_amd.echo``
is the thin ctypes binding with the same call names; importing it loads the
library and raises if it is missing.  ``error_feedback_quant_amd.inputs`` holds the
seeded synthetic workloads.  Importing this package itself loads nothing.
"""
