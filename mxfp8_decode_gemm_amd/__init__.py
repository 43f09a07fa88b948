"""MI355X (gfx950) low-batch MXFP8 publishing GEMM with a Lamport mailbox.

The product is the HIP library ``lib/libmxgemm.so`` (sources in ``csrc/``, C
ABI in ``include/mxgemm.h``); ``binding`` is its thin ctypes binding and
``build`` compiles it. Importing the package itself loads nothing, so that
the build can run first; ``from mxfp8_decode_gemm_amd import binding`` loads
the library and raises if it is missing.
"""

__all__ = ["binding", "build"]
