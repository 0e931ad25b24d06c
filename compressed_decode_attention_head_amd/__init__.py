"""MI355X-native transform-coded KV cache with compressed-domain decode attention.

The compute lives in libaatc.so (include/aatc.h): a C++ host solver for calibration and
HIP kernels for gfx950 for encode, decode (reconstruct) and decode attention.  Importing
this package does not load the library; the first call does, and it fails loudly when the
library has not been built.
"""
from .api import (AatcError, CompressedKVCache, bits_budget, calib_view, calibrate, packed_bytes,  # noqa: F401
                  v_tiles, validate)
