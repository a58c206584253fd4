"""Window-tiered KV-cache decode path for MI355X (gfx950).

The compute lives in the HIP library ``_lib/libkvtier.so`` (C ABI:
include/kvtier.h); :mod:`tiered_int2_fp16_amd.binding` marshals torch tensors
into it.  Importing the binding fails if the library has not been built.
"""
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libkvtier.so")
