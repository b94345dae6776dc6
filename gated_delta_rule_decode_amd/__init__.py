"""MI355X-native KDA (Kimi Delta Attention) decode.

The decode step runs in hand-written gfx950 HIP kernels behind the C ABI of
``libkda_mi355x.so`` (see include/kda.h); this package is its thin Python
binding.  PyTorch supplies device memory and streams only.
"""
from .api import (PackedFusedWorkspace, PreparedCall, fused_kda_decode, packed_fused_kda_decode,  # noqa: F401
                  packed_fused_kda_decode_noalloc, packed_kda_decode, prepare, recurrent_kda)
from ._lib import KDAError, load as load_library  # noqa: F401

__all__ = ["recurrent_kda", "packed_kda_decode", "fused_kda_decode", "packed_fused_kda_decode",
           "packed_fused_kda_decode_noalloc", "PackedFusedWorkspace", "prepare", "PreparedCall", "KDAError", "load_library"]
