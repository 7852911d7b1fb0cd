"""MI355X (gfx950) Video DeltaNet hybrid video-to-video attention layer.

The layer runs in hand-written HIP kernels behind the C ABI ``include/vdn.h``
(``libvdn.so`` in this directory); ``binding`` is its thin Python interface.
"""
from .binding import (VdnError, hybrid_attn, softmax_fwd, vda_gram, vda_factor_scan, merge,
                      make_layout, workspace_size, validate_layout, num_chunks, version)

__all__ = ["VdnError", "hybrid_attn", "softmax_fwd", "vda_gram", "vda_factor_scan", "merge",
           "make_layout", "workspace_size", "validate_layout", "num_chunks", "version"]
