"""KDA chunked forward on AMD Instinct MI355X (gfx950).

The compute path is libkda.so (hand-written HIP kernels behind a C ABI,
declared in include/kda.h); this package only marshals torch tensors into
that ABI.  The library is loaded on first use, and a missing library is an
error, never a fallback.
"""

from .api import chunk_bwd, chunk_fwd, chunk_fwd_noalloc, decode, decode_stats, gate_prefix, workspace_bytes  # noqa: E402,F401
from ._lib import KdaError, HipEvent  # noqa: E402,F401
