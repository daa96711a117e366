"""MI355X (gfx950) query-guided chunk-sparse attention.

The compute path lives in ``libtcsparse.so`` (hand-written HIP kernels behind a C ABI, see
``include/tcsparse.h``); ``top_chunk_sparse_amd.ops`` marshals torch tensors into it.  The
library is loaded on first use and its absence is an error: there is no fallback path.
"""
from .configs import DECODE_CONFIGS, PREFILL_CONFIGS, DecodeConfig, PrefillConfig  # noqa: F401
