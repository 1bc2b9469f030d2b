"""DeepSeek Sparse Attention hot path on MI355X (gfx950): Lightning Indexer scores, exact
top-k and sparse/dense absorbed-MLA attention as hand-written HIP kernels behind the C ABI of
libdsa.so (include/dsa.h). This package holds the kernels' sources (csrc/), their build, and a
thin ctypes binding."""
from . import dsa  # noqa: F401
from .dsa import (  # noqa: F401
    DSAError,
    dense_mla_prefill,
    indexer_scores,
    last_path,
    sparse_mla_decode,
    sparse_mla_prefill,
    topk,
)
