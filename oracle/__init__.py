"""CPU oracle for the DeepSeek Sparse Attention hot path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package. The GPU library never loads it and shares no code with it.
"""
from .ref import (  # noqa: F401
    E4M3,
    F32,
    build_oracle,
    e4m3_to_double,
    bf16_to_double,
    indexer_scores,
    topk,
    sparse_mla,
    dense_mla,
    mha,
    e4m3_from_float,
    e4m3_quantize,
    indexer_cache_write,
    latent_cache_write,
    indexer_key_project,
    indexer_query_project,
)
