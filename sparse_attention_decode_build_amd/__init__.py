"""MI355X-native sparse-attention decode step (DeepSeek-V4 style).

The hot path lives in libsad.so (HIP kernels for gfx950, C ABI in include/sad.h);
this package holds its ctypes binding, its build script and the seeded synthetic
workloads used by the benchmark.
"""

from ._lib import (  # noqa: F401
    KV_SCALE_F32,
    KV_SCALE_UE8M0,
    IndexerCache,
    KvCache,
    build_sparse_indices,
    gather_dequant_kv,
    indexer_score_topk,
    prepare_indexer_q_mxfp4,
    indexer_score_topk_workspace_size,
    indexer_topk_sparse_indices,
    insert_index_keys,
    insert_kv_rows,
    inv_rope_fp8_quant,
    last_error,
    load,
    sparse_mla_decode,
    sparse_mla_decode_workspace_size,
    sparse_mla_decode_noalloc,
)
