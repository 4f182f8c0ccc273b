"""DSA decode over a packed paged cache on MI355X (gfx950): HIP kernels behind a C ABI.

The Python functions are a thin ctypes layer over libdsa.so (include/dsa.h):
dsa_indexer_score, dsa_topk, dsa_sparse_mla, dsa_decode_step (each decode-step and
indexer call takes an optional rows_per_seq), dsa_cache_append, and dsa_topk_dcp (the
exact top-k merge of decode context parallelism, emulated over token-strided shards);
dsa_device_status reads the per-device word in which kernels report repaired bad data;
dsa_decode_step_noalloc runs the decode step on the library's static per-GPU scratch.
"""
from .binding import (  # noqa: F401
    DSAError, CacheDesc, load_library, make_cache_desc, decode_scores_view, EXPORTED, LIB_PATH,
    dsa_abi_version, dsa_status_string, dsa_workspace_bytes, dsa_decode_scores_ld,
    dsa_indexer_score, dsa_topk, dsa_sparse_mla, dsa_decode_step, dsa_cache_append,
    dsa_topk_dcp, dcp_send_count, dsa_device_status, dsa_hbm_read_probe, dsa_decode_step_noalloc,
    DSA_STATIC_SCRATCH_BYTES, dsa_decode_step_stages, DSA_STAGE_INDEXER, DSA_STAGE_TOPK, DSA_STAGE_ATTENTION,
    DSA_STAGE_MERGE, DSA_STAGE_ALL,
    DSA_DEV_CTX_CLAMPED, DSA_DEV_BLOCK_CLAMPED, DSA_DEV_INDEX_RANGE,
    DSA_INDEX_FP8, DSA_INDEX_MXFP4, DSA_LATENT_FP8, DSA_LATENT_NVFP4, DSA_OP_TOPK, DSA_OP_SPARSE_MLA, DSA_OP_DECODE_STEP,
)
from . import accounting  # noqa: F401
