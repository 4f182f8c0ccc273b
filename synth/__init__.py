"""Seeded synthetic inputs for the DSA decode path.

This package builds the bytes both sides read: a packed paged cache, block
tables, per-row context lengths and the quantised query tensors. It holds
none of the method's arithmetic (no scoring, selection or attention); its only
numerics are the random draws and the quantisation that turns them into cache
bytes, which happens here exactly once.
"""
from .layout import (CacheLayout, default_layout, D_IDX, H_IDX, D_LAT, D_V, H_Q, MXFP4_GROUP,
                     LATENT_FP8, LATENT_NVFP4)
from .cases import (DecodeCase, make_case, make_decode_case, make_prefill_case,
                    config_small, config_batch16, config_long_1m, config_prefill_append,
                    config_mixed_mxfp4, config_headline_256k)

__all__ = [
    "CacheLayout", "default_layout", "D_IDX", "H_IDX", "D_LAT", "D_V", "H_Q", "MXFP4_GROUP",
    "LATENT_FP8", "LATENT_NVFP4",
    "DecodeCase", "make_case", "make_decode_case", "make_prefill_case",
    "config_small", "config_batch16", "config_long_1m", "config_prefill_append",
    "config_mixed_mxfp4", "config_headline_256k",
]
