"""Algorithmic bytes and flops of one decode layer-step: what the method itself
must move or compute, independent of how the kernels are written.

Per query row with context n and top-k k (vLLM "Day-0 support for Kimi K3.1
Pro", section "Sparse attention in K3.1 Pro": the decode step scans every index
key, then reads the full latent of only the kept tokens):
  indexer reads   n * (128 + 4)  bytes of FP8 index keys   (n * 68 for MXFP4)
                  + the query: 32*128 codes + 32 scales + 32 weights
  attention reads min(k, n) * (576 + 4) bytes of FP8 latents (codes + fp32 scale),
                  min(k, n) * (352 + 4) with NVFP4 latent records
                  + the latent query 96*576 bf16
  writes          96*512 fp32 outputs (+ 96 fp32 lse) + k int32 indices
Scores and split partials are implementation traffic and are not counted.
"""
IDX_FP8 = 128 + 4
IDX_MXFP4 = 64 + 4
LAT = 576 + 4
LAT_NVFP4 = 352 + 4
Q_IDX = 32 * 128 + 32 * 4 + 32 * 4
Q_IDX_MX = 32 * 64 + 32 * 4 + 32 * 4
Q_LAT = 96 * 576 * 2
OUT = 96 * 512 * 4 + 96 * 4


def indexer_bytes(ctx: int, index_fmt: str = "fp8") -> int:
    per = IDX_FP8 if index_fmt == "fp8" else IDX_MXFP4
    return ctx * per + (Q_IDX if index_fmt == "fp8" else Q_IDX_MX)


def attention_bytes(ctx: int, k: int, latent_fmt: str = "fp8") -> int:
    per = LAT if latent_fmt == "fp8" else LAT_NVFP4
    return min(k, ctx) * per + Q_LAT + OUT + 4 * k


def layer_step_bytes(ctxs, k: int = 2048, index_fmt: str = "fp8", latent_fmt: str = "fp8") -> int:
    """Bytes for a batch of rows with context lengths ``ctxs``."""
    return sum(indexer_bytes(c, index_fmt) + attention_bytes(c, k, latent_fmt) for c in ctxs)


def indexer_flops(ctxs) -> int:
    """32 heads x 128 dims multiply-adds per (row, token)."""
    return sum(2 * 32 * 128 * c for c in ctxs)


def attention_flops(ctxs, k: int = 2048) -> int:
    """QK^T over 576 dims and PV over 512 dims for 96 heads."""
    return sum(2 * 96 * min(k, c) * (576 + 512) for c in ctxs)
