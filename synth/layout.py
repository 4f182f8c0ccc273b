"""Byte layout of one packed cache block row.

A block row is one contiguous range of memory holding, for every DSA layer,
that layer's latent page and index-key page for the ``block_size`` token slots
of the block (vLLM "Day-0 support for Kimi K3.1 Pro", section on the KV cache
that serves three kinds of state: one row per block, pages of different sizes
inside a row, power-of-two block size).

Inside a row, layer ``l`` owns two pages:

* latent page at ``lat_off[l]``: ``block_size`` token records, then ``block_size``
  little-endian fp32 per-token scales. A record is
  - FP8:   576 e4m3 codes (slot ``s`` at ``s * 576``);
  - NVFP4: 352 bytes (the width the page quotes for NVFP4 latents): 256 bytes of
    packed e2m1 pairs for dims 0..511 (element ``2i`` in the low nibble of byte
    ``i``), 32 e4m3 block scales (one per 16 dims), 64 e4m3 codes for dims 512..575.
* index page at ``idx_off[l]``:
  - FP8:   ``block_size * 128`` bytes of e4m3 codes, then ``block_size`` fp32 scales
    (128 + 4 = 132 bytes per token, the width the page quotes for FP8 index keys);
  - MXFP4: ``block_size * 64`` bytes of packed e2m1 pairs (element ``2i`` in the
    low nibble of byte ``i``), then ``block_size * 4`` E8M0 bytes, one per group
    of 32 elements (64 + 4 = 68 bytes per token).

Codes come before scales (structure of arrays) so that every 576-, 128- or
64-byte code vector starts on a 16-byte boundary.
"""
from dataclasses import dataclass, field, asdict

D_IDX = 128       # indexer head dimension
H_IDX = 32        # indexer heads
D_LAT = 576       # MLA latent width (keys use all of it)
D_V = 512         # value width (first 512 latent dims)
H_Q = 96          # latent-query heads
MXFP4_GROUP = 32  # elements per E8M0 scale

NV_BLOCK = 16     # dims per NVFP4 block scale

INDEX_FP8 = "fp8"
INDEX_MXFP4 = "mxfp4"
LATENT_FP8 = "fp8"
LATENT_NVFP4 = "nvfp4"


def index_token_bytes(index_fmt: str) -> int:
    return D_IDX + 4 if index_fmt == INDEX_FP8 else D_IDX // 2 + D_IDX // MXFP4_GROUP


def latent_record_bytes(latent_fmt: str = LATENT_FP8) -> int:
    return D_LAT if latent_fmt == LATENT_FP8 else D_V // 2 + D_V // NV_BLOCK + (D_LAT - D_V)


def latent_token_bytes(latent_fmt: str = LATENT_FP8) -> int:
    return latent_record_bytes(latent_fmt) + 4


@dataclass(frozen=True)
class CacheLayout:
    block_size: int
    num_layers: int
    index_fmt: str
    row_bytes: int
    lat_off: tuple = field(default_factory=tuple)
    idx_off: tuple = field(default_factory=tuple)
    latent_fmt: str = LATENT_FP8

    @property
    def latent_page_bytes(self) -> int:
        return self.block_size * latent_token_bytes(self.latent_fmt)

    @property
    def index_page_bytes(self) -> int:
        return self.block_size * index_token_bytes(self.index_fmt)

    def as_dict(self) -> dict:
        d = asdict(self)
        d["lat_off"] = list(self.lat_off)
        d["idx_off"] = list(self.idx_off)
        return d


def default_layout(block_size: int, num_layers: int = 1, index_fmt: str = INDEX_FP8,
                   row_pad: int = 0, latent_fmt: str = LATENT_FP8) -> CacheLayout:
    """Layer-major row: [lat_0 | idx_0 | lat_1 | idx_1 | ...] (+ optional tail pad)."""
    if block_size <= 0 or block_size & (block_size - 1):
        raise ValueError("block_size must be a power of two")
    if index_fmt not in (INDEX_FP8, INDEX_MXFP4):
        raise ValueError(index_fmt)
    if latent_fmt not in (LATENT_FP8, LATENT_NVFP4):
        raise ValueError(latent_fmt)
    lat, idx, off = [], [], 0
    lp = block_size * latent_token_bytes(latent_fmt)
    ip = block_size * index_token_bytes(index_fmt)
    for _ in range(num_layers):
        lat.append(off)
        off += lp
        idx.append(off)
        off += ip
    off += row_pad
    off = (off + 15) // 16 * 16
    return CacheLayout(block_size, num_layers, index_fmt, off, tuple(lat), tuple(idx), latent_fmt)
