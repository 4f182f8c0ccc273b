"""Seeded synthetic decode / prefill-append cases over a packed paged cache.

Every value here is drawn from a seeded ``torch.Generator`` on the device the
case is built on (CPU for small cases, the GPU for large ones), then quantised
once into the bytes that the cache and the query tensors hold:

* e4m3 (OCP E4M3FN, max 448) with one fp32 scale per vector, ``amax / 448``
  (``1.0`` when the vector is all zero), values clamped to +-448 before a
  round-to-nearest-even cast;
* MXFP4: e2m1 codes with one E8M0 scale per group of 32,
  ``2 ** (floor(log2(amax)) - 2)``, nearest e2m1 value with ties to the even
  code, magnitudes above 6 clamped to 6.

Draw order (fixed): block permutation, context lengths, then per layer the
indexer query, head weights and latent query, then per layer the latent cache
and the index keys (planted tokens last).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

from .layout import (CacheLayout, default_layout, D_IDX, H_IDX, D_LAT, D_V, H_Q,
                     MXFP4_GROUP, NV_BLOCK, INDEX_FP8, INDEX_MXFP4, LATENT_FP8, LATENT_NVFP4,
                     latent_record_bytes)

E4M3_MAX = 448.0
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


# --------------------------------------------------------------------------------------
# quantisers (generator side only)
# --------------------------------------------------------------------------------------
def quantize_e4m3_rows(x: torch.Tensor):
    """x float32 [..., D] -> (codes uint8 [..., D], scale float32 [...])."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def quantize_mxfp4_rows(x: torch.Tensor):
    """x float32 [..., D] (D % 32 == 0) -> (packed uint8 [..., D/2], e8m0 uint8 [..., D/32])."""
    shp = x.shape
    g = x.reshape(*shp[:-1], shp[-1] // MXFP4_GROUP, MXFP4_GROUP)
    amax = g.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.clamp(amax, min=1e-30))) - 2,
                    torch.zeros_like(amax)).clamp_(-127, 127)
    y = g / torch.exp2(e).unsqueeze(-1)
    nib = _e2m1_nibbles(y).reshape(*shp[:-1], shp[-1] // 2, 2)
    packed = (nib[..., 0] | (nib[..., 1] << 4)).to(torch.uint8)
    e8 = (e + 127).to(torch.uint8)
    return packed, e8


def _e2m1_nibbles(y: torch.Tensor) -> torch.Tensor:
    """Nearest e2m1 code of every element (ties to the even code, magnitudes above 6
    clamp to 6, no negative zero), int64."""
    mag = y.abs()
    grid = torch.tensor(_E2M1_MAG, dtype=torch.float32, device=y.device)
    mids = (grid[1:] + grid[:-1]) / 2
    i = torch.bucketize(mag.contiguous(), mids)          # mag == mid -> lower index
    on_mid = (i < 7) & (mag == mids[i.clamp(max=6)])
    i = torch.where(on_mid & (i % 2 == 1), i + 1, i)     # ties to the even code
    i = torch.where(mag > 6.0, torch.full_like(i, 7), i)
    sign = ((y < 0) & (i > 0)).to(torch.int64)
    return (sign << 3) | i


def quantize_nvfp4_latent_rows(x: torch.Tensor):
    """x float32 [..., 576] -> (records uint8 [..., 352], scale float32 [...]): s = amax / 448
    (1 when zero), y = x / s clamped to +-448; dims 512.. as e4m3 codes of y; per 16 dims
    of the first 512 an e4m3 block scale nearest to max|y| / 6 and e2m1 codes of y over
    that scale's value (0 when it is 0)."""
    shp = x.shape[:-1]
    amax = x.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / s.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    tail = y[..., D_V:].to(torch.float8_e4m3fn).view(torch.uint8)
    blk = y[..., :D_V].reshape(*shp, D_V // NV_BLOCK, NV_BLOCK)
    sc = (blk.abs().amax(dim=-1) / 6.0).to(torch.float8_e4m3fn)
    scv = sc.to(torch.float32).unsqueeze(-1)
    q = torch.where(scv > 0, blk / torch.where(scv > 0, scv, torch.ones_like(scv)), torch.zeros_like(blk))
    nib = _e2m1_nibbles(q).reshape(*shp, D_V // 2, 2)
    packed = (nib[..., 0] | (nib[..., 1] << 4)).to(torch.uint8)
    return torch.cat([packed, sc.view(torch.uint8), tail], dim=-1), s.to(torch.float32)


# --------------------------------------------------------------------------------------
# case container
# --------------------------------------------------------------------------------------
@dataclass
class DecodeCase:
    name: str
    layout: CacheLayout
    pool: torch.Tensor          # uint8 [num_blocks, row_bytes]
    block_table: torch.Tensor   # int32 [num_seqs, max_blocks]  (-1 = unused)
    row_seq: torch.Tensor       # int32 [R]  block-table row of each query row
    row_ctx: torch.Tensor       # int32 [R]  eligible tokens [0, row_ctx)
    q_idx: torch.Tensor         # uint8 [L, R, 32, 128] (fp8) / [L, R, 32, 64] (mxfp4)
    q_idx_scale: torch.Tensor   # float32 [L, R, 32] (fp8) / uint8 [L, R, 32, 4] (mxfp4 E8M0)
    w: torch.Tensor             # float32 [L, R, 32]
    q_lat: torch.Tensor         # bfloat16 [L, R, 96, 576]
    k: int = 2048
    sm_scale: float = 1.0 / math.sqrt(D_LAT)
    planted: dict = field(default_factory=dict)   # (layer, seq) -> sorted token positions
    seed: int = 0

    @property
    def num_rows(self) -> int:
        return int(self.row_seq.shape[0])

    @property
    def max_ctx(self) -> int:
        return int(self.row_ctx.max().item()) if self.num_rows else 0

    @property
    def num_blocks(self) -> int:
        return int(self.pool.shape[0])

    def to(self, device) -> "DecodeCase":
        mv = lambda t: t.to(device)
        return DecodeCase(self.name, self.layout, mv(self.pool), mv(self.block_table), mv(self.row_seq),
                          mv(self.row_ctx), mv(self.q_idx), mv(self.q_idx_scale), mv(self.w), mv(self.q_lat),
                          self.k, self.sm_scale, dict(self.planted), self.seed)


# --------------------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------------------
def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(g, shape, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _make_queries(g, L, R, index_fmt, device):
    q_idx, q_sc, ws, qls = [], [], [], []
    for _ in range(L):
        qf = _randn(g, (R, H_IDX, D_IDX), device)
        if index_fmt == INDEX_FP8:
            c, s = quantize_e4m3_rows(qf)
        else:
            c, s = quantize_mxfp4_rows(qf)
        w = _randn(g, (R, H_IDX), device) / math.sqrt(H_IDX)
        ql = _randn(g, (R, H_Q, D_LAT), device).to(torch.bfloat16)
        q_idx.append(c); q_sc.append(s); ws.append(w); qls.append(ql)
    return torch.stack(q_idx), torch.stack(q_sc), torch.stack(ws), torch.stack(qls)


def _dequant_query_fp64(codes, scale, index_fmt):
    """Generator-side decode of one query [32, *] used only to aim the planted keys."""
    if index_fmt == INDEX_FP8:
        v = codes.view(torch.float8_e4m3fn).to(torch.float64)
        return v * scale.to(torch.float64).unsqueeze(-1)
    mag = torch.tensor(_E2M1_MAG, dtype=torch.float64, device=codes.device)
    lo = (codes & 0xF).to(torch.int64)
    hi = (codes >> 4).to(torch.int64)
    nib = torch.stack([lo, hi], dim=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    v = mag[nib & 7] * torch.where((nib & 8) > 0, -1.0, 1.0).to(torch.float64)
    sc = torch.exp2(scale.to(torch.float64) - 127).repeat_interleave(MXFP4_GROUP, dim=-1)
    return v * sc


def make_case(ctx_lens, *, row_seq=None, block_size=64, num_layers=1, index_fmt=INDEX_FP8,
              seed=0, device="cpu", k=2048, plant=0, spare_blocks=0, name="case",
              ctx_lens_are_rows=False, latent_fmt=LATENT_FP8) -> DecodeCase:
    """General builder.

    ``ctx_lens``: per-sequence cache lengths (tokens held in the cache). By
    default there is one query row per sequence with ``row_ctx = ctx``. For
    prefill-append pass ``row_seq`` and ``ctx_lens_are_rows=True`` with
    ``ctx_lens`` giving per-row eligible lengths; the cache then holds
    ``max(row ctx)`` tokens per sequence.
    """
    device = torch.device(device)
    g = _gen(seed, device)
    layout = default_layout(block_size, num_layers, index_fmt, latent_fmt=latent_fmt)
    if ctx_lens_are_rows:
        assert row_seq is not None
        row_seq_t = torch.as_tensor(row_seq, dtype=torch.int32)
        row_ctx_t = torch.as_tensor(ctx_lens, dtype=torch.int32)
        S = int(row_seq_t.max().item()) + 1 if len(row_seq_t) else 0
        seq_len = [0] * S
        for s, c in zip(row_seq_t.tolist(), row_ctx_t.tolist()):
            seq_len[s] = max(seq_len[s], c)
    else:
        seq_len = [int(c) for c in ctx_lens]
        S = len(seq_len)
        row_seq_t = torch.arange(S, dtype=torch.int32)
        row_ctx_t = torch.as_tensor(seq_len, dtype=torch.int32)
    nblk = [(c + block_size - 1) // block_size for c in seq_len]
    total = sum(nblk) + spare_blocks
    total = max(total, 1)
    perm = torch.randperm(total, generator=g, device=device).to(torch.int32).cpu()
    maxb = max(nblk) if nblk else 1
    maxb = max(maxb, 1)
    bt = torch.full((max(S, 1), maxb), -1, dtype=torch.int32)
    off = 0
    for s, nb in enumerate(nblk):
        bt[s, :nb] = perm[off:off + nb]
        off += nb
    R = int(row_seq_t.shape[0])
    q_idx, q_sc, w, q_lat = _make_queries(g, num_layers, R, index_fmt, device)

    pool = torch.empty((total, layout.row_bytes), dtype=torch.uint8, device=device)
    if layout.row_bytes > layout.idx_off[-1] + layout.index_page_bytes:
        pool[:, layout.idx_off[-1] + layout.index_page_bytes:] = 0
    bs = block_size
    planted = {}
    chunk = max(1, (1 << 24) // (bs * D_LAT))   # blocks per generation chunk (~64 MB of fp32)
    for l in range(num_layers):
        lo = layout.lat_off[l]
        for b0 in range(0, total, chunk):
            b1 = min(total, b0 + chunk)
            x = _randn(g, (b1 - b0, bs, D_LAT), device)
            rw = latent_record_bytes(latent_fmt)
            if latent_fmt == LATENT_FP8:
                c, s = quantize_e4m3_rows(x)
            else:
                c, s = quantize_nvfp4_latent_rows(x)
            pool[b0:b1, lo:lo + bs * rw] = c.reshape(b1 - b0, bs * rw)
            pool[b0:b1, lo + bs * rw:lo + bs * (rw + 4)] = s.contiguous().view(torch.uint8).reshape(b1 - b0, bs * 4)
        io = layout.idx_off[l]
        kchunk = max(1, (1 << 24) // (bs * D_IDX))
        for b0 in range(0, total, kchunk):
            b1 = min(total, b0 + kchunk)
            x = _randn(g, (b1 - b0, bs, D_IDX), device)
            _write_index(pool, layout, io, b0, b1, x)
        if plant:
            for s_i in range(S):
                pos = _plant_positions(g, seq_len[s_i], plant, device)
                planted[(l, s_i)] = pos
                rows = (row_seq_t == s_i).nonzero().flatten().tolist()
                if not rows:
                    continue
                r0 = rows[0]
                qd = _dequant_query_fp64(q_idx[l, r0].to(device), q_sc[l, r0].to(device), index_fmt)  # [32, 128]
                sig = qd.norm(dim=-1)
                target = 3.0 * sig * torch.sign(w[l, r0].to(torch.float64).to(device))
                gram = qd @ qd.T
                delta = qd.T @ torch.linalg.solve(gram, target)                    # [128]
                pos_t = torch.as_tensor(pos, dtype=torch.int64)
                blk = bt[s_i, (pos_t // bs)].to(torch.int64)
                slot = pos_t % bs
                # regenerate those keys from fresh draws plus the shift, then re-quantise in place
                xk = _randn(g, (len(pos), D_IDX), device) + delta.to(torch.float32).unsqueeze(0)
                _write_index_tokens(pool, layout, io, blk.to(device), slot.to(device), xk)
    return DecodeCase(name, layout, pool, bt.to(device), row_seq_t.to(device), row_ctx_t.to(device),
                      q_idx, q_sc, w, q_lat, k=k, planted=planted, seed=seed)


def _write_index(pool, layout, io, b0, b1, x):
    bs = layout.block_size
    n = b1 - b0
    if layout.index_fmt == INDEX_FP8:
        c, s = quantize_e4m3_rows(x)
        pool[b0:b1, io:io + bs * D_IDX] = c.reshape(n, bs * D_IDX)
        pool[b0:b1, io + bs * D_IDX:io + bs * (D_IDX + 4)] = s.contiguous().view(torch.uint8).reshape(n, bs * 4)
    else:
        c, e = quantize_mxfp4_rows(x)
        hb = D_IDX // 2
        pool[b0:b1, io:io + bs * hb] = c.reshape(n, bs * hb)
        pool[b0:b1, io + bs * hb:io + bs * (hb + 4)] = e.reshape(n, bs * 4)


def _write_index_tokens(pool, layout, io, blk, slot, x):
    bs = layout.block_size
    if layout.index_fmt == INDEX_FP8:
        c, s = quantize_e4m3_rows(x)
        code_off = io + slot * D_IDX
        sc_off = io + bs * D_IDX + slot * 4
        cols = code_off.unsqueeze(1) + torch.arange(D_IDX, device=pool.device)
        pool[blk.unsqueeze(1), cols] = c
        cols = sc_off.unsqueeze(1) + torch.arange(4, device=pool.device)
        pool[blk.unsqueeze(1), cols] = s.contiguous().view(torch.uint8).reshape(-1, 4)
    else:
        c, e = quantize_mxfp4_rows(x)
        hb = D_IDX // 2
        cols = (io + slot * hb).unsqueeze(1) + torch.arange(hb, device=pool.device)
        pool[blk.unsqueeze(1), cols] = c
        cols = (io + bs * hb + slot * 4).unsqueeze(1) + torch.arange(4, device=pool.device)
        pool[blk.unsqueeze(1), cols] = e


def _plant_positions(g, n, count, device):
    """``count`` distinct positions floor(exp(U(0, ln n))) (log-uniform over [1, n))."""
    count = min(count, max(n - 1, 0))
    got, seen = [], set()
    while len(got) < count:
        u = torch.rand((4 * count,), generator=g, device=device, dtype=torch.float64).cpu()
        p = torch.floor(torch.exp(u * math.log(n))).to(torch.int64).clamp_(1, n - 1).tolist()
        for v in p:
            if v not in seen:
                seen.add(v)
                got.append(v)
                if len(got) == count:
                    break
    return sorted(got)


# --------------------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------------------
def make_decode_case(ctx_lens, **kw) -> DecodeCase:
    return make_case(ctx_lens, **kw)


def make_prefill_case(prefix, append, **kw) -> DecodeCase:
    rows = [prefix + r + 1 for r in range(append)]
    return make_case(rows, row_seq=[0] * append, ctx_lens_are_rows=True, **kw)


def config_small(seed=0, device="cpu") -> DecodeCase:
    """Single decode query, 8192-token context, block size 64, one layer, FP8 keys."""
    return make_case([8192], block_size=64, seed=seed, device=device, name="decode_b1_ctx8k")


def config_headline_256k(seed=0, device="cpu", num_layers=24) -> DecodeCase:
    """Single decode query at 262,144 tokens; ``num_layers`` independent layers in one row."""
    return make_case([262144], block_size=64, num_layers=num_layers, seed=seed, device=device,
                     name=f"decode_b1_ctx256k_x{num_layers}layers")


def config_batch16(seed=0, device="cpu") -> DecodeCase:
    """16 decode rows, context lengths uniform on [16384, 65536], pages shuffled in one pool."""
    g = _gen(seed + 1000003, "cpu")
    ctx = torch.randint(16384, 65536 + 1, (16,), generator=g).tolist()
    return make_case(ctx, block_size=64, seed=seed, device=device, name="decode_b16_ctx16k-64k")


def config_long_1m(seed=0, device="cpu", plant=2048) -> DecodeCase:
    """One decode row at 1,048,576 tokens with ``plant`` log-uniformly placed elevated keys."""
    return make_case([1 << 20], block_size=64, seed=seed, device=device, plant=plant,
                     name="decode_b1_ctx1m_planted")


def config_prefill_append(seed=0, device="cpu", prefix=150000, append=2048) -> DecodeCase:
    """``append`` new query rows on a ``prefix``-token cache, causal (row r sees t <= prefix + r)."""
    return make_prefill_case(prefix, append, block_size=64, seed=seed, device=device,
                             name=f"prefill_append_{append}_on_{prefix}")


def config_mixed_mxfp4(seed=0, device="cpu", batch=64, num_layers=24) -> DecodeCase:
    """64 decode rows, log-uniform lengths in [4096, 262144], 24 layers per row, bs 128, MXFP4 keys."""
    g = _gen(seed + 2000003, "cpu")
    u = torch.rand((batch,), generator=g, dtype=torch.float64)
    ctx = torch.floor(torch.exp(math.log(4096) + u * (math.log(262144) - math.log(4096)))).to(torch.int64).tolist()
    return make_case(ctx, block_size=128, num_layers=num_layers, index_fmt=INDEX_MXFP4, seed=seed,
                     device=device, name=f"decode_b{batch}_mxfp4_x{num_layers}layers")
