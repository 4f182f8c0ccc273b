"""Plain CPU oracle for DSA decode over a packed paged cache.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library or its Python binding, and it never imports either.

What it computes follows vLLM "Day-0 support for Kimi K3.1 Pro", section
"Sparse attention in K3.1 Pro" (an indexer scores every earlier token with 32
light heads, the 2,048 best are kept, and MLA attention runs exactly over only
those), together with the fixed definitions the method is graded by:

* indexer score   s_t = sum_h w_h * ReLU(q_h . k_t)        (32 heads x 128 dims)
* selection       the min(k, n) largest s_t, equal scores -> lower token index,
                  compared in fp32 (the precision the GPU kernel decides in)
* attention       softmax_t((q . c_t) / sqrt(576)) weighted sum of c_t[:512],
                  per latent-query head, plus the natural-log LSE.

Every floating-point step runs in float64 from exactly dequantised values
(e4m3 / e2m1 codes times their fp32 / E8M0 scales). There is no blocking,
fusion or reordering beyond a chunked matrix product over tokens.
"""
from __future__ import annotations

import math
import numpy as np

H_IDX = 32
D_IDX = 128
H_Q = 96
D_LAT = 576
D_V = 512
MX_GROUP = 32

# ---------------------------------------------------------------------------
# Dequantisation tables, written out from the format definitions.
# ---------------------------------------------------------------------------

def e4m3fn_value(code: int) -> float:
    """OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
    S.1111.111 is NaN; exponent 0 encodes subnormals m/8 * 2^-6. Max 448.
    (The cache's FP8 latent and index keys, page 1, KV-cache section.)"""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e8m0_value(code: int) -> float:
    """E8M0 shared scale of the MX formats: 2^(code - 127); 0xFF is NaN."""
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


def e2m1_value(nibble: int) -> float:
    """E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is
    subnormal m * 0.5. Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}."""
    sign = -1.0 if nibble & 0x8 else 1.0
    e = (nibble >> 1) & 0x3
    m = nibble & 0x1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


E4M3_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(n) for n in range(16)], dtype=np.float64)


def _f32_from_bytes(b: np.ndarray) -> np.ndarray:
    """Little-endian fp32 from a [..., 4] uint8 array."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return b.view("<f4").reshape(b.shape[:-1]).astype(np.float64)


# ---------------------------------------------------------------------------
# Page walk over the packed cache (page 1: a block is one contiguous row that
# holds every DSA layer's latent page and index-key page; the block table plus
# the slot give the page address of a token).
# ---------------------------------------------------------------------------

class Layout:
    """Plain view of the row layout numbers: block_size, index_fmt, latent_fmt
    ("fp8" when absent), row_bytes, lat_off[layer], idx_off[layer]. Accepts any
    object or dict carrying them."""

    def __init__(self, src):
        get = (lambda k: src[k]) if isinstance(src, dict) else (lambda k: getattr(src, k))
        has = (lambda k: k in src) if isinstance(src, dict) else (lambda k: hasattr(src, k))
        self.block_size = int(get("block_size"))
        self.index_fmt = str(get("index_fmt"))
        self.latent_fmt = str(get("latent_fmt")) if has("latent_fmt") else "fp8"
        self.row_bytes = int(get("row_bytes"))
        self.lat_off = [int(v) for v in get("lat_off")]
        self.idx_off = [int(v) for v in get("idx_off")]


def token_pages(bt_row: np.ndarray, tokens: np.ndarray, block_size: int):
    """Token t lives in physical block bt_row[t // block_size], slot t % block_size."""
    tokens = np.asarray(tokens, dtype=np.int64)
    blk = np.asarray(bt_row, dtype=np.int64)[tokens // block_size]
    slot = tokens % block_size
    return blk, slot


def read_index_keys(pool: np.ndarray, lay: Layout, layer: int, bt_row, tokens) -> np.ndarray:
    """Dequantised index keys [n, 128] (float64) for the given token positions."""
    pool = pool.reshape(-1, lay.row_bytes)
    blk, slot = token_pages(bt_row, tokens, lay.block_size)
    base = lay.idx_off[layer]
    bs = lay.block_size
    if lay.index_fmt == "fp8":
        codes = pool[blk[:, None], base + slot[:, None] * D_IDX + np.arange(D_IDX)]
        sc = _f32_from_bytes(pool[blk[:, None], base + bs * D_IDX + slot[:, None] * 4 + np.arange(4)])
        return E4M3_TABLE[codes] * sc[:, None]
    if lay.index_fmt == "mxfp4":
        half = D_IDX // 2
        packed = pool[blk[:, None], base + slot[:, None] * half + np.arange(half)]
        e8 = pool[blk[:, None], base + bs * half + slot[:, None] * 4 + np.arange(4)]
        return mxfp4_decode(packed, e8)
    raise ValueError(lay.index_fmt)


def mxfp4_decode(packed: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """[..., 64] packed e2m1 (element 2i in the low nibble of byte i) and
    [..., 4] E8M0 (one per 32 elements) -> float64 [..., 128]."""
    lo = packed & 0xF
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    vals = E2M1_TABLE[nib]
    scale = np.repeat(E8M0_TABLE[e8], MX_GROUP, axis=-1)
    return vals * scale


def read_latents(pool: np.ndarray, lay: Layout, layer: int, bt_row, tokens) -> np.ndarray:
    """Dequantised latents c_t [n, 576] (float64): the record's values times the
    token's fp32 scale (FP8: 576 e4m3 codes; NVFP4: see nvfp4_latent_decode)."""
    pool = pool.reshape(-1, lay.row_bytes)
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size == 0:
        return np.zeros((0, D_LAT))
    blk, slot = token_pages(bt_row, tokens, lay.block_size)
    base = lay.lat_off[layer]
    w = latent_record_bytes(lay.latent_fmt)
    rec = pool[blk[:, None], base + slot[:, None] * w + np.arange(w)]
    sc = _f32_from_bytes(pool[blk[:, None], base + lay.block_size * w + slot[:, None] * 4 + np.arange(4)])
    vals = E4M3_TABLE[rec] if lay.latent_fmt == "fp8" else nvfp4_latent_decode(rec)
    return vals * sc[:, None]


# ---------------------------------------------------------------------------
# NVFP4 latent records (page 1, KV-cache section: a token's MLA latent takes 576
# bytes in FP8 and 352 in NVFP4; FlashInfer's PrimsTS kernel reads NVFP4 latents).
# The pages give only the width. Reading: the 512 value dims in NVFP4 -- e2m1
# codes (element 2i in the low nibble of byte i, 256 B) with one e4m3 scale per 16
# dims (32 B) -- and the last 64 dims as plain e4m3 codes (64 B): 256 + 32 + 64 =
# 352 B. As for the FP8 latent, each token also has one fp32 scale (the format's
# second-level scale, taken per token) in the page's scale array:
#   dim d < 512:   s * E4M3(block_scale[d // 16]) * E2M1(code[d])
#   dim d >= 512:  s * E4M3(tail[d - 512])
# ---------------------------------------------------------------------------
NV_BLOCK = 16
NV_RECORD = D_V // 2 + D_V // NV_BLOCK + (D_LAT - D_V)   # 352


def latent_record_bytes(latent_fmt: str) -> int:
    """Bytes of one token's latent record before the page's fp32 scale array."""
    return {"fp8": D_LAT, "nvfp4": NV_RECORD}[latent_fmt]


def nvfp4_latent_decode(rec: np.ndarray) -> np.ndarray:
    """[..., 352] NVFP4 latent records -> float64 [..., 576], before the token scale."""
    rec = np.asarray(rec, dtype=np.uint8)
    packed = rec[..., :D_V // 2]
    bsc = rec[..., D_V // 2:D_V // 2 + D_V // NV_BLOCK]
    tail = rec[..., D_V // 2 + D_V // NV_BLOCK:]
    nib = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(*packed.shape[:-1], D_V)
    vals = E2M1_TABLE[nib] * np.repeat(E4M3_TABLE[bsc], NV_BLOCK, axis=-1)
    return np.concatenate([vals, E4M3_TABLE[tail]], axis=-1)


def index_query(q_codes: np.ndarray, q_scale: np.ndarray, index_fmt: str) -> np.ndarray:
    """Dequantised indexer query [32, 128]: FP8 codes times one fp32 scale per head,
    or MXFP4 codes with one E8M0 per 32 elements."""
    if index_fmt == "fp8":
        return E4M3_TABLE[np.asarray(q_codes)] * np.asarray(q_scale, dtype=np.float32).astype(np.float64)[:, None]
    return mxfp4_decode(np.asarray(q_codes), np.asarray(q_scale))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    u = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# The three steps.
# ---------------------------------------------------------------------------

def indexer_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray, chunk: int = 65536) -> np.ndarray:
    """s_t = sum_h w_h * max(0, q_h . k_t), float64 [n]."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    out = np.empty(keys.shape[0], dtype=np.float64)
    for a in range(0, keys.shape[0], chunk):
        dots = keys[a:a + chunk] @ q.T                 # [m, 32]
        out[a:a + chunk] = np.maximum(dots, 0.0) @ w
    return out


def indexer_magnitude(q: np.ndarray, w: np.ndarray, keys: np.ndarray, chunk: int = 65536) -> np.ndarray:
    """sum_h |w_h| * sum_d |q_hd * k_td|: the size of the terms a score adds up
    (used only to state rounding tolerances)."""
    w = np.abs(np.asarray(w, dtype=np.float32).astype(np.float64))
    out = np.empty(keys.shape[0], dtype=np.float64)
    for a in range(0, keys.shape[0], chunk):
        out[a:a + chunk] = (np.abs(keys[a:a + chunk]) @ np.abs(q).T) @ w
    return out


def select_topk(scores32: np.ndarray, k: int) -> np.ndarray:
    """The min(k, n) largest scores, equal scores ordered by lower token index;
    returned as ascending token positions (int64)."""
    s = np.asarray(scores32, dtype=np.float32)
    n = s.shape[0]
    if n == 0 or k <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(n), -s.astype(np.float64)))
    return np.sort(order[:min(k, n)])


def sparse_mla(q_lat: np.ndarray, lat: np.ndarray, sm_scale: float):
    """Exact attention of every latent-query head over the given latents.

    logits[h, t] = (q_h . c_t) * sm_scale over all 576 dims; p = softmax over t;
    out[h] = sum_t p[h, t] * c_t[:512]; lse[h] = ln sum_t exp(logits[h, t]).
    No tokens -> out = 0, lse = -inf.
    """
    if lat.shape[0] == 0:
        return np.zeros((q_lat.shape[0], D_V)), np.full(q_lat.shape[0], -np.inf)
    logits = (q_lat @ lat.T) * sm_scale                  # [96, m]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ lat[:, :D_V]) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# One query row of the decode step, and the byte accounting quoted on the pages.
# ---------------------------------------------------------------------------

def decode_row(pool, layout, layer, bt_row, ctx, q_codes, q_scale, w, q_lat_bits, k, sm_scale,
               idx_override=None, want_magnitude=False):
    """Indexer over tokens [0, ctx), top-k, sparse MLA over the selected tokens.

    ``idx_override`` (token positions) replaces the oracle's own selection in the
    attention step, so attention can be checked on another implementation's set.
    Returns dict(scores=float64 [ctx], scores32, idx (ascending, int64), out, lse[, mag]).
    """
    lay = layout if isinstance(layout, Layout) else Layout(layout)
    ctx = max(0, int(ctx))
    q = index_query(q_codes, q_scale, lay.index_fmt)
    s = np.empty(ctx, dtype=np.float64)
    mag = np.empty(ctx, dtype=np.float64) if want_magnitude else None
    for a in range(0, ctx, 65536):                       # keys are read 64K tokens at a time
        toks = np.arange(a, min(a + 65536, ctx))
        keys = read_index_keys(pool, lay, layer, bt_row, toks)
        s[a:a + toks.size] = indexer_scores(q, w, keys)
        if want_magnitude:
            mag[a:a + toks.size] = indexer_magnitude(q, w, keys)
    s32 = s.astype(np.float32)
    idx = select_topk(s32, k)
    use = idx if idx_override is None else np.asarray(idx_override, dtype=np.int64)
    lat = read_latents(pool, lay, layer, bt_row, use)
    out, lse = sparse_mla(bf16_to_f64(q_lat_bits), lat, sm_scale)
    res = dict(scores=s, scores32=s32, idx=idx, out=out, lse=lse)
    if want_magnitude:
        res["mag"] = mag
    return res


def index_key_bytes(index_fmt: str) -> int:
    """Per-token index-key bytes: FP8 128 codes + fp32 scale; MXFP4 64 B of e2m1
    pairs + 4 E8M0 (page 1, KV-cache section; page 1, AMD section)."""
    return D_IDX + 4 if index_fmt == "fp8" else D_IDX // 2 + D_IDX // MX_GROUP


def latent_bytes(latent_fmt: str) -> int:
    """Per-token latent bytes: 576 one-byte e4m3 codes in FP8; the page quotes
    352 for NVFP4 (page 1, section on the KV cache serving three kinds of state)."""
    return {"fp8": D_LAT, "nvfp4": 352}[latent_fmt]


def dsa_layer_bytes(ctx: int, k: int, index_fmt: str = "fp8", latent_fmt: str = "fp8") -> int:
    """Bytes one decode step reads per layer: every index key, then the latent of
    min(k, ctx) tokens (page 1, "Sparse attention in K3.1 Pro")."""
    return ctx * index_key_bytes(index_fmt) + min(k, ctx) * latent_bytes(latent_fmt)


def dense_mla_layer_bytes(ctx: int, latent_fmt: str = "fp8") -> int:
    return ctx * latent_bytes(latent_fmt)


def kv_bytes_per_token(layers: int, latent_fmt: str, index_fmt) -> int:
    """Per-GPU per-token cache bytes over ``layers`` DSA layers (TP replicates both caches)."""
    return layers * (latent_bytes(latent_fmt) + (index_key_bytes(index_fmt) if index_fmt else 0))


# ---------------------------------------------------------------------------
# New-token cache append: the step just before the hot path (page 1, fused
# front-end: the new token's index key is quantised and written, and its latent
# is written into the cache, before scoring). The pages do not spell out the
# quantiser; the reading used here, per vector:
#   FP8   scale = amax / 448 in fp32 (1 when amax = 0); y = x / scale in fp32,
#         clamped to +-448 and rounded to the nearest e4m3 value, ties to the
#         even code; the sign bit follows the sign of y (so -0 gives 0x80).
#   MXFP4 per 32 elements E = floor(log2 amax) - 2 clamped to [-127, 127] (0 when
#         amax = 0), stored as the E8M0 byte E + 127; y = x / 2^E rounded to the
#         nearest e2m1 magnitude, ties to the even code, 6 at most; no negative 0.
# Rounding is done by searching the value tables above, not by formula.
# ---------------------------------------------------------------------------

_E4M3_POS = np.array([E4M3_TABLE[c] for c in range(0x7F)], dtype=np.float64)  # codes 0x00..0x7E
_E2M1_POS = E2M1_TABLE[:8]                                                       # nibbles 0..7


def _nearest_even(table: np.ndarray, mag: float) -> int:
    """Index of the table value nearest to mag; on a tie the even index."""
    d = np.abs(table - mag)
    best = np.flatnonzero(d == d.min())
    even = [int(i) for i in best if i % 2 == 0]
    return even[0] if even else int(best[0])


def e4m3_encode(y: float) -> int:
    """e4m3 code of an fp32 value already inside [-448, 448]."""
    y = float(np.float32(y))
    code = _nearest_even(_E4M3_POS, abs(y))
    return code | (0x80 if math.copysign(1.0, y) < 0 else 0)


def e2m1_encode(y: float) -> int:
    """e2m1 nibble of a value (magnitudes above 6 clamp to 6)."""
    m = _nearest_even(_E2M1_POS, min(abs(y), 6.0))
    return m | (0x8 if (y < 0 and m > 0) else 0)


def quantize_fp8_vector(x) -> tuple:
    """(codes uint8 [D], fp32 scale) of one vector, per the reading above."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    y = np.clip((x / scale).astype(np.float32), np.float32(-448.0), np.float32(448.0))
    return np.array([e4m3_encode(v) for v in y], dtype=np.uint8), scale


def quantize_mxfp4_vector(x) -> tuple:
    """(packed uint8 [D/2] with element 2i in the low nibble of byte i, E8M0 uint8 [D/32])."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    groups = x.reshape(-1, MX_GROUP)
    nib = np.zeros(x.size, dtype=np.uint8)
    e8 = np.zeros(groups.shape[0], dtype=np.uint8)
    for gi, g in enumerate(groups):
        amax = float(np.max(np.abs(g)))
        if amax > 0:
            _, ex = math.frexp(amax)          # amax = m * 2^ex, m in [0.5, 1)
            E = min(max(ex - 1 - 2, -127), 127)
        else:
            E = 0
        e8[gi] = E + 127
        for j, v in enumerate(g):
            nib[gi * MX_GROUP + j] = e2m1_encode(v / 2.0 ** E)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    return packed, e8


def quantize_nvfp4_latent(x) -> tuple:
    """(record uint8 [352], fp32 token scale) of one 576-dim latent, per the NVFP4
    record reading above: s = amax / 448 (1 when amax = 0) and y = x / s clamped to
    +-448, as for FP8; the tail dims are e4m3 codes of y; each 16-dim block of the
    first 512 gets the e4m3 scale code nearest to max|y_block| / 6 (ties to even)
    and e2m1 codes of y / that scale's value (all 0 when the value is 0)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    y = np.clip((x / s).astype(np.float32), np.float32(-448.0), np.float32(448.0))
    nib = np.zeros(D_V, dtype=np.uint8)
    bsc = np.zeros(D_V // NV_BLOCK, dtype=np.uint8)
    for b in range(D_V // NV_BLOCK):
        blk = y[b * NV_BLOCK:(b + 1) * NV_BLOCK]
        code = e4m3_encode(np.float32(np.max(np.abs(blk))) / np.float32(6.0))
        bsc[b] = code
        sv = np.float32(E4M3_TABLE[code])
        if sv > 0:
            for j, v in enumerate(blk):
                nib[b * NV_BLOCK + j] = e2m1_encode(float(np.float32(v) / sv))
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    tail = np.array([e4m3_encode(v) for v in y[D_V:]], dtype=np.uint8)
    return np.concatenate([packed, bsc, tail]), s


def append_tokens(pool: np.ndarray, lay: Layout, layer: int, bt: np.ndarray, row_seq, pos,
                  idx_key=None, latent=None) -> np.ndarray:
    """A copy of ``pool`` with row r's quantised index key (fp32 [R][128]) and
    latent (fp32 [R][576]) written at token pos[r] of block-table row row_seq[r].
    Rows whose position or block id falls outside the table or the pool are skipped."""
    out = np.array(pool, dtype=np.uint8, copy=True).reshape(-1, lay.row_bytes)
    nb = out.shape[0]
    bs = lay.block_size
    bt = np.asarray(bt)
    for r in range(len(pos)):
        p = int(pos[r])
        row = bt[int(row_seq[r])]
        if p < 0 or p >= row.size * bs:
            continue
        blk, slot = int(row[p // bs]), p % bs
        if blk < 0 or blk >= nb:
            continue
        if latent is not None:
            if lay.latent_fmt == "fp8":
                codes, sc = quantize_fp8_vector(latent[r])
            else:
                codes, sc = quantize_nvfp4_latent(latent[r])
            w = codes.size
            o = lay.lat_off[layer]
            out[blk, o + slot * w: o + (slot + 1) * w] = codes
            out[blk, o + bs * w + 4 * slot: o + bs * w + 4 * slot + 4] = np.frombuffer(
                np.float32(sc).tobytes(), dtype=np.uint8)
        if idx_key is not None:
            o = lay.idx_off[layer]
            if lay.index_fmt == "fp8":
                codes, sc = quantize_fp8_vector(idx_key[r])
                out[blk, o + slot * D_IDX: o + (slot + 1) * D_IDX] = codes
                out[blk, o + bs * D_IDX + 4 * slot: o + bs * D_IDX + 4 * slot + 4] = np.frombuffer(
                    np.float32(sc).tobytes(), dtype=np.uint8)
            else:
                packed, e8 = quantize_mxfp4_vector(idx_key[r])
                half = D_IDX // 2
                out[blk, o + slot * half: o + (slot + 1) * half] = packed
                ng = D_IDX // MX_GROUP
                out[blk, o + bs * half + ng * slot: o + bs * half + ng * (slot + 1)] = e8
    return out.reshape(pool.shape)


# ---------------------------------------------------------------------------
# The exact top-k merge of decode context parallelism, emulated on one set of
# scores (page 1, DCP section: each of W GPUs holds every W-th token; each sends
# only its best 1.5 * k / W candidates, each packed with its score into 32 bits
# from the BF16 score; every GPU radix-selects the same global top-k from the
# gathered words; a GPU that holds more of the top-k than it sent is detected and
# resends its full local top-k). Reading: a word is (orderable BF16 key << 16) |
# slot, slot = the candidate's place in its shard's list; T = the BF16 key of the
# k-th largest word; a shard whose list was full resends when its weakest sent key
# reaches T; the answer is the exact fp32 top-k over the sent candidates with key
# >= T and the resent lists.
# ---------------------------------------------------------------------------

def bf16_key(x32) -> np.ndarray:
    """Orderable 16-bit key of fp32 values rounded to BF16 (nearest, ties to even):
    larger value -> larger key, -0 == +0; 0 only for the all-ones NaN pattern."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16          # round to nearest even on the dropped half
    b = (r & 0xFFFF).astype(np.uint32)
    b = np.where(b == 0x8000, 0, b)
    return np.where(b & 0x8000, (~b) & 0xFFFF, b | 0x8000).astype(np.uint32)


def dcp_merge(scores32: np.ndarray, k: int, W: int):
    """(selected tokens ascending, resend mask over shards, words exchanged)."""
    s = np.asarray(scores32, dtype=np.float32)
    n = s.shape[0]
    M = -(-3 * k // (2 * W))                           # ceil(1.5 k / W)
    sent, words = [], []
    for r in range(W):
        tok = np.arange(r, n, W)
        loc = select_topk(s[tok], M)
        g = tok[loc]
        sent.append((tok, g))
        keys = bf16_key(s[g]) if g.size else np.zeros(0, np.uint32)
        words.extend(((keys.astype(np.uint64) << 16) | np.arange(g.size, dtype=np.uint64)).tolist())
    words = np.array(sorted(words, reverse=True), dtype=np.uint64)
    T = int(words[k - 1] >> 16) if words.size >= k else 0
    mask = 0
    union = []
    for r, (tok, g) in enumerate(sent):
        keys = bf16_key(s[g]) if g.size else np.zeros(0, np.uint32)
        if tok.size > g.size and g.size and int(keys.min()) >= T:
            mask |= 1 << r
            union.append(tok[select_topk(s[tok], k)])
        else:
            union.append(g[keys >= T])
    u = np.sort(np.concatenate(union)) if union else np.zeros(0, np.int64)   # token order: ties by token
    pick = select_topk(s[u], k)
    return np.sort(u[pick]), mask, int(words.size)
