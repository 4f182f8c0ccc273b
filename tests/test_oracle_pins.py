"""Pins for the CPU oracle, against facts that do not come from the oracle itself:
library conversions, closed forms, brute force on tiny inputs, invariants of
the definitions, and the byte figures the pages print (tests/golden)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


# ------------------------------------------------------------------ dequant tables
def test_e4m3_table_matches_torch_exhaustive():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(O.E4M3_TABLE)
    assert np.array_equal(np.isnan(ref), np.isnan(O.E4M3_TABLE))
    assert np.all((ref == O.E4M3_TABLE) | both_nan)
    assert O.E4M3_TABLE[0x7E] == 448.0 and O.E4M3_TABLE[0x01] == 2.0 ** -9


def test_e8m0_table_matches_torch_exhaustive():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(O.E8M0_TABLE))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], O.E8M0_TABLE[ok])
    assert O.E8M0_TABLE[127] == 1.0


def test_e2m1_table_matches_spec_listing():
    # OCP MX v1.0 FP4 (E2M1) value listing, codes 0..15.
    spec = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert list(O.E2M1_TABLE) == spec


def test_mxfp4_decode_nibble_order_and_group_scale():
    packed = np.zeros((1, 64), np.uint8)
    packed[0, 0] = 0x2 | (0x7 << 4)       # element 0 = 1.0 (low nibble), element 1 = 6.0
    packed[0, 16] = 0xB                    # element 32 = -1.5
    e8 = np.array([[127, 129, 0, 254]], np.uint8)
    v = O.mxfp4_decode(packed, e8)[0]
    assert v[0] == 1.0 and v[1] == 6.0
    assert v[32] == -1.5 * 4.0
    assert np.count_nonzero(v) == 3


# ------------------------------------------------------------------ page walk
def _struct_pool(bs, n_blocks, layers, fmt):
    """A pool built through numpy structured dtypes (a different route from the
    oracle's offset arithmetic): per layer a latent page {codes[bs][576], scales[bs]}
    followed by an index page."""
    fields = []
    for l in range(layers):
        fields.append((f"lat{l}", [("c", "u1", (bs, 576)), ("s", "<f4", (bs,))]))
        if fmt == "fp8":
            fields.append((f"idx{l}", [("c", "u1", (bs, 128)), ("s", "<f4", (bs,))]))
        else:
            fields.append((f"idx{l}", [("c", "u1", (bs, 64)), ("e", "u1", (bs, 4))]))
    dt = np.dtype(fields)
    rows = np.zeros(n_blocks, dtype=dt)
    lat_off = [dt.fields[f"lat{l}"][1] for l in range(layers)]
    idx_off = [dt.fields[f"idx{l}"][1] for l in range(layers)]
    lay = dict(block_size=bs, index_fmt=fmt, row_bytes=dt.itemsize, lat_off=lat_off, idx_off=idx_off)
    return rows, lay


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_page_walk_against_structured_pool(fmt):
    bs, nb, L = 16, 7, 2
    rows, lay = _struct_pool(bs, nb, L, fmt)
    bt = np.array([5, 2, 6, 0, 3], np.int32)          # logical block j -> physical row
    n_tok = 70
    code = rng.integers(0, 0x7E, size=(L, n_tok, 576), dtype=np.uint8)     # no NaN codes
    scale = rng.uniform(0.5, 2.0, size=(L, n_tok)).astype(np.float32)
    kcode = rng.integers(0, 0x7E, size=(L, n_tok, 128), dtype=np.uint8)
    kscale = rng.uniform(0.5, 2.0, size=(L, n_tok)).astype(np.float32)
    kpack = rng.integers(0, 256, size=(L, n_tok, 64), dtype=np.uint8)
    ke8 = rng.integers(120, 135, size=(L, n_tok, 4), dtype=np.uint8)
    for l in range(L):
        for t in range(n_tok):
            r, s = bt[t // bs], t % bs
            rows[r][f"lat{l}"]["c"][s] = code[l, t]
            rows[r][f"lat{l}"]["s"][s] = scale[l, t]
            if fmt == "fp8":
                rows[r][f"idx{l}"]["c"][s] = kcode[l, t]
                rows[r][f"idx{l}"]["s"][s] = kscale[l, t]
            else:
                rows[r][f"idx{l}"]["c"][s] = kpack[l, t]
                rows[r][f"idx{l}"]["e"][s] = ke8[l, t]
    pool = rows.view(np.uint8).reshape(nb, -1)
    layout = O.Layout(lay)
    toks = np.arange(n_tok)
    for l in range(L):
        lat = O.read_latents(pool, layout, l, bt, toks)
        ref = torch.from_numpy(code[l]).view(torch.float8_e4m3fn).double().numpy() * scale[l, :, None].astype(np.float64)
        assert np.array_equal(lat, ref)
        keys = O.read_index_keys(pool, layout, l, bt, toks)
        if fmt == "fp8":
            refk = torch.from_numpy(kcode[l]).view(torch.float8_e4m3fn).double().numpy() * kscale[l, :, None].astype(np.float64)
        else:
            lo, hi = kpack[l] & 15, kpack[l] >> 4
            nib = np.empty((n_tok, 128), np.uint8)
            nib[:, 0::2], nib[:, 1::2] = lo, hi
            spec = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
            mag = spec[nib & 7] * np.where(nib & 8, -1.0, 1.0)
            refk = mag * np.repeat(2.0 ** (ke8[l].astype(np.float64) - 127), 32, axis=1)
        assert np.array_equal(keys, refk)


def test_decode_row_paging_invariance():
    from synth import make_case
    c = make_case([700], block_size=16, seed=3)
    pool = c.pool.numpy()
    bt = c.block_table.numpy()[0]
    nb = pool.shape[0]
    perm = np.random.default_rng(1).permutation(nb)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool                                   # physical row i moves to perm[i]
    bt2 = perm[bt[bt >= 0]]
    args = (c.q_idx[0, 0].numpy(), c.q_idx_scale[0, 0].numpy(), c.w[0, 0].numpy(),
            c.q_lat[0, 0].view(torch.int16).numpy().view(np.uint16), 64, c.sm_scale)
    a = O.decode_row(pool, c.layout, 0, bt, 700, *args)
    b = O.decode_row(pool2, c.layout, 0, bt2, 700, *args)
    assert np.array_equal(a["scores"], b["scores"])
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


def test_generated_cache_statistics():
    """The generator draws N(0,1) keys and latents: the dequantised cache read
    back through the page walk must have mean ~0, variance ~1, and each token's
    largest code is exactly +-448 (scale = amax / 448)."""
    from synth import make_case
    c = make_case([4096], block_size=64, num_layers=2, seed=5)
    pool = c.pool.numpy()
    bt = c.block_table.numpy()[0]
    lay = O.Layout(c.layout)
    for l in range(2):
        k = O.read_index_keys(pool, lay, l, bt, np.arange(4096))
        v = O.read_latents(pool, lay, l, bt, np.arange(4096))
        for x in (k, v):
            assert abs(x.mean()) < 0.01 and abs(x.var() - 1.0) < 0.02
        base = lay.idx_off[l]
        codes = pool[:, base:base + 64 * 128].reshape(-1, 128)
        assert np.all(np.abs(O.E4M3_TABLE[codes]).max(axis=1) == 448.0)
    k0 = O.read_index_keys(pool, lay, 0, bt, np.arange(64))
    k1 = O.read_index_keys(pool, lay, 1, bt, np.arange(64))
    assert not np.array_equal(k0, k1)


# ------------------------------------------------------------------ scores
def _brute_scores(q, w, keys):
    out = []
    for t in range(keys.shape[0]):
        s = 0.0
        for h in range(q.shape[0]):
            d = 0.0
            for j in range(q.shape[1]):
                d += q[h, j] * keys[t, j]
            s += float(np.float32(w[h])) * (d if d > 0 else 0.0)
        out.append(s)
    return np.array(out)


def test_scores_brute_force_tiny():
    q = rng.standard_normal((32, 128))
    w = (rng.standard_normal(32) / math.sqrt(32)).astype(np.float32)
    keys = rng.standard_normal((12, 128))
    got = O.indexer_scores(q, w, keys)
    ref = _brute_scores(q, w, keys)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_scores_closed_forms():
    keys = rng.standard_normal((50, 128))
    d = rng.integers(0, 128, size=32)
    q = np.zeros((32, 128))
    q[np.arange(32), d] = 1.0
    w = np.ones(32, np.float32)
    assert np.allclose(O.indexer_scores(q, w, keys), np.maximum(keys[:, d], 0).sum(axis=1), rtol=0, atol=1e-12)
    # ReLU before the weights: negative dots contribute nothing, whatever the sign of w
    wneg = -np.abs(rng.standard_normal(32)).astype(np.float32)
    assert np.all(O.indexer_scores(-np.abs(q), wneg, np.abs(keys)) == 0.0)
    assert np.all(O.indexer_scores(q, w, np.zeros((5, 128))) == 0.0)
    # one live head: s = w_h * (q_h . k)
    q1 = np.zeros((32, 128)); q1[3] = rng.standard_normal(128)
    w1 = np.zeros(32, np.float32); w1[3] = 2.5
    dots = keys @ q1[3]
    assert np.allclose(O.indexer_scores(q1, w1, keys), 2.5 * np.maximum(dots, 0), atol=1e-12)


def test_mxfp4_query_and_score_brute_force():
    packed = rng.integers(0, 256, size=(32, 64), dtype=np.uint8)
    e8 = rng.integers(124, 131, size=(32, 4), dtype=np.uint8)
    q = O.index_query(packed, e8, "mxfp4")
    kp = rng.integers(0, 256, size=(9, 64), dtype=np.uint8)
    ke = rng.integers(124, 131, size=(9, 4), dtype=np.uint8)
    keys = O.mxfp4_decode(kp, ke)
    w = rng.standard_normal(32).astype(np.float32)
    assert np.allclose(O.indexer_scores(q, w, keys), _brute_scores(q, w, keys), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ selection
def _brute_select(s, k):
    """t is kept iff fewer than k tokens beat it (higher score, or equal score
    and lower index)."""
    n = len(s)
    keep = []
    for t in range(n):
        beat = sum(1 for u in range(n) if s[u] > s[t] or (s[u] == s[t] and u < t))
        if beat < k:
            keep.append(t)
    return np.array(keep, dtype=np.int64)


@pytest.mark.parametrize("n,k", [(10, 3), (12, 12), (9, 20), (11, 1)])
def test_select_brute_force(n, k):
    for trial in range(20):
        s = rng.integers(-3, 4, size=n).astype(np.float32)   # many ties
        assert np.array_equal(O.select_topk(s, k), _brute_select(s, k))


def test_select_matches_stable_argsort():
    s = rng.standard_normal(5000).astype(np.float32)
    s[::7] = s[3]                                            # plant equal scores
    ref = np.sort(np.argsort(-s, kind="stable")[:2048])
    assert np.array_equal(O.select_topk(s, 2048), ref)


def test_select_constant_and_signed_zero():
    assert np.array_equal(O.select_topk(np.zeros(5000, np.float32), 2048), np.arange(2048))
    s = np.zeros(10, np.float32); s[::2] = -0.0
    assert np.array_equal(O.select_topk(s, 4), np.arange(4))
    assert O.select_topk(np.zeros(0, np.float32), 2048).size == 0


# ------------------------------------------------------------------ attention
def _sdpa_f64(q, lat, scale):
    qt = torch.from_numpy(q)[None, :, None, :]                 # [1, 96, 1, 576]
    kt = torch.from_numpy(lat)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(lat[:, :512]))[None, None].expand(1, q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0].numpy()


def test_attention_matches_sdpa():
    q = rng.standard_normal((96, 576))
    lat = rng.standard_normal((300, 576)) * 0.5
    out, lse = O.sparse_mla(q, lat, 1 / 24)
    assert np.allclose(out, _sdpa_f64(q, lat, 1 / 24), rtol=1e-10, atol=1e-12)
    from scipy.special import logsumexp
    assert np.allclose(lse, logsumexp((q @ lat.T) / 24, axis=1), rtol=1e-12)


def test_attention_invariants():
    q = rng.standard_normal((96, 576))
    lat = rng.standard_normal((257, 576))
    out, lse = O.sparse_mla(q, lat, 1 / 24)
    logits = (q @ lat.T) / 24
    assert np.allclose(np.exp(logits - lse[:, None]).sum(axis=1), 1.0, atol=1e-12)
    perm = rng.permutation(257)
    out2, lse2 = O.sparse_mla(q, lat[perm], 1 / 24)
    assert np.allclose(out, out2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
    one, l1 = O.sparse_mla(q, lat[5:6], 1 / 24)
    assert np.array_equal(one, np.broadcast_to(lat[5, :512], (96, 512)))
    assert np.allclose(l1, logits[:, 5])
    same = np.repeat(lat[7:8], 40, axis=0)
    o3, _ = O.sparse_mla(q, same, 1 / 24)
    assert np.allclose(o3, lat[7, :512], atol=1e-12)
    oe, le = O.sparse_mla(q, np.zeros((0, 576)), 1 / 24)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def test_decode_row_short_context_is_dense_mla():
    from synth import make_case
    c = make_case([1000], block_size=64, seed=9)
    pool = c.pool.numpy(); bt = c.block_table.numpy()[0]
    ql = c.q_lat[0, 0].view(torch.int16).numpy().view(np.uint16)
    r = O.decode_row(pool, c.layout, 0, bt, 1000, c.q_idx[0, 0].numpy(), c.q_idx_scale[0, 0].numpy(),
                     c.w[0, 0].numpy(), ql, 2048, c.sm_scale)
    assert np.array_equal(r["idx"], np.arange(1000))
    lat = O.read_latents(pool, O.Layout(c.layout), 0, bt, np.arange(1000))
    ref = _sdpa_f64(O.bf16_to_f64(ql), lat, c.sm_scale)
    assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-12)


def test_planted_tokens_dominate_selection():
    """Keys shifted by +3 sigma along every head (sign of w) must outrank the rest."""
    from synth import make_case
    c = make_case([20000], block_size=64, seed=4, plant=256)
    pool = c.pool.numpy(); bt = c.block_table.numpy()[0]
    r = O.decode_row(pool, c.layout, 0, bt, 20000, c.q_idx[0, 0].numpy(), c.q_idx_scale[0, 0].numpy(),
                     c.w[0, 0].numpy(), c.q_lat[0, 0].view(torch.int16).numpy().view(np.uint16), 256, c.sm_scale)
    planted = set(c.planted[(0, 0)])
    assert len(planted & set(r["idx"].tolist())) >= 0.95 * 256


# ------------------------------------------------------------------ byte accounting (pages)
def test_byte_accounting_golden():
    g = json.load(open(os.path.join(GOLDEN, "page_byte_accounting.json")))
    assert O.latent_bytes("fp8") == g["fp8_latent_bytes_per_token"]["value"]
    assert O.latent_bytes("nvfp4") == g["nvfp4_latent_bytes_per_token"]["value"]
    assert O.index_key_bytes("fp8") == g["fp8_index_key_bytes_per_token"]["value"]
    assert O.index_key_bytes("mxfp4") == g["mxfp4_index_key_bytes_per_token"]["value"]
    red = 100.0 * (1 - O.index_key_bytes("mxfp4") / O.index_key_bytes("fp8"))
    e = g["mxfp4_index_storage_reduction_pct"]
    assert abs(red - e["value"]) <= e["tol"]
    e = g["dsa_over_dense_mla_bytes_long_context_pct"]
    frac = 100.0 * O.dsa_layer_bytes(e["ctx"], e["k"]) / O.dense_mla_layer_bytes(e["ctx"])
    assert abs(frac - e["value"]) <= e["tol"]
    for key in ("kv_bytes_per_token_24_layers_k3_fp8", "kv_bytes_per_token_24_layers_fp8_fp8",
                "kv_bytes_per_token_24_layers_nvfp4_mxfp4"):
        e = g[key]
        assert O.kv_bytes_per_token(e["layers"], e["latent"], e["index"]) == e["value"], key
    assert (O.H_IDX, O.D_IDX, O.H_Q) == (g["indexer_heads"]["value"], g["indexer_head_dim"]["value"],
                                          g["attention_heads"]["value"])


# ----------------------------------------------------------------------------- cache append
def test_e4m3_encode_matches_torch_cast_on_every_midpoint():
    """The oracle's table-search rounding against torch's own float8_e4m3fn cast: every
    code value, every midpoint between neighbouring codes (the ties), and random values."""
    import torch
    pos = O.E4M3_TABLE[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(3)
    vals = np.concatenate([pos, mids, -pos, -mids, rng.uniform(-448, 448, 3000),
                           rng.normal(0, 0.01, 1000)]).astype(np.float32)
    want = torch.tensor(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_encode_round_trip_and_ties():
    for c in range(256):
        v = O.E4M3_TABLE[c]
        if np.isnan(v):
            continue
        assert O.e4m3_encode(v) == c, hex(c)
    assert O.e4m3_encode(1.0625) == 0x38      # 1.0 | 1.125: even code
    assert O.e4m3_encode(1.1875) == 0x3A      # 1.125 | 1.25: even code
    assert O.e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal: even (zero)


def test_e2m1_encode_ties_clamp_and_round_trip():
    for n in range(16):
        if n == 8:
            continue                          # -0 is never produced
        assert O.e2m1_encode(O.E2M1_TABLE[n]) == n
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, n in ties.items():
        assert O.e2m1_encode(v) == n and O.e2m1_encode(-v) == (n | 8 if n else 0)
    assert O.e2m1_encode(7.9) == 7 and O.e2m1_encode(-100.0) == 15


def test_quantize_fp8_vector_error_bound():
    """Every dequantised element is within half a code spacing (times the scale) of the input."""
    rng = np.random.default_rng(4)
    for x in [rng.normal(0, 1, 576), rng.normal(0, 1e-3, 128), np.zeros(128), np.r_[np.zeros(127), -5.0]]:
        codes, sc = O.quantize_fp8_vector(x)
        x32 = np.asarray(x, dtype=np.float32).astype(np.float64)
        deq = O.E4M3_TABLE[codes] * float(sc)
        amax = np.abs(x32).max()
        assert float(sc) == (float(np.float32(amax / np.float32(448))) if amax > 0 else 1.0)
        mag = np.abs(x32 / float(sc))
        e = np.floor(np.log2(np.maximum(mag, 2.0 ** -6)))
        half = 2.0 ** (e - 3) / 2 * float(sc)         # half the spacing at that binade (3 mantissa bits)
        assert np.all(np.abs(deq - x32) <= half * (1 + 1e-6) + 1e-30)
        if amax > 0:
            assert np.max(np.abs(deq)) == pytest.approx(amax, rel=1e-6)


def test_quantize_mxfp4_vector_exponent_and_bound():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, 128) * np.repeat([1e-3, 1.0, 40.0, 0.0], 32)
    packed, e8 = O.quantize_mxfp4_vector(x)
    assert e8[3] == 127                                  # an all-zero group keeps scale 1
    deq = O.mxfp4_decode(packed[None], e8[None])[0]
    x32 = np.asarray(x, dtype=np.float32).astype(np.float64)
    for g in range(3):
        s = slice(32 * g, 32 * g + 32)
        amax = np.abs(x32[s]).max()
        E = int(e8[g]) - 127
        assert 2.0 ** (E + 2) <= amax < 2.0 ** (E + 3)   # amax / 2^E in [4, 8)
        # nearest e2m1 step is at most 2 (between 4 and 6), and 6 caps values up to 8
        assert np.all(np.abs(deq[s] - x32[s]) <= 2.0 * 2.0 ** E + 1e-30)


def test_append_tokens_writes_only_the_token_slot():
    from synth import make_case
    c = make_case([200, 90], block_size=16, seed=8, k=64)
    lay = O.Layout(c.layout)
    pool = c.pool.numpy().copy()
    bt = c.block_table.numpy()
    rng = np.random.default_rng(6)
    key = rng.normal(0, 1, (3, 128)).astype(np.float32)
    lat = rng.normal(0, 2, (3, 576)).astype(np.float32)
    row_seq, pos = [0, 1, 1], [150, 5, 10 ** 6]        # the last row is outside its table: skipped
    out = O.append_tokens(pool, lay, 0, bt, row_seq, pos, idx_key=key, latent=lat)
    diff = np.flatnonzero(out.reshape(-1) != pool.reshape(-1))
    rows = set((diff // lay.row_bytes).tolist())
    assert rows <= {int(bt[0][150 // 16]), int(bt[1][5 // 16])}
    for r in range(2):
        k_back = O.read_index_keys(out, lay, 0, bt[row_seq[r]], [pos[r]])[0]
        l_back = O.read_latents(out, lay, 0, bt[row_seq[r]], [pos[r]])[0]
        assert np.max(np.abs(k_back - key[r])) <= np.abs(key[r]).max() / 448 * 16 + 1e-12
        assert np.max(np.abs(l_back - lat[r])) <= np.abs(lat[r]).max() / 448 * 16 + 1e-12


# ----------------------------------------------------------------------------- DCP merge
def test_bf16_key_orders_like_the_rounded_values():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.normal(0, 1, 4000), [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40]]).astype(np.float32)
    import torch
    b = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)   # torch's own RNE
    k = O.bf16_key(x).astype(np.int64)
    i, j = rng.integers(0, x.size, (2, 20000))
    assert np.array_equal(np.sign(k[i] - k[j]), np.sign(b[i] - b[j]))
    assert O.bf16_key(np.float32(-0.0)) == O.bf16_key(np.float32(0.0))


@pytest.mark.parametrize("W", [2, 4, 8])
def test_dcp_merge_equals_the_plain_top_k(W):
    """Random rows, rows with ties, and rows whose top-k sits in one shard's tokens (which
    forces that shard to resend): the merged selection is the exact top-k every time."""
    rng = np.random.default_rng(20 + W)
    cases = [rng.normal(0, 1, 20000), np.round(rng.normal(0, 1, 20000), 1), rng.normal(0, 1, 300)]
    hot = rng.normal(0, 1, 20000)
    hot[3::W] += 5.0                                    # shard 3 % W holds the whole top-k
    cases.append(hot)
    for c in cases:
        s = c.astype(np.float32)
        got, mask, nw = O.dcp_merge(s, 512, W)
        assert np.array_equal(got, O.select_topk(s, 512))
    assert mask & (1 << (3 % W)), "the shard holding the whole top-k must resend"
    _, mask_rand, nw = O.dcp_merge(cases[0], 512, W)
    assert nw == W * -(-3 * 512 // (2 * W))              # 32-bit words exchanged: W x ceil(1.5 k / W)


def test_dcp_merge_resend_rule_by_hand():
    """Two shards, k = 4, M = 3: shard 0 holds the four largest scores, so its weakest sent
    word ties the threshold and it must resend; shard 1 does not."""
    s = np.array([9, 1, 8, 2, 7, 3, 6, 0.5], dtype=np.float32)   # shard 0: 9 8 7 6, shard 1: 1 2 3 .5
    got, mask, nw = O.dcp_merge(s, 4, 2)
    assert np.array_equal(got, [0, 2, 4, 6]) and mask == 1 and nw == 6


# ----------------------------------------------------------------------------- NVFP4 latents

def test_nvfp4_latent_record_by_hand():
    """The NVFP4 latent record (352 B: 256 B of e2m1 pairs, 32 e4m3 block scales, 64 e4m3
    tail codes) decoded by hand from the format definitions."""
    rec = np.zeros(352, np.uint8)
    rec[0] = 0x3 | (0xA << 4)      # dims 0, 1: e2m1 1.5 and -1.0 (0xA: sign | exponent 1)
    rec[255] = 0x70                # dims 510, 511: e2m1 0 and 6.0
    rec[256] = 0x40                # block 0 (dims 0..15): e4m3 2.0
    rec[256 + 31] = 0x30           # block 31 (dims 496..511): e4m3 0.5
    rec[288] = 0x38                # dim 512: e4m3 1.0
    rec[351] = 0xFE                # dim 575: e4m3 -448
    v = O.nvfp4_latent_decode(rec)
    want = np.zeros(576)
    want[0], want[1], want[511], want[512], want[575] = 3.0, -2.0, 3.0, 1.0, -448.0
    assert v.shape == (576,) and np.array_equal(v, want)
    assert O.latent_record_bytes("nvfp4") == O.latent_bytes("nvfp4") == 352


def test_nvfp4_latent_round_trip_of_representable_vectors():
    """A vector that the format represents exactly (token scale 1: the largest value is a
    448 tail code; each block's largest magnitude is 6 times its scale) comes back with the
    same record."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        rec = np.zeros(352, np.uint8)
        nib = rng.integers(0, 16, 512).astype(np.uint8)
        nib[nib == 0x8] = 0                                  # no negative zero
        for b in range(32):
            nib[16 * b + rng.integers(0, 16)] = rng.choice([0x7, 0xF])   # |6| in every block
        rec[:256] = nib[0::2] | (nib[1::2] << 4)
        # block scales: positive normal e4m3 values up to 64 (6 * 64 < 448)
        rec[256:288] = rng.integers(0x08, 0x58, 32)
        tail = rng.integers(0, 0x7E, 64).astype(np.uint8) | (rng.integers(0, 2, 64).astype(np.uint8) << 7)
        tail[tail == 0x80] = 0
        tail[rng.integers(0, 64)] = 0x7E                     # 448: the token's largest value
        rec[288:] = tail
        x = O.nvfp4_latent_decode(rec).astype(np.float32)
        got, s = O.quantize_nvfp4_latent(x)
        assert s == np.float32(1.0) and np.array_equal(got, rec)


def test_nvfp4_latent_quantiser_error_bound_and_scales():
    """Random latents: every block scale is torch's own e4m3 cast of max|y| / 6, and each
    dequantised dim lies within one block-scale step (NVFP4 dims) or half an e4m3 step
    (tail dims) of the input."""
    import torch
    rng = np.random.default_rng(6)
    for t in range(12):
        x = (rng.normal(0, 1, 576) * (10.0 ** rng.uniform(-3, 3))).astype(np.float32)
        if t == 0:
            x[:32] = 0.0                                     # all-zero blocks: scale 0, codes 0
        rec, s = O.quantize_nvfp4_latent(x)
        y = np.clip(x / s, -448, 448).astype(np.float32)
        bam = np.abs(y[:512]).reshape(32, 16).max(axis=1).astype(np.float32) / np.float32(6.0)
        ref = torch.tensor(bam).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(rec[256:288], ref)
        xh = O.nvfp4_latent_decode(rec) * float(s)
        scv = np.repeat(O.E4M3_TABLE[rec[256:288]], 16)
        err = np.abs(xh - x.astype(np.float64))
        assert np.all(err[:512] <= float(s) * scv * 1.0 + 1e-30)
        assert np.all(err[512:] <= float(s) * np.maximum(np.abs(y[512:]) / 16.0, 2.0 ** -10) * 1.0000001)
        if t == 0:
            assert np.all(rec[:16] == 0) and np.all(rec[256:258] == 0)


def test_generator_writes_nvfp4_records_as_the_oracle_reads_them():
    """The synthetic cache's NVFP4 quantiser (torch, generator side) and the oracle's
    reading of it give the same bytes on CPU."""
    import torch
    from synth.cases import quantize_nvfp4_latent_rows
    rng = np.random.default_rng(8)
    x = (rng.normal(0, 1, (16, 576)) * (10.0 ** rng.uniform(-2, 2, (16, 1)))).astype(np.float32)
    x[3, :40] = 0.0
    rec, s = quantize_nvfp4_latent_rows(torch.from_numpy(x))
    for i in range(16):
        want, ws = O.quantize_nvfp4_latent(x[i])
        assert np.array_equal(rec[i].numpy(), want) and np.float32(s[i].item()) == ws


# ------------------------------------------------------------------ pins for index_query's
# FP8 per-head scale, decode_row past one 65,536-token key chunk, and indexer_magnitude
def _e4m3_lib(codes):
    """e4m3 codes -> float64 through torch's float8_e4m3fn (a library decode)."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _hand_pool_fp8(bs, n_blocks):
    """Zeroed single-layer FP8 pool laid out by hand: latent page (bs x 576 codes, bs
    fp32 scales) then index page (bs x 128 codes, bs fp32 scales)."""
    lat_page = bs * (576 + 4)
    row = lat_page + bs * (128 + 4)
    lay = dict(block_size=bs, index_fmt="fp8", row_bytes=row, lat_off=[0], idx_off=[lat_page])
    return np.zeros((n_blocks, row), np.uint8), lay


def _put_key(pool, lay, bt, t, codes, scale):
    bs = lay["block_size"]
    blk, s = int(bt[t // bs]), t % bs
    o = lay["idx_off"][0]
    pool[blk, o + s * 128:o + (s + 1) * 128] = codes
    pool[blk, o + bs * 128 + 4 * s:o + bs * 128 + 4 * s + 4] = np.frombuffer(np.float32(scale).tobytes(), np.uint8)


def _finite_e4m3_codes(shape):
    c = rng.integers(0, 0x7F, size=shape, dtype=np.uint8)        # 0x00..0x7E: finite
    return c | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)


def test_index_query_fp8_per_head_scale_closed_form():
    """s_t = sum_h w_h * ReLU(sq_h * sk_t * (codes_q[h] . codes_k[t])), one fp32 scale
    per query head. Each head in turn is the only live one, with scales that differ
    from head to head, so a dropped, shared or misindexed query scale changes the
    result. The code dot products are exact in float64 (e4m3 products have 8
    significant bits and 128 of them fit in 53), decoded through torch."""
    bs, nb, n = 16, 6, 90
    pool, lay = _hand_pool_fp8(bs, nb)
    bt = rng.permutation(nb).astype(np.int32)
    kc = _finite_e4m3_codes((n, 128))
    ks = rng.uniform(0.25, 4.0, size=n).astype(np.float32)
    for t in range(n):
        _put_key(pool, lay, bt, t, kc[t], ks[t])
    qc_all = _finite_e4m3_codes((32, 128))
    qs = (2.0 ** rng.integers(-6, 7, size=32) * rng.uniform(1.0, 2.0, size=32)).astype(np.float32)
    assert len(set(qs.tolist())) == 32
    w = (rng.standard_normal(32) / math.sqrt(32)).astype(np.float32)
    dots = _e4m3_lib(kc) @ _e4m3_lib(qc_all).T                    # [n, 32] exact integer-scaled sums
    ql = np.zeros((96, 576), np.uint16)
    for h in (0, 5, 17, 31):
        qc = np.zeros((32, 128), np.uint8)
        qc[h] = qc_all[h]
        r = O.decode_row(pool, lay, 0, bt, n, qc, qs, w, ql, 8, 1 / 24)
        ref = float(w[h]) * np.maximum(float(qs[h]) * ks.astype(np.float64) * dots[:, h], 0.0)
        assert np.allclose(r["scores"], ref, rtol=1e-12, atol=0), h
        assert np.count_nonzero(ref) > 0
    # every head live at once: the per-head sum of the same closed form
    r = O.decode_row(pool, lay, 0, bt, n, qc_all, qs, w, ql, 8, 1 / 24)
    ref = (np.maximum(dots * qs.astype(np.float64)[None, :] * ks.astype(np.float64)[:, None], 0.0)
           * w.astype(np.float64)[None, :]).sum(axis=1)
    assert np.allclose(r["scores"], ref, rtol=1e-12, atol=1e-300)


def test_decode_row_past_one_key_chunk_closed_form():
    """A 70,000-token context: every key is zero except one-hot tokens spread over
    both 65,536-token chunks and straddling the chunk boundary, so each score is
    known in closed form, s_t = sum_h w_h * ReLU(sq_h * e4m3(q[h, d_t]) * v_t * sk_t),
    and the top-k is the positive scores, then the zero scores by token order."""
    bs, ctx = 1024, 70000
    nb = -(-ctx // bs)
    pool, lay = _hand_pool_fp8(bs, nb)
    bt = rng.permutation(nb).astype(np.int32)
    sc1 = np.frombuffer(np.float32(1.0).tobytes(), np.uint8)
    o = lay["idx_off"][0]
    pool[:, o + bs * 128:o + bs * 132] = np.tile(sc1, bs)[None, :]
    hot = sorted(set([0, 5, 40000, 65534, 65535, 65536, 65537, 69999]
                     + rng.integers(0, ctx, size=40).tolist()))
    dpos = rng.integers(0, 128, size=len(hot))
    vcode = _finite_e4m3_codes(len(hot))
    vcode[vcode == 0] = 0x38
    vcode[vcode == 0x80] = 0xB8
    ksc = rng.uniform(0.5, 2.0, size=len(hot)).astype(np.float32)
    for i, t in enumerate(hot):
        c = np.zeros(128, np.uint8)
        c[dpos[i]] = vcode[i]
        _put_key(pool, lay, bt, t, c, ksc[i])
    qc = _finite_e4m3_codes((32, 128))
    qs = rng.uniform(0.01, 0.1, size=32).astype(np.float32)
    w = (rng.standard_normal(32) / math.sqrt(32)).astype(np.float32)
    qv = _e4m3_lib(qc) * qs.astype(np.float64)[:, None]
    vv = _e4m3_lib(vcode)
    ref = np.zeros(ctx)
    for i, t in enumerate(hot):
        ref[t] = sum(float(w[h]) * max(0.0, qv[h, dpos[i]] * vv[i] * float(ksc[i])) for h in range(32))
    k = 2048
    r = O.decode_row(pool, lay, 0, bt, ctx, qc, qs, w, np.zeros((96, 576), np.uint16), k, 1 / 24)
    assert r["scores"].shape == (ctx,)
    assert np.allclose(r["scores"], ref, rtol=1e-12, atol=0)
    assert np.count_nonzero(r["scores"][[t for t in range(ctx) if t not in set(hot)]]) == 0
    s32 = ref.astype(np.float32)
    expect = sorted(sorted(range(ctx), key=lambda t: (-float(s32[t]), t))[:k])
    assert np.array_equal(r["idx"], np.array(expect))
    assert any(t >= 65536 for t in r["idx"]) and {65535, 65536} & set(r["idx"].tolist()) == \
        {t for t in (65535, 65536) if s32[t] >= 0}


def test_indexer_magnitude_brute_force_and_bound():
    """mag_t = sum_h |w_h| sum_d |q_hd k_td| by explicit loops; |s_t| <= mag_t; and
    with non-negative q, k and w every term is added at full size, so mag_t = s_t."""
    q = rng.standard_normal((32, 128))
    w = rng.standard_normal(32).astype(np.float32)
    keys = rng.standard_normal((7, 128))
    got = O.indexer_magnitude(q, w, keys)
    ref = []
    for t in range(keys.shape[0]):
        m = 0.0
        for h in range(32):
            a = 0.0
            for d in range(128):
                a += abs(q[h, d] * keys[t, d])
            m += abs(float(w[h])) * a
        ref.append(m)
    assert np.allclose(got, np.array(ref), rtol=1e-12, atol=0)
    keys = rng.standard_normal((3000, 128))
    s = O.indexer_scores(q, w, keys)
    mag = O.indexer_magnitude(q, w, keys)
    assert np.all(np.abs(s) <= mag * (1 + 1e-12))
    qp, kp, wp = np.abs(q), np.abs(keys[:50]), np.abs(w)
    assert np.allclose(O.indexer_magnitude(qp, wp, kp), O.indexer_scores(qp, wp, kp), rtol=1e-12, atol=0)
