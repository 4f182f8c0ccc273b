"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/dsa.h declares, sizes its workspaces, and rejects bad arguments
before anything reaches the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

dsa = pytest.importorskip("sparse_attention_decode_paged_amd")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    return dsa.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 9
    raw = ctypes.CDLL(dsa.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(dsa.EXPORTED) == set(names)


def test_version_and_status_strings(lib):
    assert dsa.dsa_abi_version() == 1
    assert dsa.dsa_status_string(0) == "ok"
    for s in range(1, 8):
        assert dsa.dsa_status_string(s) not in ("ok", "unknown status")
    assert dsa.dsa_status_string(99) == "unknown status"


def test_workspace_sizes(lib):
    for op in (dsa.DSA_OP_TOPK, dsa.DSA_OP_SPARSE_MLA, dsa.DSA_OP_DECODE_STEP):
        assert dsa.dsa_workspace_bytes(op, 1, 8192, 2048) > 0
    assert dsa.dsa_workspace_bytes(42, 1, 8192, 2048) == 0
    assert dsa.dsa_workspace_bytes(dsa.DSA_OP_TOPK, 1, 8192, 0) == 0
    assert dsa.dsa_workspace_bytes(dsa.DSA_OP_TOPK, 1, 8192, 4096) == 0
    small = dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, 1, 8192, 2048)
    big = dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, 1, 1 << 20, 2048)
    assert big > small + 4 * ((1 << 20) - 8192)          # holds at least the fp32 scores
    assert dsa.dsa_decode_scores_ld(8192) == 8192
    assert dsa.dsa_decode_scores_ld(8193) % 64 == 0 and dsa.dsa_decode_scores_ld(8193) >= 8193


@pytest.mark.parametrize("R, splits", [(1, 32), (4, 8), (16, 5), (32, 8), (64, 4), (96, 4), (160, 1), (2048, 1)])
def test_mla_workspace_holds_the_larger_plans_partials(lib, R, splits):
    """The sparse-MLA workspace holds fp16 split averages (96 heads x 512) and fp32 (m, l)
    for the split count of the plan that splits more, FP8 latents (which may take the
    four-wave kernel: 5 splits at 32 rows, 3 at 96) or NVFP4 latents (the eight-wave
    kernel: 8 at 32 rows, 4 at 96); unsplit rows need no partials."""
    def a256(x):
        return (x + 255) // 256 * 256
    want = 256 if splits == 1 else a256(R * splits * 96 * 512 * 2) + a256(R * splits * 96 * 2 * 4)
    assert dsa.dsa_workspace_bytes(dsa.DSA_OP_SPARSE_MLA, R, 0, 2048) == want


def _desc(**over):
    d = dsa.CacheDesc()
    d.pool = 0x10000
    d.row_bytes = 45568
    d.num_blocks = 128
    d.block_size = 64
    d.num_layers = 1
    d.index_fmt = 0
    d.lat_off[0] = 0
    d.idx_off[0] = 37120
    for k, v in over.items():
        setattr(d, k, v)
    return d


FAKE = 0x20000   # never dereferenced: every call below fails validation first


def _score(lib, d, **kw):
    a = dict(layer=0, q=FAKE, qs=FAKE, w=FAKE, bt=FAKE, stride=128, rs=FAKE, rc=FAKE, R=1, max_ctx=8192,
             scores=FAKE, ld=8192)
    a.update(kw)
    return lib.dsa_indexer_score(ctypes.byref(d) if d is not None else None, a["layer"], a["q"], a["qs"], a["w"],
                                 a["bt"], a["stride"], a["rs"], a["rc"], a["R"], a["max_ctx"], a["scores"], a["ld"],
                                 None)


@pytest.mark.parametrize("over,kw,status", [
    ({}, dict(layer=1), 2),                                 # layer out of range
    ({"block_size": 48}, {}, 3),                            # not a power of two
    ({"row_bytes": 45560}, {}, 5),                          # row not a multiple of 16
    ({"idx_off": (ctypes.c_int64 * 64)(*([45000] + [0] * 63))}, {}, 3),   # index page past the row end
    ({"pool": 0x10008}, {}, 5),                             # misaligned pool
    ({"index_fmt": 7}, {}, 7),
    ({"latent_fmt": 2}, {}, 7),                             # unknown latent format
    ({"latent_fmt": 1, "row_bytes": 22784 + 8448 - 16, "idx_off": (ctypes.c_int64 * 64)(*([22784] + [0] * 63))},
     {}, 3),                                                # NVFP4 latent page 64 x 356 B, index page one short
    ({}, dict(q=None), 1),
    ({}, dict(max_ctx=128 * 64 + 1), 2),                    # beyond block-table capacity
    ({}, dict(ld=100), 2),
    ({}, dict(R=-1), 2),
    ({"num_layers": 0}, {}, 3),
])
def test_indexer_rejects_bad_arguments(lib, over, kw, status):
    st = _score(lib, _desc(**over), **kw)
    assert st == status, dsa.load_library().dsa_last_error_detail()
    assert lib.dsa_last_error_detail().decode() != ""


def test_null_descriptor(lib):
    assert _score(lib, None) == 1


def test_device_status_rejects_null(lib):
    assert lib.dsa_device_status(None, 1, None) == 1
    assert "status" in lib.dsa_last_error_detail().decode()


def test_hbm_read_probe_rejects_bad_arguments(lib):
    assert lib.dsa_hbm_read_probe(None, 1024, FAKE, 64, None) == 1      # NULL buffer
    assert lib.dsa_hbm_read_probe(FAKE, 1000, FAKE, 64, None) == 5      # bytes % 16
    assert lib.dsa_hbm_read_probe(FAKE, 1024, FAKE, 0, None) == 2       # grid < 1
    assert lib.dsa_hbm_read_probe(FAKE, 0, FAKE, 64, None) == 0         # nothing to read, no launch


def test_topk_and_mla_reject_bad_arguments(lib):
    ws = dsa.dsa_workspace_bytes(dsa.DSA_OP_TOPK, 1, 8192, 2048)
    assert lib.dsa_topk(FAKE, 8192, FAKE, 1, 8192, 0, FAKE, FAKE, ws, None) == 2          # k = 0
    assert lib.dsa_topk(FAKE, 8192, FAKE, 1, 8192, 2049, FAKE, FAKE, ws, None) == 2       # k > 2048
    assert lib.dsa_topk(FAKE, 8192, FAKE, 1, 8192, 2048, FAKE, FAKE, ws - 1, None) == 4   # workspace
    assert lib.dsa_topk(FAKE, 100, FAKE, 1, 8192, 2048, FAKE, FAKE, ws, None) == 2        # ld < max_ctx
    assert lib.dsa_topk(None, 8192, FAKE, 1, 8192, 2048, FAKE, FAKE, ws, None) == 1
    d = _desc()
    mws = dsa.dsa_workspace_bytes(dsa.DSA_OP_SPARSE_MLA, 1, 0, 2048)
    assert lib.dsa_sparse_mla(ctypes.byref(d), 0, FAKE, FAKE, 128, FAKE, FAKE, 1, 2048, 0.04, FAKE, FAKE, FAKE,
                              mws - 1, None) == 4
    assert lib.dsa_sparse_mla(ctypes.byref(d), 0, FAKE + 8, FAKE, 128, FAKE, FAKE, 1, 2048, 0.04, FAKE, FAKE,
                              FAKE, mws, None) == 5                                       # misaligned q_lat
    dws = dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, 1, 8192, 2048)
    assert lib.dsa_decode_step(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1, 8192, 2048,
                               0.04, FAKE, FAKE, FAKE, FAKE, dws - 256, None) == 4
    assert lib.dsa_decode_step(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1, 8192, 3000,
                               0.04, FAKE, FAKE, FAKE, FAKE, dws, None) == 2


def test_multi_and_append_reject_bad_arguments(lib):
    d = _desc()
    dws = dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, 1, 8192, 2048)
    assert lib.dsa_decode_step_multi(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1, 8192,
                                     2048, 0, 0.04, FAKE, FAKE, FAKE, FAKE, dws, None) == 2   # rows_per_seq 0
    assert lib.dsa_indexer_score_multi(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1, 8192, 0,
                                       FAKE, 8192, None) == 2
    assert lib.dsa_cache_append(ctypes.byref(d), 0, FAKE, 128, FAKE, FAKE, None, None, 1, None) == 1  # no input
    assert lib.dsa_cache_append(ctypes.byref(d), 0, None, 128, FAKE, FAKE, FAKE, None, 1, None) == 1
    assert lib.dsa_cache_append(ctypes.byref(d), 0, FAKE, 128, FAKE, FAKE, FAKE + 2, None, 1, None) == 5
    assert lib.dsa_cache_append(ctypes.byref(d), 0, FAKE, 0, FAKE, FAKE, FAKE, None, 1, None) == 2
    assert lib.dsa_cache_append(ctypes.byref(d), 0, FAKE, 128, FAKE, FAKE, FAKE, None, -1, None) == 2
    assert lib.dsa_cache_append(ctypes.byref(d), 0, FAKE, 128, FAKE, FAKE, FAKE, None, 0, None) == 0   # nothing to do
    assert lib.dsa_cache_append(ctypes.byref(d), 5, FAKE, 128, FAKE, FAKE, FAKE, None, 1, None) != 0   # no layer 5


def test_dcp_merge_rejects_bad_arguments(lib):
    ws = lib.dsa_topk_dcp_workspace_bytes(2, 40000, 2048, 4)
    assert ws > 0
    assert lib.dsa_topk_dcp_workspace_bytes(2, 40000, 2048, 1) == 0     # one shard is no split
    assert lib.dsa_topk_dcp_workspace_bytes(2, 40000, 2048, 33) == 0    # mask holds 32 shards
    assert lib.dsa_topk_dcp_workspace_bytes(2, 40000, 0, 4) == 0
    # grows with the shards' candidate lists and with the context
    assert lib.dsa_topk_dcp_workspace_bytes(2, 80000, 2048, 4) > ws
    call = lambda R, mc, k, W, w=ws, p=FAKE: lib.dsa_topk_dcp(p, 40000, FAKE, R, mc, k, W, FAKE, None, None, FAKE, w, None)
    assert call(2, 40000, 2048, 1) == 2
    assert call(2, 40000, 2048, 33) == 2
    assert call(20000, 40000, 2048, 4) == 2        # R * W above 65535
    assert call(2, 40000, 0, 4) == 2
    assert call(2, 40000, 2049, 4) == 2
    assert call(2, 50000, 2048, 4) == 2            # ld 40000 < max_ctx
    assert call(2, 40000, 2048, 4, w=ws - 1) == 4
    assert call(2, 40000, 2048, 4, p=None) == 1
    assert call(0, 40000, 2048, 4, w=lib.dsa_topk_dcp_workspace_bytes(0, 40000, 2048, 4)) == 0  # nothing to do


def test_binding_refuses_cpu_tensors(lib):
    import torch
    pool = torch.zeros((4, 45568), dtype=torch.uint8)
    with pytest.raises(ValueError):
        dsa.make_cache_desc(pool, dict(row_bytes=45568, block_size=64, num_layers=1, index_fmt="fp8",
                                       lat_off=[0], idx_off=[37120]))


def test_accounting_matches_oracle_byte_definition():
    from oracle import dsa_oracle as O
    from sparse_attention_decode_paged_amd import accounting as A
    for ctx in (100, 8192, 262144, 1 << 20):
        # the library's accounting adds query/output bytes and the 4-byte latent scale on
        # top of the pages' per-token figures; the token terms must agree with the oracle's
        tok = A.indexer_bytes(ctx) - A.Q_IDX + A.attention_bytes(ctx, 2048) - A.Q_LAT - A.OUT - 4 * 2048
        assert tok == O.dsa_layer_bytes(ctx, 2048) + 4 * min(2048, ctx)
