"""ctypes binding of libdsa.so: same names as the C ABI in include/dsa.h.

Argument marshalling only. Torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels. There is
no fallback: if libdsa.so is missing or a tensor is not on the GPU, the call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_INDEX_FP8 = 0
DSA_INDEX_MXFP4 = 1
DSA_LATENT_FP8 = 0
DSA_LATENT_NVFP4 = 1
DSA_OP_TOPK = 1
DSA_OP_SPARSE_MLA = 2
DSA_OP_DECODE_STEP = 3
DSA_MAX_LAYERS = 64
H_IDX, D_IDX, H_Q, D_LAT, D_V = 32, 128, 96, 576, 512

EXPORTED = ("dsa_abi_version", "dsa_status_string", "dsa_last_error_detail", "dsa_workspace_bytes",
            "dsa_decode_scores_ld", "dsa_indexer_score", "dsa_topk", "dsa_sparse_mla", "dsa_decode_step",
            "dsa_indexer_score_multi", "dsa_decode_step_multi", "dsa_cache_append",
            "dsa_topk_dcp_workspace_bytes", "dsa_topk_dcp", "dsa_device_status",
            "dsa_hbm_read_probe", "dsa_decode_step_noalloc", "dsa_decode_step_stages")


class DSAError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn} failed: status {status}: {detail}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("pool", ctypes.c_void_p),
        ("row_bytes", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("index_fmt", ctypes.c_int32),
        ("latent_fmt", ctypes.c_int32),
        ("lat_off", ctypes.c_int64 * DSA_MAX_LAYERS),
        ("idx_off", ctypes.c_int64 * DSA_MAX_LAYERS),
    ]


_lib = None
_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


def load_library(path: str = LIB_PATH):
    """Load libdsa.so and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    L.dsa_abi_version.restype = _i32
    L.dsa_abi_version.argtypes = []
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_status_string.argtypes = [_i32]
    L.dsa_last_error_detail.restype = ctypes.c_char_p
    L.dsa_last_error_detail.argtypes = []
    L.dsa_workspace_bytes.restype = _sz
    L.dsa_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
    L.dsa_decode_scores_ld.restype = _i64
    L.dsa_decode_scores_ld.argtypes = [_i32]
    P = ctypes.POINTER(CacheDesc)
    L.dsa_indexer_score.restype = _i32
    L.dsa_indexer_score.argtypes = [P, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _i64, _vp]
    L.dsa_topk.restype = _i32
    L.dsa_topk.argtypes = [_vp, _i64, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp]
    L.dsa_sparse_mla.restype = _i32
    L.dsa_sparse_mla.argtypes = [P, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]
    L.dsa_decode_step.restype = _i32
    L.dsa_decode_step.argtypes = [P, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32,
                                  _vp, _vp, _vp, _vp, _sz, _vp]
    L.dsa_indexer_score_multi.restype = _i32
    L.dsa_indexer_score_multi.argtypes = [P, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _i64,
                                          _vp]
    L.dsa_cache_append.restype = _i32
    L.dsa_cache_append.argtypes = [P, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp]
    L.dsa_decode_step_multi.restype = _i32
    L.dsa_decode_step_multi.argtypes = [P, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _f32, _vp, _vp, _vp, _vp, _sz, _vp]
    L.dsa_topk_dcp_workspace_bytes.restype = _sz
    L.dsa_topk_dcp_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
    L.dsa_topk_dcp.restype = _i32
    L.dsa_topk_dcp.argtypes = [_vp, _i64, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    L.dsa_device_status.restype = _i32
    L.dsa_device_status.argtypes = [_vp, _i32, ctypes.POINTER(ctypes.c_uint32)]
    L.dsa_decode_step_noalloc.restype = _i32
    L.dsa_decode_step_noalloc.argtypes = [P, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                          _f32, _vp, _vp, _vp, _vp]
    L.dsa_decode_step_stages.restype = _i32
    L.dsa_decode_step_stages.argtypes = [P, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                         _f32, _vp, _vp, _vp, _vp, _sz, ctypes.c_uint32, _vp]
    L.dsa_hbm_read_probe.restype = _i32
    L.dsa_hbm_read_probe.argtypes = [_vp, _sz, _vp, _i32, _vp]
    _lib = L
    return L


def _check(st: int, fn: str):
    if st != 0:
        L = load_library()
        raise DSAError(st, fn, L.dsa_last_error_detail().decode())


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def make_cache_desc(pool: torch.Tensor, layout) -> CacheDesc:
    """Descriptor for a pool tensor uint8 [num_blocks, row_bytes] and a layout object
    or dict with block_size, num_layers, index_fmt ('fp8'|'mxfp4'), latent_fmt
    ('fp8'|'nvfp4', default 'fp8'), row_bytes, lat_off, idx_off."""
    get = (lambda k: layout[k]) if isinstance(layout, dict) else (lambda k: getattr(layout, k))
    has = (lambda k: k in layout) if isinstance(layout, dict) else (lambda k: hasattr(layout, k))
    d = CacheDesc()
    d.pool = _dev(pool, "pool", torch.uint8)
    d.row_bytes = int(get("row_bytes"))
    d.num_blocks = pool.numel() // d.row_bytes
    d.block_size = int(get("block_size"))
    d.num_layers = int(get("num_layers"))
    fmt = get("index_fmt")
    d.index_fmt = {"fp8": DSA_INDEX_FP8, "mxfp4": DSA_INDEX_MXFP4}.get(fmt, fmt if isinstance(fmt, int) else -1)
    lf = get("latent_fmt") if has("latent_fmt") else "fp8"
    d.latent_fmt = {"fp8": DSA_LATENT_FP8, "nvfp4": DSA_LATENT_NVFP4}.get(lf, lf if isinstance(lf, int) else -1)
    for i, v in enumerate(get("lat_off")):
        d.lat_off[i] = int(v)
    for i, v in enumerate(get("idx_off")):
        d.idx_off[i] = int(v)
    return d


def dsa_abi_version() -> int:
    return load_library().dsa_abi_version()


def dsa_status_string(status: int) -> str:
    return load_library().dsa_status_string(status).decode()


def dsa_workspace_bytes(op: int, R: int, max_ctx: int, k: int) -> int:
    return load_library().dsa_workspace_bytes(op, R, max_ctx, k)


def dsa_decode_scores_ld(max_ctx: int) -> int:
    return load_library().dsa_decode_scores_ld(max_ctx)


def _bt_stride(block_table: torch.Tensor) -> int:
    return block_table.shape[-1]


def dsa_indexer_score(pool, layout, layer, q_idx, q_idx_scale, w, block_table, row_seq, row_ctx, max_ctx,
                      scores=None, ld_scores=None, rows_per_seq=1):
    """Scores fp32 [R][ld_scores] of every token t < row_ctx[r]. rows_per_seq > 1:
    runs of that many consecutive rows share a sequence (dsa_indexer_score_multi)."""
    L = load_library()
    R = row_seq.shape[0]
    if ld_scores is None:
        ld_scores = max(int(max_ctx), 1)
    if scores is None:
        scores = torch.empty((R, ld_scores), dtype=torch.float32, device=pool.device)
    d = make_cache_desc(pool, layout)
    args = [ctypes.byref(d), layer, _dev(q_idx, "q_idx"), _dev(q_idx_scale, "q_idx_scale"),
            _dev(w, "w", torch.float32), _dev(block_table, "block_table", torch.int32),
            _bt_stride(block_table), _dev(row_seq, "row_seq", torch.int32),
            _dev(row_ctx, "row_ctx", torch.int32), R, int(max_ctx)]
    tail = [_dev(scores, "scores", torch.float32), int(ld_scores), _stream(pool.device)]
    if int(rows_per_seq) == 1:
        _check(L.dsa_indexer_score(*args, *tail), "dsa_indexer_score")
    else:
        _check(L.dsa_indexer_score_multi(*args, int(rows_per_seq), *tail), "dsa_indexer_score_multi")
    return scores


def dsa_topk(scores, row_ctx, max_ctx, k, idx=None, workspace=None, ld_scores=None):
    """Exact top-k token indices int32 [R][k] (ascending, -1 padded)."""
    L = load_library()
    R = row_ctx.shape[0]
    if ld_scores is None:
        ld_scores = scores.shape[-1]
    if idx is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=scores.device)
    need = L.dsa_workspace_bytes(DSA_OP_TOPK, R, int(max_ctx), int(k))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=scores.device)
    st = L.dsa_topk(_dev(scores, "scores", torch.float32), int(ld_scores), _dev(row_ctx, "row_ctx", torch.int32), R,
                    int(max_ctx), int(k), _dev(idx, "idx", torch.int32), _dev(workspace, "workspace"),
                    workspace.numel() * workspace.element_size(), _stream(scores.device))
    _check(st, "dsa_topk")
    return idx


DSA_DEV_CTX_CLAMPED = 1
DSA_DEV_BLOCK_CLAMPED = 2
DSA_DEV_INDEX_RANGE = 4


def dsa_device_status(device=None, clear=True):
    """The current device's status word (DSA_DEV_* bits) once the current stream's work
    has finished; cleared afterwards when `clear`. Synchronises the stream."""
    L = load_library()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    v = ctypes.c_uint32(0)
    with torch.cuda.device(dev):
        _check(L.dsa_device_status(_stream(dev), 1 if clear else 0, ctypes.byref(v)), "dsa_device_status")
    return int(v.value)


def dsa_hbm_read_probe(buf, sink, grid=2048):
    """Enqueue one streaming read of the whole tensor `buf` (measurement reference)."""
    L = load_library()
    nbytes = buf.numel() * buf.element_size()
    _check(L.dsa_hbm_read_probe(_dev(buf, "buf"), nbytes, _dev(sink, "sink"), int(grid), _stream(buf.device)),
           "dsa_hbm_read_probe")


def dcp_send_count(k, W):
    """Candidates each shard sends: ceil(1.5 k / W)."""
    return -(-3 * int(k) // (2 * int(W)))


def dsa_topk_dcp(scores, row_ctx, max_ctx, k, W, idx=None, resend_mask=None, words=None, workspace=None,
                 ld_scores=None, with_words=False):
    """Exact top-k through the emulated context-parallel merge over W token-strided shards.
    Returns (idx int32 [R][k], resend_mask int32 [R] (uint32 bits), words int32 [R][W*M] or None)."""
    L = load_library()
    R = row_ctx.shape[0]
    dev = scores.device
    if ld_scores is None:
        ld_scores = scores.shape[-1]
    if idx is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    if resend_mask is None:
        resend_mask = torch.empty((R,), dtype=torch.int32, device=dev)
    if words is None and with_words:
        words = torch.empty((R, W * dcp_send_count(k, W)), dtype=torch.int32, device=dev)
    need = L.dsa_topk_dcp_workspace_bytes(R, int(max_ctx), int(k), int(W))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = L.dsa_topk_dcp(_dev(scores, "scores", torch.float32), int(ld_scores), _dev(row_ctx, "row_ctx", torch.int32),
                        R, int(max_ctx), int(k), int(W), _dev(idx, "idx", torch.int32),
                        _dev(resend_mask, "resend_mask", torch.int32), _dev(words, "words", torch.int32),
                        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "dsa_topk_dcp")
    return idx, resend_mask, words


def dsa_sparse_mla(pool, layout, layer, q_lat, block_table, row_seq, idx, k, sm_scale, out=None, lse=None,
                   workspace=None):
    """Sparse MLA over idx: out fp32 [R][96][512], lse fp32 [R][96]."""
    L = load_library()
    R = row_seq.shape[0]
    dev = pool.device
    if out is None:
        out = torch.empty((R, H_Q, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((R, H_Q), dtype=torch.float32, device=dev)
    need = L.dsa_workspace_bytes(DSA_OP_SPARSE_MLA, R, 0, int(k))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    d = make_cache_desc(pool, layout)
    st = L.dsa_sparse_mla(ctypes.byref(d), layer, _dev(q_lat, "q_lat", torch.bfloat16),
                          _dev(block_table, "block_table", torch.int32), _bt_stride(block_table),
                          _dev(row_seq, "row_seq", torch.int32), _dev(idx, "idx", torch.int32), R, int(k),
                          float(sm_scale), _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32),
                          _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "dsa_sparse_mla")
    return out, lse


def dsa_decode_step(pool, layout, layer, q_idx, q_idx_scale, w, q_lat, block_table, row_seq, row_ctx, max_ctx, k,
                    sm_scale, idx=None, out=None, lse=None, workspace=None, rows_per_seq=1):
    """Indexer -> exact top-k -> sparse MLA -> merge. Returns (idx, out, lse, workspace);
    the scores sit at the start of the workspace with row stride dsa_decode_scores_ld(max_ctx).
    rows_per_seq > 1: runs of that many consecutive rows share a sequence (dsa_decode_step_multi)."""
    L = load_library()
    R = row_seq.shape[0]
    dev = pool.device
    if idx is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((R, H_Q, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((R, H_Q), dtype=torch.float32, device=dev)
    need = L.dsa_workspace_bytes(DSA_OP_DECODE_STEP, R, int(max_ctx), int(k))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    d = make_cache_desc(pool, layout)
    head = [ctypes.byref(d), layer, _dev(q_idx, "q_idx"), _dev(q_idx_scale, "q_idx_scale"),
            _dev(w, "w", torch.float32), _dev(q_lat, "q_lat", torch.bfloat16),
            _dev(block_table, "block_table", torch.int32), _bt_stride(block_table),
            _dev(row_seq, "row_seq", torch.int32), _dev(row_ctx, "row_ctx", torch.int32), R, int(max_ctx), int(k)]
    tail = [_dev(idx, "idx", torch.int32), _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(dev)]
    if int(rows_per_seq) == 1:
        _check(L.dsa_decode_step(*head, float(sm_scale), *tail), "dsa_decode_step")
    else:
        _check(L.dsa_decode_step_multi(*head, int(rows_per_seq), float(sm_scale), *tail), "dsa_decode_step_multi")
    return idx, out, lse, workspace


DSA_STATIC_SCRATCH_BYTES = 32 << 20


def dsa_decode_step_noalloc(pool, layout, layer, q_idx, q_idx_scale, w, q_lat, block_table, row_seq, row_ctx, max_ctx,
                            k, sm_scale, idx=None, out=None, lse=None, rows_per_seq=1):
    """The decode step on the library's static per-GPU scratch (no workspace argument):
    returns (idx, out, lse). Calls that overlap on one GPU race (shared scratch)."""
    L = load_library()
    R = row_seq.shape[0]
    dev = pool.device
    if idx is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((R, H_Q, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((R, H_Q), dtype=torch.float32, device=dev)
    d = make_cache_desc(pool, layout)
    st = L.dsa_decode_step_noalloc(ctypes.byref(d), layer, _dev(q_idx, "q_idx"), _dev(q_idx_scale, "q_idx_scale"),
                                   _dev(w, "w", torch.float32), _dev(q_lat, "q_lat", torch.bfloat16),
                                   _dev(block_table, "block_table", torch.int32), _bt_stride(block_table),
                                   _dev(row_seq, "row_seq", torch.int32), _dev(row_ctx, "row_ctx", torch.int32), R,
                                   int(max_ctx), int(k), int(rows_per_seq), float(sm_scale),
                                   _dev(idx, "idx", torch.int32), _dev(out, "out", torch.float32),
                                   _dev(lse, "lse", torch.float32), _stream(dev))
    _check(st, "dsa_decode_step_noalloc")
    return idx, out, lse


DSA_STAGE_INDEXER, DSA_STAGE_TOPK, DSA_STAGE_ATTENTION, DSA_STAGE_MERGE, DSA_STAGE_ALL = 1, 2, 4, 8, 15


def dsa_decode_step_stages(pool, layout, layer, q_idx, q_idx_scale, w, q_lat, block_table, row_seq, row_ctx, max_ctx,
                           k, sm_scale, idx, out, lse, workspace, stages, rows_per_seq=1):
    """Enqueue only the chosen stages (DSA_STAGE_* bits) of a decode step on `workspace`
    (a measurement entry point: each kernel of the step timed alone)."""
    L = load_library()
    R = row_seq.shape[0]
    dev = pool.device
    d = make_cache_desc(pool, layout)
    st = L.dsa_decode_step_stages(ctypes.byref(d), layer, _dev(q_idx, "q_idx"), _dev(q_idx_scale, "q_idx_scale"),
                                  _dev(w, "w", torch.float32), _dev(q_lat, "q_lat", torch.bfloat16),
                                  _dev(block_table, "block_table", torch.int32), _bt_stride(block_table),
                                  _dev(row_seq, "row_seq", torch.int32), _dev(row_ctx, "row_ctx", torch.int32), R,
                                  int(max_ctx), int(k), int(rows_per_seq), float(sm_scale),
                                  _dev(idx, "idx", torch.int32), _dev(out, "out", torch.float32),
                                  _dev(lse, "lse", torch.float32), _dev(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), int(stages), _stream(dev))
    _check(st, "dsa_decode_step_stages")


def dsa_cache_append(pool, layout, layer, block_table, row_seq, pos, idx_key=None, latent=None):
    """Quantise and write each row's new index key (fp32 [R][128]) and / or latent
    (fp32 [R][576]) at token pos[r] of block-table row row_seq[r] (in place)."""
    L = load_library()
    R = row_seq.shape[0]
    d = make_cache_desc(pool, layout)
    st = L.dsa_cache_append(ctypes.byref(d), layer, _dev(block_table, "block_table", torch.int32),
                            _bt_stride(block_table), _dev(row_seq, "row_seq", torch.int32),
                            _dev(pos, "pos", torch.int32),
                            _dev(idx_key, "idx_key", torch.float32) if idx_key is not None else None,
                            _dev(latent, "latent", torch.float32) if latent is not None else None,
                            R, _stream(pool.device))
    _check(st, "dsa_cache_append")
    return pool


def decode_scores_view(workspace: torch.Tensor, R: int, max_ctx: int) -> torch.Tensor:
    """The fp32 score array [R][ld] kept at the start of a decode-step workspace."""
    ld = dsa_decode_scores_ld(max_ctx)
    return workspace[:R * ld * 4].view(torch.float32).view(R, ld)
