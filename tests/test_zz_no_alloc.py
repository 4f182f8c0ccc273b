"""The allocation-free decode step (dsa_decode_step_noalloc, for callers that cannot
allocate device memory): through the C ABI it gives the same bytes as dsa_decode_step
with a caller workspace, on two calls in a row, the second with a smaller input (the
static scratch keeps the first call's contents); a call needing more scratch than the
array holds is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

from synth import make_case

pytestmark = pytest.mark.gpu

dsa = pytest.importorskip("sparse_attention_decode_paged_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.load_library()
    return torch.device("cuda:0")


def _step_with_workspace(c):
    idx, out, lse, _ = dsa.dsa_decode_step(c.pool, c.layout, 0, c.q_idx[0], c.q_idx_scale[0], c.w[0], c.q_lat[0],
                                           c.block_table, c.row_seq, c.row_ctx, c.max_ctx, c.k, c.sm_scale)
    return idx, out, lse


def _step_noalloc(c):
    """Straight through ctypes: the C entry point with no workspace argument."""
    L = dsa.load_library()
    R = c.num_rows
    idx = torch.full((R, c.k), -7, dtype=torch.int32, device=c.pool.device)
    out = torch.full((R, 96, 512), float("nan"), dtype=torch.float32, device=c.pool.device)
    lse = torch.full((R, 96), float("nan"), dtype=torch.float32, device=c.pool.device)
    d = dsa.make_cache_desc(c.pool, c.layout)
    st = L.dsa_decode_step_noalloc(ctypes.byref(d), 0, c.q_idx[0].data_ptr(), c.q_idx_scale[0].data_ptr(),
                                   c.w[0].data_ptr(), c.q_lat[0].data_ptr(), c.block_table.data_ptr(),
                                   c.block_table.shape[-1], c.row_seq.data_ptr(), c.row_ctx.data_ptr(), R, c.max_ctx,
                                   c.k, 1, c.sm_scale, idx.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   torch.cuda.current_stream(c.pool.device).cuda_stream)
    assert st == 0, L.dsa_last_error_detail().decode()
    return idx, out, lse


def test_noalloc_step_equals_workspace_step_twice(dev):
    # first a batch of three rows (one long enough for the candidate top-k), then a
    # smaller single-row call on the scratch the first one left behind
    cases = [make_case([9000, 70000, 4000], block_size=64, seed=41, k=2048).to(dev),
             make_case([3000], block_size=64, seed=42, k=512).to(dev)]
    for i, c in enumerate(cases):
        print(f"case {i}: rows {c.num_rows} max ctx {c.max_ctx} k {c.k}", flush=True)
        got = _step_noalloc(c)
        want = _step_with_workspace(c)
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            assert np.array_equal(g.cpu().numpy(), w.cpu().numpy())


def test_noalloc_refuses_a_step_larger_than_the_scratch(dev):
    L = dsa.load_library()
    need = L.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, 64, 1 << 20, 2048)
    assert need > dsa.DSA_STATIC_SCRATCH_BYTES
    c = make_case([100], block_size=64, seed=43, k=64).to(dev)
    d = dsa.make_cache_desc(c.pool, c.layout)
    # 64 rows of 1M tokens: refused by size before any argument is dereferenced
    st = L.dsa_decode_step_noalloc(ctypes.byref(d), 0, c.q_idx[0].data_ptr(), c.q_idx_scale[0].data_ptr(),
                                   c.w[0].data_ptr(), c.q_lat[0].data_ptr(), c.block_table.data_ptr(),
                                   c.block_table.shape[-1], c.row_seq.data_ptr(), c.row_ctx.data_ptr(), 64, 1 << 20,
                                   2048, 1, c.sm_scale, 0x10000, 0x10000, 0x10000, None)
    assert st == 4  # DSA_ERR_WORKSPACE
    assert "static scratch" in L.dsa_last_error_detail().decode()
