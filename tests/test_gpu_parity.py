"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded bytes.

Bars:
* scores: |gpu - oracle| <= 2e-5 * sum_h |w_h| sum_d |q_hd k_td|. The kernel sums
  128 exact code products in fp32, scales by fp32 factors and adds 32 weighted
  heads in fp32; (128 + 32 + a few) roundings of 2^-24 bound the error by
  ~1e-5 of that magnitude.
* top-k: bit-exact against the oracle's selection rule applied to the GPU's
  own fp32 scores; against the oracle's scores, the two sets may differ only in
  tokens within 1e-4 * |s_(k)| of the k-th score.
* attention (on the GPU's own index set): |gpu - oracle| <= 2e-3 + 1e-2 * |oracle|
  for out and lse.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from synth import (make_case, make_prefill_case, config_small, config_batch16, config_long_1m,
                   config_prefill_append, config_mixed_mxfp4)

pytestmark = pytest.mark.gpu

dsa = pytest.importorskip("sparse_attention_decode_paged_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.load_library()          # raises if the HIP library is missing
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def run_step(case, dev, layer=0, k=None, rows_per_seq=1):
    g = case if case.pool.is_cuda else case.to(dev)
    k = case.k if k is None else k
    R = g.num_rows
    idx, out, lse, ws = dsa.dsa_decode_step(g.pool, g.layout, layer, g.q_idx[layer], g.q_idx_scale[layer], g.w[layer],
                                            g.q_lat[layer], g.block_table, g.row_seq, g.row_ctx, case.max_ctx, k,
                                            case.sm_scale, rows_per_seq=rows_per_seq)
    torch.cuda.synchronize()
    scores = dsa.decode_scores_view(ws, R, case.max_ctx).cpu().numpy().copy()
    return scores, idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


class HostCase:
    """Host copies of a case for the oracle."""

    def __init__(self, case):
        self.c = case
        self.pool = case.pool.cpu().numpy()
        self.bt = case.block_table.cpu().numpy()
        self.row_seq = case.row_seq.cpu().numpy()
        self.row_ctx = case.row_ctx.cpu().numpy()
        self.q_idx = case.q_idx.cpu().numpy()
        self.q_sc = case.q_idx_scale.cpu().numpy()
        self.w = case.w.cpu().numpy()
        self.q_lat = case.q_lat.cpu().view(torch.int16).numpy().view(np.uint16)

    def oracle(self, r, layer=0, k=None, want_magnitude=True):
        k = self.c.k if k is None else k
        return O.decode_row(self.pool, self.c.layout, layer, self.bt[self.row_seq[r]], int(self.row_ctx[r]),
                            self.q_idx[layer, r], self.q_sc[layer, r], self.w[layer, r], self.q_lat[layer, r], k,
                            self.c.sm_scale, want_magnitude=want_magnitude)

    def attend(self, r, tokens, layer=0):
        lat = O.read_latents(self.pool, O.Layout(self.c.layout), layer, self.bt[self.row_seq[r]], tokens)
        return O.sparse_mla(O.bf16_to_f64(self.q_lat[layer, r]), lat, self.c.sm_scale)


def check_scores(gs, ref, ctx):
    err = np.abs(gs[:ctx].astype(np.float64) - ref["scores"])
    bound = 2e-5 * ref["mag"] + 1e-30
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"{bad.size} scores off, worst ratio {np.max(err / bound):.3g} at t={bad[:5]}"


def check_selection(gs, gidx, ref, ctx, k):
    total = min(k, ctx)
    assert np.all(gidx[total:] == -1), "padding"
    sel = gidx[:total]
    assert np.all(sel >= 0) and np.all(np.diff(sel) > 0), "not ascending / duplicates"
    assert np.array_equal(sel, O.select_topk(gs[:ctx], k)), "top-k differs from exact selection on GPU scores"
    if total:
        s_k = ref["scores"][ref["idx"]].min()
        diff = np.setxor1d(sel, ref["idx"])
        if diff.size:
            far = np.abs(ref["scores"][diff] - s_k) > 1e-4 * abs(s_k)
            assert not far.any(), f"{far.sum()} set differences outside the tie band"
    return sel


def check_attention(hc, r, sel, gout, glse, layer=0):
    out, lse = hc.attend(r, sel, layer)
    e = np.abs(gout - out)
    assert np.all(e <= 2e-3 + 1e-2 * np.abs(out)), f"out max abs err {e.max():.3g}"
    if sel.size == 0:
        assert np.all(np.isneginf(glse)) and np.all(gout == 0)
    else:
        el = np.abs(glse - lse)
        assert np.all(el <= 2e-3 + 1e-2 * np.abs(lse)), f"lse max err {el.max():.3g}"
    return float(e.max()) if e.size else 0.0


def full_check(case, dev, rows=None, layer=0):
    hc = HostCase(case)
    scores, idx, out, lse = run_step(case, dev, layer)
    rows = range(case.num_rows) if rows is None else rows
    for r in rows:
        ctx = int(hc.row_ctx[r])
        say(f"  row {r} ctx {ctx}")
        ref = hc.oracle(r, layer)
        check_scores(scores[r], ref, ctx)
        sel = check_selection(scores[r], idx[r], ref, ctx, case.k)
        check_attention(hc, r, sel, out[r], lse[r], layer)
    return scores, idx, out, lse


# ----------------------------------------------------------------------------- cases
def test_small_decode_8k(dev):
    say("case: decode B=1 ctx 8192 bs 64 k 2048 seed 0")
    full_check(config_small(), dev)


@pytest.mark.parametrize("bs", [8, 16, 32, 128, 256])
def test_block_sizes_ragged(dev, bs):
    say(f"case: ragged rows bs {bs}")
    c = make_case([1, 5, 100, 2047, 2048, 2049, 4100, 9000], block_size=bs, seed=bs, k=2048)
    full_check(c, dev)


@pytest.mark.parametrize("k", [1, 7, 64, 100, 2000])
def test_small_k(dev, k):
    say(f"case: k {k}")
    c = make_case([5000, 64, 3], block_size=64, seed=100 + k, k=k)
    full_check(c, dev)


def test_empty_rows(dev):
    say("case: empty rows")
    c = make_case([0, 300, 0], block_size=64, seed=7, k=128)
    scores, idx, out, lse = full_check(c, dev)
    assert np.all(idx[0] == -1) and np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("ctx", [10000, 40000])
def test_constant_scores_ties(dev, ctx):
    """All index keys zero -> every score is 0: the first k tokens win (ties to the
    lower index); 40000 ties overflow the candidate list and take the rescan path."""
    say(f"case: constant scores ctx {ctx}")
    c = make_case([ctx], block_size=64, seed=3, k=2048)
    lay = c.layout
    c.pool[:, lay.idx_off[0]:lay.idx_off[0] + lay.block_size * 128] = 0
    scores, idx, out, lse = full_check(c, dev)
    assert np.all(scores[0, :ctx] == 0)
    assert np.array_equal(idx[0], np.arange(2048))


def test_determinism_and_staged_calls(dev):
    say("case: determinism + staged vs fused, B=3")
    c = make_case([9000, 20000, 4000], block_size=64, seed=21, k=2048).to(dev)
    a = run_step(c, dev)
    b = run_step(c, dev)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    # staged: indexer -> topk -> sparse_mla through the three separate entry points
    s = dsa.dsa_indexer_score(c.pool, c.layout, 0, c.q_idx[0], c.q_idx_scale[0], c.w[0], c.block_table, c.row_seq,
                              c.row_ctx, c.max_ctx)
    i = dsa.dsa_topk(s, c.row_ctx, c.max_ctx, c.k)
    o, l = dsa.dsa_sparse_mla(c.pool, c.layout, 0, c.q_lat[0], c.block_table, c.row_seq, i, c.k, c.sm_scale)
    torch.cuda.synchronize()
    for r in range(3):
        ctx = int(c.row_ctx[r])
        assert np.array_equal(s[r, :ctx].cpu().numpy(), a[0][r, :ctx])
    assert np.array_equal(i.cpu().numpy(), a[1])
    assert np.array_equal(o.cpu().numpy(), a[2]) and np.array_equal(l.cpu().numpy(), a[3])


@pytest.mark.parametrize("ctxs", [[200000], [70000, 30000], [9000]])
def test_stages_equal_step(dev, ctxs):
    """The step runs the select and the attention as one launch for these batches; the
    stage-by-stage launches (indexer, select, attention + merge: separate kernels) must
    give the same scores, indices, output and lse bit for bit."""
    say(f"case: staged launches vs the step, ctx {ctxs}")
    c = make_case(ctxs, block_size=64, seed=41, k=2048).to(dev)
    s_f, i_f, o_f, l_f = run_step(c, dev)
    R = c.num_rows
    ws = torch.empty(dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, R, c.max_ctx, c.k), dtype=torch.uint8,
                     device=dev)
    idx = torch.empty((R, c.k), dtype=torch.int32, device=dev)
    out = torch.empty((R, 96, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, 96), dtype=torch.float32, device=dev)
    for bits in (dsa.DSA_STAGE_INDEXER, dsa.DSA_STAGE_TOPK, dsa.DSA_STAGE_ATTENTION | dsa.DSA_STAGE_MERGE):
        dsa.dsa_decode_step_stages(c.pool, c.layout, 0, c.q_idx[0], c.q_idx_scale[0], c.w[0], c.q_lat[0],
                                   c.block_table, c.row_seq, c.row_ctx, c.max_ctx, c.k, c.sm_scale, idx, out, lse,
                                   ws, bits)
    torch.cuda.synchronize()
    s_s = dsa.decode_scores_view(ws, R, c.max_ctx).cpu().numpy()
    for r in range(R):
        ctx = int(c.row_ctx[r])
        assert np.array_equal(s_s[r, :ctx], s_f[r, :ctx])
    assert np.array_equal(idx.cpu().numpy(), i_f)
    assert np.array_equal(out.cpu().numpy(), o_f) and np.array_equal(lse.cpu().numpy(), l_f)


@pytest.mark.parametrize("ctxs", [[100000, 40000]])
def test_planted_rescans_staged_and_fused(dev, ctxs):
    """Rows whose top 2,048 crowd into a few units: 2,048 elevated keys log-uniform over each
    row, so the first units hold far more of them than they send and the select rescans
    those units from the scores (256-token units at 100,000 tokens, 64-token units at
    40,000). The step (select and attention in one launch) is checked against the oracle,
    and the staged launches (the standalone select) must equal it bit for bit."""
    say(f"case: planted keys, rescanned units, ctx {ctxs}")
    c = make_case(ctxs, block_size=64, seed=43, k=2048, plant=2048).to(dev)
    s_f, i_f, o_f, l_f = full_check(c, dev)
    for r in range(c.num_rows):
        planted = np.array(c.planted[(0, r)])
        hit = np.intersect1d(planted, i_f[r]).size
        say(f"  row {r}: planted selected {hit}/{planted.size}")
    R = c.num_rows
    ws = torch.empty(dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, R, c.max_ctx, c.k), dtype=torch.uint8,
                     device=dev)
    idx = torch.empty((R, c.k), dtype=torch.int32, device=dev)
    out = torch.empty((R, 96, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, 96), dtype=torch.float32, device=dev)
    for bits in (dsa.DSA_STAGE_INDEXER, dsa.DSA_STAGE_TOPK, dsa.DSA_STAGE_ATTENTION | dsa.DSA_STAGE_MERGE):
        dsa.dsa_decode_step_stages(c.pool, c.layout, 0, c.q_idx[0], c.q_idx_scale[0], c.w[0], c.q_lat[0],
                                   c.block_table, c.row_seq, c.row_ctx, c.max_ctx, c.k, c.sm_scale, idx, out, lse,
                                   ws, bits)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), i_f)
    assert np.array_equal(out.cpu().numpy(), o_f) and np.array_equal(lse.cpu().numpy(), l_f)


def test_batch_invariance(dev):
    """A row's scores and selection do not depend on the batch it runs in (bit for bit).
    Its attention output may: sparse MLA splits a row's tokens into a number of splits
    chosen from the batch size, and each split rounds its probabilities to fp16 against
    its own running maximum, so outputs agree to that rounding (2^-11 relative per
    probability), well inside the parity bar."""
    say("case: batch invariance")
    c = make_case([30000, 17000, 50000, 2500], block_size=64, seed=31, k=2048).to(dev)
    s_all, i_all, o_all, l_all = run_step(c, dev)
    for r in range(4):
        one = type(c)(c.name, c.layout, c.pool, c.block_table, c.row_seq[r:r + 1].contiguous(),
                      c.row_ctx[r:r + 1].contiguous(), c.q_idx[:, r:r + 1].contiguous(),
                      c.q_idx_scale[:, r:r + 1].contiguous(), c.w[:, r:r + 1].contiguous(),
                      c.q_lat[:, r:r + 1].contiguous(), c.k, c.sm_scale)
        s1, i1, o1, l1 = run_step(one, dev)
        ctx = int(c.row_ctx[r])
        assert np.array_equal(s1[0, :ctx], s_all[r, :ctx])
        assert np.array_equal(i1[0], i_all[r])
        err = np.abs(o1[0] - o_all[r])
        say(f"  row {r}: attention max abs diff across batch sizes {err.max():.3g}")
        assert np.all(err <= 1e-4 + 1e-3 * np.abs(o_all[r]))


def test_batch16_mixed_lengths(dev):
    say("case: decode B=16 ctx U[16K,64K] shared shuffled pool")
    c = config_batch16(device=dev)
    full_check(c, dev)


@pytest.mark.parametrize("bs", [16, 128])
def test_mxfp4_keys_ragged(dev, bs):
    """MXFP4 index keys (bs 16: per-token key gathers; bs 128: page-contiguous tiles); rows
    below, at and above k, and two long enough for the candidate top-k."""
    say(f"case: mxfp4 keys, bs {bs}")
    c = make_case([1, 700, 2048, 2049, 9000, 20000, 70000], block_size=bs, seed=70 + bs, k=2048, index_fmt="mxfp4")
    full_check(c, dev)


def test_mxfp4_mixed_batch_layers(dev):
    """The mixed-length MXFP4 workload at reduced size: B=8, lengths log-uniform in [4K, 256K],
    3 layers in one packed row, bs 128; every row checked on the last layer."""
    say("case: mxfp4 B=8 log-uniform [4K, 256K], 3 layers, bs 128")
    c = config_mixed_mxfp4(device=dev, batch=8, num_layers=3)
    full_check(c, dev, layer=2)


def test_long_context_1m_planted(dev):
    say("case: decode B=1 ctx 1,048,576 with 2048 planted keys")
    c = config_long_1m(device=dev)
    scores, idx, out, lse = full_check(c, dev)
    planted = np.array(c.planted[(0, 0)])
    hit = np.intersect1d(planted, idx[0]).size
    say(f"  planted selected: {hit}/{planted.size}")
    assert hit >= 0.95 * planted.size


def test_decode_256k_24_layers_graph_replay(dev):
    """The 262,144-token decode step in the form the benchmark times it: 24 layers in one
    packed cache row, the step for every layer captured in one HIP graph on a side stream
    and replayed. Every replay is compared bit for bit with eager calls (eager work and
    synchronisations between replays), and two layers are checked against the oracle in full
    (all 262,144 scores, the selection, all 96 heads)."""
    L, ctx = 24, 262144
    say(f"case: decode B=1 ctx {ctx}, {L} layers, bs 64, graph replay")
    c = make_case([ctx], block_size=64, num_layers=L, seed=0, device=dev, k=2048,
                  name="decode_b1_ctx262144_x24layers")
    R, K, M = c.num_rows, c.k, c.max_ctx     # M read once: no device sync may run under capture
    ws = torch.empty(dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, R, M, K), dtype=torch.uint8, device=dev)
    bufs = [(torch.empty((R, K), dtype=torch.int32, device=dev), torch.empty((R, 96, 512), device=dev),
             torch.empty((R, 96), device=dev)) for _ in range(L)]

    def step(l, b):
        dsa.dsa_decode_step(c.pool, c.layout, l, c.q_idx[l], c.q_idx_scale[l], c.w[l], c.q_lat[l], c.block_table,
                            c.row_seq, c.row_ctx, M, K, c.sm_scale, idx=b[0], out=b[1], lse=b[2], workspace=ws)

    check_layers = (0, L - 1)
    eager, eager_scores = [], {}
    for l in range(L):
        step(l, bufs[l])
        if l in check_layers:
            eager_scores[l] = dsa.decode_scores_view(ws, R, M).cpu().numpy().copy()
        eager.append(tuple(x.cpu().numpy().copy() for x in bufs[l]))
    torch.cuda.synchronize()

    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for l in range(L):
            step(l, bufs[l])
    torch.cuda.synchronize()
    scratch = tuple(torch.empty_like(x) for x in bufs[0])
    for rep in range(3):
        for b in bufs:
            for x in b:
                x.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            for got, want in zip(bufs[l], eager[l]):
                assert np.array_equal(got.cpu().numpy(), want), f"replay {rep} layer {l} differs from eager"
        step((rep * 7) % L, scratch)        # eager work between replays
        torch.cuda.synchronize()
    say("  3 replays bit-identical to eager")

    hc = HostCase(c)
    for l in check_layers:
        say(f"  oracle layer {l}")
        ref = hc.oracle(0, l)
        check_scores(eager_scores[l][0], ref, ctx)
        sel = check_selection(eager_scores[l][0], eager[l][0][0], ref, ctx, K)
        check_attention(hc, 0, sel, eager[l][1][0], eager[l][2][0], l)


@pytest.mark.timeout(900)
def test_prefill_append_150k(dev):
    """2048 appended rows on a 150,000-token prefix (row r sees t <= 150000 + r), run as the
    benchmark times it: rows_per_seq = 2048, i.e. the row-group indexer with 16 rows per
    group and 256-token send units. The result must equal the row-by-row path byte for
    byte; 40 rows, among them all 16 rows of the first and of the last row group, are
    checked against the oracle in full."""
    say("case: prefill-append 2048 rows on 150000 prefix, rows_per_seq 2048 and 1")
    c = config_prefill_append(device=dev)
    hc = HostCase(c)
    R = c.num_rows
    scores, idx, out, lse = run_step(c, dev, rows_per_seq=R)
    say("  row-group path done; row-by-row path")
    a = run_step(c, dev, rows_per_seq=1)
    for r in range(R):
        ctx = 150000 + r + 1
        assert hc.row_ctx[r] == ctx
        assert np.array_equal(a[0][r, :ctx], scores[r, :ctx]), f"scores row {r}"
        row = idx[r]
        assert row.min() >= 0 and row.max() < ctx and np.all(np.diff(row) > 0)
    for x, y in zip(a[1:], (idx, out, lse)):
        assert np.array_equal(x, y)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(0)
    sample = sorted(set(range(16)) | set(range(R - 16, R)) | set(rng.integers(16, R - 16, 8).tolist()))
    assert len(sample) >= 32
    for r in sample:
        say(f"  oracle row {r}")
        ref = hc.oracle(r)
        ctx = int(hc.row_ctx[r])
        check_scores(scores[r], ref, ctx)
        sel = check_selection(scores[r], idx[r], ref, ctx, c.k)
        check_attention(hc, r, sel, out[r], lse[r])


@pytest.mark.timeout(1200)
def test_mixed_mxfp4_b64_24_layers_full_size(dev):
    """The batch-64 workload at its stated size: 64 rows, lengths log-uniform in
    [4096, 262144], 24 layers in one packed row (about 62 GB of cache), block size 128,
    MXFP4 index keys. Layers 0, 11 and 23 run and every row of each is checked against the
    oracle (only that layer's pages travel to the host)."""
    say("case: mxfp4 B=64 log-uniform [4K, 256K], 24 layers, bs 128 (full size)")
    c = config_mixed_mxfp4(device=dev)
    torch.cuda.synchronize()
    say(f"  pool {c.pool.numel() / 1e9:.1f} GB, rows {c.num_rows}, max ctx {c.max_ctx}")
    lay = c.layout
    bt = c.block_table.cpu().numpy()
    seq = c.row_seq.cpu().numpy()
    ctxs = c.row_ctx.cpu().numpy()
    for layer in (0, 11, 23):
        scores, idx, out, lse = run_step(c, dev, layer)
        lo, hi = lay.lat_off[layer], lay.idx_off[layer] + lay.index_page_bytes
        pool = c.pool[:, lo:hi].cpu().numpy()
        sub = dict(block_size=lay.block_size, index_fmt=lay.index_fmt, latent_fmt=lay.latent_fmt,
                   row_bytes=hi - lo, lat_off=[0], idx_off=[lay.idx_off[layer] - lo])
        q_idx = c.q_idx[layer].cpu().numpy()
        q_sc = c.q_idx_scale[layer].cpu().numpy()
        w = c.w[layer].cpu().numpy()
        q_lat = c.q_lat[layer].cpu().view(torch.int16).numpy().view(np.uint16)
        for r in range(c.num_rows):
            ctx = int(ctxs[r])
            ref = O.decode_row(pool, sub, 0, bt[seq[r]], ctx, q_idx[r], q_sc[r], w[r], q_lat[r], c.k, c.sm_scale,
                               want_magnitude=True)
            check_scores(scores[r], ref, ctx)
            sel = check_selection(scores[r], idx[r], ref, ctx, c.k)
            lat = O.read_latents(pool, O.Layout(sub), 0, bt[seq[r]], sel)
            o_ref, l_ref = O.sparse_mla(O.bf16_to_f64(q_lat[r]), lat, c.sm_scale)
            e = np.abs(out[r] - o_ref)
            assert np.all(e <= 2e-3 + 1e-2 * np.abs(o_ref)), f"layer {layer} row {r}: out err {e.max():.3g}"
            el = np.abs(lse[r] - l_ref)
            assert np.all(el <= 2e-3 + 1e-2 * np.abs(l_ref)), f"layer {layer} row {r}: lse err {el.max():.3g}"
        say(f"  layer {layer}: 64 rows match the oracle")
        del pool


@pytest.mark.parametrize("fmt,bs", [("fp8", 64), ("mxfp4", 128)])
def test_prefill_append_row_groups(dev, fmt, bs):
    """The row-group indexer (rows_per_seq = all rows) on a 300-row append to a 20,000-token
    prefix, FP8 or MXFP4 keys: identical bytes to the row-by-row path, and oracle parity on
    sampled rows."""
    say(f"case: prefill-append 300 rows on 20000 prefix, {fmt} keys, rows_per_seq 300 vs 1")
    c = make_prefill_case(20000, 300, block_size=bs, seed=81, device=dev, index_fmt=fmt)
    hc = HostCase(c)
    a = run_step(c, dev, rows_per_seq=1)
    b = run_step(c, dev, rows_per_seq=c.num_rows)
    for r in range(c.num_rows):
        ctx = int(hc.row_ctx[r])
        assert np.array_equal(a[0][r, :ctx], b[0][r, :ctx]), f"scores row {r}"
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(x, y)
    for r in [0, 1, 17, 150, 299]:
        say(f"  oracle row {r}")
        ref = hc.oracle(r)
        ctx = int(hc.row_ctx[r])
        check_scores(b[0][r], ref, ctx)
        sel = check_selection(b[0][r], b[1][r], ref, ctx, c.k)
        check_attention(hc, r, sel, b[2][r], b[3][r])


@pytest.mark.parametrize("fmt,bs,hint", [("fp8", 64, 4), ("fp8", 64, 3), ("mxfp4", 128, 4), ("mxfp4", 128, 3),
                                         ("mxfp4", 16, 4)])
def test_speculative_verify_rows(dev, fmt, bs, hint):
    """Speculative verification: 5 sequences x 4 verify tokens, row j of sequence b sees
    t < L_b + j + 1, with FP8 or MXFP4 index keys. hint 4 matches the runs; hint 3 makes
    workgroups straddle sequences, which reload keys: the result must not change. Every
    row against the oracle."""
    say(f"case: speculative verify 5 x 4 rows, {fmt} keys, bs {bs}, rows_per_seq {hint}")
    lens = [3000, 17000, 40000, 9000, 70000]
    T = 4
    row_seq = [b for b in range(len(lens)) for _ in range(T)]
    row_ctx = [lens[b] + j + 1 for b in range(len(lens)) for j in range(T)]
    c = make_case(row_ctx, row_seq=row_seq, ctx_lens_are_rows=True, block_size=bs, seed=90, k=2048, device=dev,
                  index_fmt=fmt)
    hc = HostCase(c)
    base = run_step(c, dev, rows_per_seq=1)
    got = run_step(c, dev, rows_per_seq=hint)
    for r in range(c.num_rows):
        ctx = int(hc.row_ctx[r])
        assert np.array_equal(base[0][r, :ctx], got[0][r, :ctx]), f"scores row {r}"
    for x, y in zip(base[1:], got[1:]):
        assert np.array_equal(x, y)
    for r in range(c.num_rows):
        ctx = int(hc.row_ctx[r])
        ref = hc.oracle(r)
        check_scores(got[0][r], ref, ctx)
        sel = check_selection(got[0][r], got[1][r], ref, ctx, c.k)
        check_attention(hc, r, sel, got[2][r], got[3][r])


def test_out_of_range_block_ids_do_not_fault(dev):
    """Block ids outside the pool are clamped on the device: no fault, finite results."""
    say("case: corrupt block table entries")
    c = make_case([3000], block_size=64, seed=5, k=256).to(dev)
    bt = c.block_table.clone()
    bt[0, 3] = 10 ** 6
    bt[0, 5] = -7
    c2 = type(c)(c.name, c.layout, c.pool, bt, c.row_seq, c.row_ctx, c.q_idx, c.q_idx_scale, c.w, c.q_lat, c.k,
                 c.sm_scale)
    scores, idx, out, lse = run_step(c2, dev)
    assert np.all(np.isfinite(scores[0, :3000])) and np.all(np.isfinite(out))


def test_device_status_word(dev):
    """Repairs of bad data are reported in the device status word, and only then: a
    clean step leaves it at 0; a corrupt block table, a row_ctx above max_ctx (which
    then behaves as a row of max_ctx tokens), an MLA index past the block table
    (skipped like -1) and an append into a block outside the pool each set their bit."""
    say("case: device status word")
    dsa.dsa_device_status(clear=True)
    c = make_case([3000, 5000], block_size=64, seed=6, k=256, spare_blocks=1).to(dev)
    ref = run_step(c, dev)
    assert dsa.dsa_device_status(clear=True) == 0

    bt = c.block_table.clone()
    bt[0, 3] = 10 ** 6
    c_bad = type(c)(c.name, c.layout, c.pool, bt, c.row_seq, c.row_ctx, c.q_idx, c.q_idx_scale, c.w, c.q_lat, c.k,
                    c.sm_scale)
    run_step(c_bad, dev)
    assert dsa.dsa_device_status(clear=True) == dsa.DSA_DEV_BLOCK_CLAMPED
    assert dsa.dsa_device_status(clear=False) == 0

    # row 1 claims 5000 tokens but the call's bound is 4000: it is scored as 4000 tokens
    say("  row_ctx above max_ctx")
    lim = 4000
    idx, out, lse, _ = dsa.dsa_decode_step(c.pool, c.layout, 0, c.q_idx[0], c.q_idx_scale[0], c.w[0], c.q_lat[0],
                                           c.block_table, c.row_seq, c.row_ctx, lim, c.k, c.sm_scale)
    assert dsa.dsa_device_status(clear=True) == dsa.DSA_DEV_CTX_CLAMPED
    short = c.row_ctx.clone()
    short[1] = lim
    idx2, out2, lse2, _ = dsa.dsa_decode_step(c.pool, c.layout, 0, c.q_idx[0], c.q_idx_scale[0], c.w[0], c.q_lat[0],
                                              c.block_table, c.row_seq, short, lim, c.k, c.sm_scale)
    assert dsa.dsa_device_status(clear=True) == 0
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2)
    assert np.array_equal(idx.cpu().numpy()[0], ref[1][0])

    say("  standalone top-k, row_ctx above max_ctx")
    sc = torch.tensor(ref[0], device=dev)
    dsa.dsa_topk(sc, c.row_ctx, lim, c.k)
    assert dsa.dsa_device_status(clear=True) == dsa.DSA_DEV_CTX_CLAMPED

    say("  sparse MLA index past the block table")
    cap = c.block_table.shape[1] * c.layout.block_size
    sel = torch.tensor(ref[1], device=dev)
    bad = sel.clone()
    bad[0, 5] = cap + 3
    skip = sel.clone()
    skip[0, 5] = -1
    o1, l1 = dsa.dsa_sparse_mla(c.pool, c.layout, 0, c.q_lat[0], c.block_table, c.row_seq, bad, c.k, c.sm_scale)
    assert dsa.dsa_device_status(clear=True) == dsa.DSA_DEV_INDEX_RANGE
    o2, l2 = dsa.dsa_sparse_mla(c.pool, c.layout, 0, c.q_lat[0], c.block_table, c.row_seq, skip, c.k, c.sm_scale)
    assert dsa.dsa_device_status(clear=True) == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

    say("  cache append into a block outside the pool")
    before = c.pool.clone()
    pos = c.row_ctx.clone()
    bt2 = c.block_table.clone()
    bt2[:, pos[0].item() // c.layout.block_size] = -5
    bt2[1, pos[1].item() // c.layout.block_size] = 10 ** 6
    dsa.dsa_cache_append(c.pool, c.layout, 0, bt2, c.row_seq, pos, latent=torch.ones((2, 576), device=dev))
    assert dsa.dsa_device_status(clear=True) == dsa.DSA_DEV_BLOCK_CLAMPED
    assert torch.equal(before, c.pool)


def test_hbm_read_probe_reads_without_writing(dev):
    """The streaming-read reference launches at every grid size bench.py uses, over a
    buffer with a partial last chunk, and writes nothing: its XOR of zeros never equals
    the sink's trigger constant, so the sink keeps its sentinel."""
    say("case: hbm read probe")
    buf = torch.zeros((1 << 20) + 48, dtype=torch.uint8, device=dev)
    sink = torch.full((1,), 7, dtype=torch.int32, device=dev)
    for grid in (256, 512, 1024, 2048, 4096):
        dsa.dsa_hbm_read_probe(buf, sink, grid)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def test_select_paths_mixed_batch(dev):
    """One batch whose rows take every selection path: ctx <= k, whole row in LDS
    (<= 16384), and block candidates with rescans (> 16384)."""
    say("case: select paths mixed batch")
    c = make_case([1500, 3000, 16384, 16385, 20000, 33000, 70000], block_size=64, seed=44, k=2048)
    full_check(c, dev)


def test_four_wave_attention_short_and_empty_rows(dev):
    """160 rows take one attention split each (the cost model's choice once three head
    groups per row overfill the CUs), so the step runs the four-wave 32-head kernel on
    32-token chunks. Rows shorter than k leave -1 entries and partly empty chunks: an
    empty row, one token, chunk edges (31, 32, 33, 63, 64, 65), k - 1, k, k + 1, and
    longer rows up to 20,000 tokens (own-score and candidate selects). Every row with a
    listed length and every 8th of the rest is checked against the oracle."""
    say("case: four-wave attention, 160 rows, short and empty rows")
    edge = [0, 1, 2, 31, 32, 33, 63, 64, 65, 100, 2047, 2048, 2049, 4097, 16384, 16385, 20000]
    rng = np.random.default_rng(71)
    ctxs = edge + [int(x) for x in rng.integers(1, 6000, size=160 - len(edge))]
    c = make_case(ctxs, block_size=64, seed=71, k=2048)
    R = c.num_rows
    # one split per row: the attention needs no partials workspace
    assert R * 3 > 256 and dsa.dsa_workspace_bytes(dsa.DSA_OP_SPARSE_MLA, R, 0, 2048) <= 256
    rows = list(range(len(edge))) + list(range(len(edge), R, 8))
    full_check(c, dev, rows=rows)


def test_four_wave_attention_uneven_splits(dev):
    """32 rows: the eight-wave plan (8 splits) would take three rounds of workgroups, so
    FP8 latents run the four-wave kernel over 5 splits of a row's list (448 tokens each,
    the last 256) and the merge. Short rows leave whole splits empty. Every row is checked
    against the oracle; the NVFP4-latent path keeps the eight-wave kernel and is covered
    by the NVFP4 tests."""
    say("case: four-wave attention, 32 rows, 5 splits")
    edge = [0, 1, 40, 447, 448, 449, 1000, 1791, 1792, 1793, 2047, 2048, 2049, 30000]
    rng = np.random.default_rng(72)
    ctxs = edge + [int(x) for x in rng.integers(2048, 24000, size=32 - len(edge))]
    c = make_case(ctxs, block_size=64, seed=72, k=2048)
    full_check(c, dev)


def test_workspace_reuse_across_inputs(dev):
    """The workspace carries nothing from one call to the next."""
    say("case: workspace reuse")
    a = make_case([50000, 9000], block_size=64, seed=51, k=2048).to(dev)
    b = make_case([70000, 30000], block_size=64, seed=52, k=2048).to(dev)
    ws = torch.empty(dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, 2, 70000, 2048), dtype=torch.uint8, device=dev)
    ws.fill_(0xA5)

    def go(c, w):
        idx, out, lse, _ = dsa.dsa_decode_step(c.pool, c.layout, 0, c.q_idx[0], c.q_idx_scale[0], c.w[0], c.q_lat[0],
                                               c.block_table, c.row_seq, c.row_ctx, c.max_ctx, 2048, c.sm_scale,
                                               workspace=w)
        torch.cuda.synchronize()
        return idx.cpu().numpy(), out.cpu().numpy()

    go(a, ws)
    i1, o1 = go(b, ws)
    i2, o2 = go(b, None)
    assert np.array_equal(i1, i2) and np.array_equal(o1, o2)


# ----------------------------------------------------------------------------- cache append
def _append_inputs(R, seed):
    """fp32 keys / latents with the cases that decide rounding: exact ties of the e4m3
    grid (amax 448 makes the scale 1), e2m1 midpoints, zero vectors, tiny values, signs."""
    rng = np.random.default_rng(seed)
    key = rng.normal(0, 1, (R, 128)).astype(np.float32)
    lat = rng.normal(0, 3, (R, 576)).astype(np.float32)
    mids = np.array([1.0625, 1.1875, 3.25, -5.5, 0.0068359375, 448.0], dtype=np.float32)  # e4m3 midpoints (+ amax)
    lat[0, :6] = mids
    lat[0, 6:] = 0.5
    key[0, :6] = mids
    key[0, 6:] = 0.25
    key[1] = 0.0                                                  # all-zero key: scale 1
    lat[1] = 0.0
    key[2, :32] = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4, dtype=np.float32)  # e2m1 ties, E = 0
    key[2, 32:64] = np.float32(1e-30)                             # tiny group
    key[3] *= -1e5                                                # large values
    # NVFP4 block-scale decisions (token scale 1: dim 575 holds the amax 448)
    lat[4, 575] = 448.0
    lat[4, 0:16] = 0.5
    lat[4, 0] = 6.375                                             # max/6 = 1.0625: e4m3 tie -> 1.0, then clamp at 6
    lat[4, 16:32] = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 2, dtype=np.float32)  # e2m1 ties, scale 1
    lat[4, 32:48] = np.float32(1e-5)                              # block scale rounds to 0: codes 0
    lat[4, 48:64] = 0.0
    lat[4, 512:518] = np.array([1.0625, 1.1875, 3.25, -5.5, 0.0068359375, -0.0], dtype=np.float32)
    return key, lat


@pytest.mark.parametrize("fmt,bs,lat_fmt", [("fp8", 64, "fp8"), ("fp8", 16, "fp8"), ("mxfp4", 128, "fp8"),
                                            ("mxfp4", 16, "fp8"), ("fp8", 64, "nvfp4"), ("mxfp4", 16, "nvfp4")])
def test_cache_append_bit_exact(dev, fmt, bs, lat_fmt):
    """New-token append: the whole pool after the GPU append equals the oracle's append of
    the same inputs byte for byte; rows outside their table or on an unmapped block write nothing."""
    say(f"case: cache append {fmt} bs {bs} latents {lat_fmt}")
    c = make_case([300, 1000, 64, 2000, 5], block_size=bs, seed=95, k=64, index_fmt=fmt, num_layers=2,
                  spare_blocks=2, latent_fmt=lat_fmt).to(dev)
    R = 9
    key, lat = _append_inputs(R, 96)
    # rows 5, 6, 8 write nothing: a negative position, one past the table, one on an unmapped (-1) block
    row_seq = np.array([0, 1, 2, 3, 4, 0, 1, 3, 4], dtype=np.int32)
    pos = np.array([299, 1000, 10, 1999, 4, -1, 10 ** 7, 300, 200], dtype=np.int32)
    bt = c.block_table.cpu().numpy()
    assert bt[4][200 // bs] == -1
    pool0 = c.pool.cpu().numpy()
    want = O.append_tokens(pool0, O.Layout(c.layout), 1, bt, row_seq, pos, idx_key=key, latent=lat)
    dsa.dsa_cache_append(c.pool, c.layout, 1, c.block_table, torch.tensor(row_seq, device=dev),
                         torch.tensor(pos, device=dev), idx_key=torch.tensor(key, device=dev),
                         latent=torch.tensor(lat, device=dev))
    torch.cuda.synchronize()
    got = c.pool.cpu().numpy()
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
    assert np.any(got != pool0), "nothing was written"


def test_append_then_decode(dev):
    """Append a token's key and latent at position ctx, then decode over ctx + 1 tokens:
    the new token is scored and attended like any other (oracle on the appended bytes)."""
    say("case: append then decode")
    c = make_case([5000, 30000], block_size=64, seed=97, k=2048, spare_blocks=2).to(dev)
    rng = np.random.default_rng(98)
    key = (rng.normal(0, 1, (2, 128)) * 4).astype(np.float32)
    lat = rng.normal(0, 1, (2, 576)).astype(np.float32)
    pos = c.row_ctx.clone()                                        # the next token of each sequence
    dsa.dsa_cache_append(c.pool, c.layout, 0, c.block_table, c.row_seq, pos,
                         idx_key=torch.tensor(key, device=dev), latent=torch.tensor(lat, device=dev))
    c.row_ctx += 1
    scores, idx, out, lse = full_check(c, dev)
    for r in range(2):
        assert int(c.row_ctx[r]) - 1 < scores.shape[1]


# ----------------------------------------------------------------------------- NVFP4 latents

@pytest.mark.parametrize("bs", [16, 64])
def test_nvfp4_latents_ragged(dev, bs):
    """NVFP4 latent records (352 B) through the whole step: ragged rows, one shorter than k."""
    say(f"case: nvfp4 latents bs {bs}")
    c = make_case([300, 5000, 9001, 40000], block_size=bs, seed=120 + bs, k=2048, latent_fmt="nvfp4")
    full_check(c, dev)


def test_nvfp4_latents_batch_of_six(dev):
    """Batches above four rows run sparse MLA with 32 heads per workgroup (16 below):
    the NVFP4 path of the wider group."""
    say("case: NVFP4 latents, batch 6")
    c = make_case([300, 5000, 9001, 40000, 1500, 17000], block_size=64, seed=127, k=2048, latent_fmt="nvfp4")
    full_check(c, dev)


def test_nvfp4_latents_with_mxfp4_keys_and_empty_rows(dev):
    """The pages' smallest cache: NVFP4 latents with MXFP4 index keys, block size 128, two
    layers; an empty row gives zeros and -inf."""
    say("case: nvfp4 latents + mxfp4 keys")
    c = make_case([20000, 0, 70000, 700], block_size=128, seed=131, k=2048, index_fmt="mxfp4",
                  latent_fmt="nvfp4", num_layers=2)
    _, idx, out, lse = full_check(c, dev, layer=1)
    assert np.all(idx[1] == -1) and np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("k", [7, 100])
def test_nvfp4_latents_small_k(dev, k):
    say(f"case: nvfp4 latents k {k}")
    c = make_case([5000, 64, 3], block_size=64, seed=140 + k, k=k, latent_fmt="nvfp4")
    full_check(c, dev)


def test_nvfp4_append_then_decode(dev):
    """Append into an NVFP4 latent page, then decode over the new token."""
    say("case: nvfp4 append then decode")
    c = make_case([5000, 30000], block_size=64, seed=151, k=2048, spare_blocks=2, latent_fmt="nvfp4").to(dev)
    rng = np.random.default_rng(152)
    key = (rng.normal(0, 1, (2, 128)) * 4).astype(np.float32)
    lat = rng.normal(0, 1, (2, 576)).astype(np.float32)
    dsa.dsa_cache_append(c.pool, c.layout, 0, c.block_table, c.row_seq, c.row_ctx.clone(),
                         idx_key=torch.tensor(key, device=dev), latent=torch.tensor(lat, device=dev))
    c.row_ctx += 1
    full_check(c, dev)


def test_topk_long_rows_send_paths(dev):
    """dsa_topk on score rows long enough for 512-token send units (the threshold route of
    eight-wave units), bit for bit against the exact selection: heavy ties (most units fall
    back to the sort-and-merge route), a descending ramp (the whole top-k in four units),
    last units with 10 and 40 valid tokens (a wave with no key, so the threshold is 0),
    m = 8 above 776,192 tokens, all-negative scores, one unit holding 512 of the top k
    (rescanned), and a 1,048,576-token row."""
    say("case: dsa_topk on long synthetic rows")
    rng = np.random.default_rng(77)
    n = 262144
    hot = rng.normal(0, 1, n)
    hot[7 * 512:8 * 512] = 10.0 + rng.normal(0, 0.1, 512)
    rows = [np.round(rng.normal(0, 1, n), 1), -np.arange(n, dtype=np.float64), rng.normal(0, 1, n + 10),
            rng.normal(0, 1, 600 * 512 + 40), rng.normal(0, 1, 800000), rng.normal(-5.0, 1.0, n), hot,
            rng.normal(0, 1, 1 << 20)]
    rows = [x.astype(np.float32) for x in rows]
    ctx = [len(x) for x in rows]
    max_ctx = max(ctx)
    S = np.zeros((len(rows), max_ctx), dtype=np.float32)
    for r, x in enumerate(rows):
        S[r, :len(x)] = x
    idx = dsa.dsa_topk(torch.from_numpy(S).to(dev), torch.tensor(ctx, dtype=torch.int32, device=dev), max_ctx,
                       2048)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for r, x in enumerate(rows):
        say(f"  row {r} ctx {len(x)}")
        assert np.array_equal(idx[r], O.select_topk(x, 2048)), f"row {r}: selection differs"
    assert np.array_equal(idx[1], np.arange(2048)), "ramp: the first k tokens"
    assert np.all(np.isin(np.arange(7 * 512, 8 * 512), idx[6])), "the hot unit's keys are all selected"


# ----------------------------------------------------------------------------- context-parallel merge

def _dcp_check(dev, rows, k, W):
    """rows: list of fp32 score arrays. Bit-exact against the oracle's merge (tokens,
    resend mask, the words themselves) and against the plain top-k."""
    R = len(rows)
    ctx = [len(x) for x in rows]
    max_ctx = max(ctx)
    ld = max(max_ctx, 1)
    S = np.zeros((R, ld), dtype=np.float32)
    for r, x in enumerate(rows):
        S[r, :len(x)] = x
    st = torch.from_numpy(S).to(dev)
    rc = torch.tensor(ctx, dtype=torch.int32, device=dev)
    idx, mask, words = dsa.dsa_topk_dcp(st, rc, max_ctx, k, W, with_words=True)
    plain = dsa.dsa_topk(st, rc, max_ctx, k)
    torch.cuda.synchronize()
    idx, plain = idx.cpu().numpy(), plain.cpu().numpy()
    mask = mask.cpu().numpy().view(np.uint32)
    words = words.cpu().numpy().view(np.uint32)
    M = dsa.dcp_send_count(k, W)
    masks = []
    for r, x in enumerate(rows):
        tok, omask, nw = O.dcp_merge(x, k, W)
        total = min(k, len(x))
        assert np.array_equal(tok, O.select_topk(x, k)), "oracle merge is not the plain top-k"
        assert np.array_equal(idx[r, :total], tok) and np.all(idx[r, total:] == -1), f"row {r}: selection"
        assert np.array_equal(idx[r], plain[r]), f"row {r}: differs from dsa_topk"
        assert int(mask[r]) == omask, f"row {r}: resend mask {int(mask[r]):#x} vs {omask:#x}"
        assert int(np.count_nonzero(words[r] != 0xFFFFFFFF)) == nw, f"row {r}: words sent"
        for s in range(W):
            sh = np.arange(s, len(x), W)
            g = sh[O.select_topk(x[sh], M)]
            want = ((O.bf16_key(x[g]).astype(np.uint64) << 16) | np.arange(g.size, dtype=np.uint64)).astype(np.uint32)
            got = words[r, s * M:(s + 1) * M]
            assert np.array_equal(got[:g.size], want) and np.all(got[g.size:] == 0xFFFFFFFF), f"row {r} shard {s}"
        masks.append(omask)
    return masks


@pytest.mark.parametrize("W", [2, 3, 8])
def test_dcp_merge_ragged(dev, W):
    """Ragged rows (shard rows above and below the whole-row select limit), rounded
    scores with many ties, one shard holding the whole top-k, a short and an empty row."""
    say(f"case: dcp merge ragged W={W}")
    rng = np.random.default_rng(300 + W)
    hot = rng.normal(0, 1, 36000)
    hot[3 % W::W] += 5.0
    rows = [rng.normal(0, 1, 40000), np.round(rng.normal(0, 1, 30000), 1), hot, rng.normal(0, 1, 1500),
            np.zeros(0), rng.normal(0, 1, 5003)]
    masks = _dcp_check(dev, [x.astype(np.float32) for x in rows], 2048, W)
    assert masks[2] & (1 << (3 % W)), "the shard holding the whole top-k resends"


def test_dcp_merge_constant_scores(dev):
    """Every score equal: every shard's weakest word ties the threshold, all resend,
    and the first k tokens win."""
    say("case: dcp merge constant scores")
    masks = _dcp_check(dev, [np.zeros(20000, np.float32), np.full(9000, -1.5, np.float32)], 2048, 4)
    assert masks == [0xF, 0xF]


@pytest.mark.parametrize("k", [1, 7, 100])
def test_dcp_merge_small_k(dev, k):
    say(f"case: dcp merge k={k}")
    rng = np.random.default_rng(400 + k)
    _dcp_check(dev, [rng.normal(0, 1, 9000).astype(np.float32), rng.normal(0, 1, 5).astype(np.float32)], k, 4)


@pytest.mark.parametrize("W", [4, 8])
def test_dcp_merge_indexer_scores_256k(dev, W):
    """The indexer's own scores at the long-context shape (262,144 tokens, plus a
    100,000-token row): the merge gives dsa_topk's selection bit for bit."""
    say(f"case: dcp merge on indexer scores 256k W={W}")
    c = make_case([262144, 100000], block_size=64, seed=61, device=dev)
    scores, idx, _, _ = run_step(c, dev)
    rows = [scores[0, :262144].copy(), scores[1, :100000].copy()]
    _dcp_check(dev, rows, 2048, W)
