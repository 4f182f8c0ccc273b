"""Benchmark: DSA decode layer-steps per second and achieved HBM bandwidth at 256K context.

One step = one dsa_decode_step call (indexer -> exact top-2048 -> sparse MLA ->
split merge) for a decode batch of one query row with a 262,144-token context,
on one DSA layer. Steps rotate over 24 independent layers of one packed cache
(186.6 MB of cache per layer, 4.48 GB in all) so that the working set is far
larger than the GPU's 256 MB last-level cache. Inputs are seeded synthetic data
already resident in HBM when timing starts.

Prints one JSON line. `roofline` is for the dominant kernel (the indexer): its
algorithmic bytes per launch divided by its average launch duration, timed with
HIP events around each launch on the stream it runs on. `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload (rank 0, one GPU only).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode layer-steps/sec + achieved HBM GB/s (% of peak) at 256K ctx"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix peak (the indexer's contraction runs in bf16)
CTX = 262144
LAYERS = 24
K = 2048
BS = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
INDEXER_SRCS = [os.path.join(ROOT, "sparse_attention_decode_paged_amd", "csrc", f)
                for f in ("indexer.hip", "topk_send.h", "common.h")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=240)
    p.add_argument("--warmup", type=int, default=48)
    p.add_argument("--ctx", type=int, default=CTX)
    p.add_argument("--layers", type=int, default=LAYERS)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--index-fmt", choices=["fp8", "mxfp4"], default="fp8",
                   help="index key format (the headline workload uses fp8)")
    p.add_argument("--block-size", type=int, default=BS)
    p.add_argument("--latent-fmt", choices=["fp8", "nvfp4"], default="fp8",
                   help="latent records: FP8 (576 B + scale) or NVFP4 (352 B + scale)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--dcp", type=int, default=0, metavar="W",
                   help="instead of the decode step, time the exact top-k merge of decode context parallelism "
                        "emulated over W token-strided shards, beside the plain top-k, on the indexer's scores")
    p.add_argument("--cpu-layers", type=int, default=4, help="layer-steps the CPU oracle runs for cpu_baseline")
    p.add_argument("--config", choices=["headline", "small", "batch16", "long1m", "prefill", "mixed_mxfp4", "verify"],
                   default="headline",
                   help="workload: headline (batch x ctx from --batch/--ctx/--layers, the default), or one of the "
                        "other measured workloads: small (1 x 8,192), batch16 (16 rows, 16K-64K), long1m (1 x 1M, "
                        "2,048 planted keys, 2 layers), prefill (2,048 rows on a 150,000-token prefix), mixed_mxfp4 "
                        "(64 rows, 4K-256K log-uniform, bs 128, MXFP4 keys, 24 layers), verify (speculative "
                        "verification: 16 sequences x 4 rows on 65,536-token contexts, keys per --index-fmt, bs 128)")
    p.add_argument("--rows-per-seq", type=int, default=0,
                   help="override the workload's rows_per_seq hint (0: the workload's own; 1: row by row)")
    p.add_argument("--cpu-configs", action="store_true",
                   help="only time the CPU oracle on bounded samples of the other workloads (8K, batch 16, 1M, "
                        "prefill-append, batch-64 MXFP4) and print one JSON line")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a 1 GiB device copy (for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def src_sha(paths):
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel_srcs):
    """HBM bytes per launch from committed counter summaries, if taken on these sources."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get("indexer_fp8_step")
    if not e or e.get("source_sha") != src_sha(kernel_srcs):
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(case, layers, k):
    """Time the CPU oracle on `layers` full layer-steps of the same workload."""
    import numpy as np
    import torch
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    lay = case.layout
    bt = case.block_table.cpu().numpy()
    q_idx = case.q_idx.cpu().numpy()
    q_sc = case.q_idx_scale.cpu().numpy()
    w = case.w.cpu().numpy()
    q_lat = case.q_lat.cpu().view(torch.int16).numpy().view(np.uint16)
    R = case.num_rows
    ctxs = case.row_ctx.cpu().numpy()
    t_total = 0.0
    n = 0
    for l in range(layers):
        # only this layer's pages travel to the host: the row bytes [lat_off, idx_off + page)
        lo = lay.lat_off[l]
        hi = lay.idx_off[l] + lay.index_page_bytes
        pool = case.pool[:, lo:hi].cpu().numpy()
        sub = dict(block_size=lay.block_size, index_fmt=lay.index_fmt, latent_fmt=lay.latent_fmt, row_bytes=hi - lo,
                   lat_off=[0], idx_off=[lay.idx_off[l] - lo])
        t0 = time.perf_counter()
        for r in range(R):
            O.decode_row(pool, sub, 0, bt[r], int(ctxs[r]), q_idx[l, r], q_sc[l, r], w[l, r], q_lat[l, r], k,
                         case.sm_scale)
        t_total += time.perf_counter() - t0
        n += 1
    return dict(value=n / t_total, unit="layer-steps/s", cores=int(threads), kind="oracle",
                sample=f"{n} of the {case.layout.num_layers} layers, {R} row(s) x {int(ctxs.max())} tokens each, "
                       f"full indexer + top-{k} + sparse MLA per layer (float64 numpy, BLAS threads={threads})")


def host_info():
    """CPU model, usable cores and the BLAS numpy calls (threadpoolctl)."""
    import os
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: i.get(k) for k in ("internal_api", "num_threads", "version")} for i in threadpool_info()]
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "cores_usable": len(os.sched_getaffinity(0)), "blas": blas}


def oracle_rows_seconds(case, layer, rows, k):
    """Wall seconds of the CPU oracle (full indexer + top-k + sparse MLA) on each row of
    `rows` of one layer; only that layer's pages are copied to the host."""
    import numpy as np
    import torch
    from oracle import dsa_oracle as O
    lay = case.layout
    lo = lay.lat_off[layer]
    hi = lay.idx_off[layer] + lay.index_page_bytes
    pool = case.pool[:, lo:hi].cpu().numpy()
    sub = dict(block_size=lay.block_size, index_fmt=lay.index_fmt, latent_fmt=lay.latent_fmt, row_bytes=hi - lo,
               lat_off=[0], idx_off=[lay.idx_off[layer] - lo])
    bt = case.block_table.cpu().numpy()
    seq = case.row_seq.cpu().numpy()
    ctxs = case.row_ctx.cpu().numpy()
    q_lat = case.q_lat[layer].cpu().view(torch.int16).numpy().view(np.uint16)
    q_idx = case.q_idx[layer].cpu().numpy()
    q_sc = case.q_idx_scale[layer].cpu().numpy()
    w = case.w[layer].cpu().numpy()
    secs = []
    for r in rows:
        t0 = time.perf_counter()
        O.decode_row(pool, sub, 0, bt[seq[r]], int(ctxs[r]), q_idx[r], q_sc[r], w[r], q_lat[r], k, case.sm_scale)
        secs.append(time.perf_counter() - t0)
    return secs


def cpu_configs(dev):
    """The oracle timed on bounded samples of the other workloads. Rows not timed are
    extrapolated in proportion to their context length (the oracle's work is the
    indexer over ctx tokens plus a top-k and attention that vary little)."""
    import torch
    from synth import config_small, config_batch16, config_long_1m, config_prefill_append, config_mixed_mxfp4
    res = {"host": host_info(), "configs": []}
    plans = [
        ("decode, batch 1, 8,192 tokens, bs 64, FP8 keys", lambda: config_small(device=dev), None),
        ("decode, batch 16, U[16384, 65536] tokens, bs 64, FP8 keys", lambda: config_batch16(device=dev), 4),
        ("decode, batch 1, 1,048,576 tokens (2,048 planted), bs 64, FP8 keys", lambda: config_long_1m(device=dev),
         None),
        ("prefill-append, 2,048 rows on a 150,000-token prefix, bs 64, FP8 keys",
         lambda: config_prefill_append(device=dev), 4),
        ("decode, batch 64, log-uniform [4096, 262144] tokens, bs 128, MXFP4 keys (one of 24 layers)",
         lambda: config_mixed_mxfp4(device=dev, num_layers=1), 4),
    ]
    for name, build, nsample in plans:
        case = build()
        if case.pool.is_cuda:
            torch.cuda.synchronize()
        R = case.num_rows
        ctxs = [int(c) for c in case.row_ctx.tolist()]
        rows = list(range(R)) if nsample is None or nsample >= R else \
            sorted(set(int(round(i * (R - 1) / (nsample - 1))) for i in range(nsample)))
        secs = oracle_rows_seconds(case, 0, rows, K)
        t_sample = sum(secs)
        t_all = t_sample * sum(ctxs) / max(1, sum(ctxs[r] for r in rows))
        res["configs"].append({
            "workload": name, "rows": R, "rows_timed": rows, "seconds_timed": round(t_sample, 3),
            "seconds_per_layer_step": round(t_all, 3), "layer_steps_per_s": round(1.0 / t_all, 4),
            "extrapolated": len(rows) < R})
        print(f"cpu oracle: {name}: {t_all:.3f} s per layer-step", file=sys.stderr, flush=True)
        del case
        if torch.cuda.is_available():
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


def timed_stage_us(dsa, case, ws, bufs, layers, max_ctx, stage, reps, rows_per_seq=1, per_graph=24):
    """Average duration of one kernel of the decode step, launched alone through
    dsa_decode_step_stages on the step's own workspace: a HIP graph holds `per_graph`
    launches back to back (layer i % layers for launch i) and is replayed `reps` times
    between one pair of events on the stream it runs on, so no host launch cost falls
    inside the timing."""
    import torch
    dev = case.pool.device
    idx, out, lse = bufs

    def launch(l):
        dsa.dsa_decode_step_stages(case.pool, case.layout, l, case.q_idx[l], case.q_idx_scale[l], case.w[l],
                                   case.q_lat[l], case.block_table, case.row_seq, case.row_ctx, max_ctx, K,
                                   case.sm_scale, idx, out, lse, ws, stage, rows_per_seq=rows_per_seq)

    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        for l in range(layers):
            launch(l)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for i in range(per_graph):
            launch(i % layers)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / (reps * per_graph)


def hbm_read_ceiling(dsa, buf, reps=3, grids=(256, 512, 1024, 2048, 4096)):
    """Streaming-read rate (GB/s) of dsa_hbm_read_probe over the whole tensor `buf`, at a
    few grid sizes: per grid the median of `reps` launches, each timed alone with
    events; the best grid's median is the ceiling."""
    import torch
    dev = buf.device
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    nbytes = buf.numel() * buf.element_size()
    per_grid = {}
    for grid in grids:
        for _ in range(2):
            dsa.dsa_hbm_read_probe(buf, sink, grid)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            dsa.dsa_hbm_read_probe(buf, sink, grid)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        rates = sorted(nbytes / (ev[i].elapsed_time(ev[i + 1]) * 1e-3) / 1e9 for i in range(reps))
        per_grid[grid] = round(rates[len(rates) // 2], 1)
    best = max(per_grid, key=per_grid.get)
    return {"gbps": per_grid[best], "grid": best, "median_by_grid": {str(g): v for g, v in per_grid.items()},
            "bytes": nbytes, "unit": "GB/s",
            "kernel": "hbm_read_kernel (dsa_hbm_read_probe: 16-byte nontemporal loads in 16-KB chunks per "
                      "256-thread workgroup, over the whole layer-rotated cache pool)"}


def size_matched_read(dsa, buf, nbytes, reps=5, per_graph=24, grids=(512, 1024, 2048, 4096)):
    """One dsa_hbm_read_probe launch over exactly `nbytes` (a kernel's algorithmic bytes),
    launched back to back from a HIP graph as the step launches its kernels: launch i
    reads slice i of `buf` (up to `per_graph` disjoint slices spread over the whole buffer,
    together at least 512 MB, so none is cache-resident when read). Per grid the average launch over `reps` replays;
    the best grid's time is the shortest a launch reading that many bytes once took."""
    import torch
    dev = buf.device
    total = buf.numel() * buf.element_size()
    flat = buf.view(-1).view(torch.uint8)
    n = (nbytes + 15) // 16 * 16
    # fewer slices when the bytes are large, as long as together they hold at least twice
    # the 256 MB last-level cache
    per_graph = min(per_graph, total // max(n, 1))
    if per_graph < 2 or per_graph * n < (512 << 20):
        return None
    stride = (total // per_graph) // 16384 * 16384
    if stride < n:
        return None
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cap = torch.cuda.Stream(dev)
    res = {}
    for grid in grids:
        slices = [flat[i * stride:i * stride + n] for i in range(per_graph)]
        cap.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cap):
            for sl in slices:
                dsa.dsa_hbm_read_probe(sl, sink, grid)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for sl in slices:
                dsa.dsa_hbm_read_probe(sl, sink, grid)
        g.replay()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        res[grid] = 1000.0 * e0.elapsed_time(e1) / (reps * per_graph)
        del g
    best = min(res, key=res.get)
    return {"us": round(res[best], 3), "grid": best, "bytes": n,
            "us_by_grid": {str(k): round(v, 3) for k, v in res.items()}}


def bench_dcp(a, dsa, case, dev):
    """Times dsa_topk_dcp (W emulated shards) and dsa_topk on the same indexer scores,
    one call per layer from a HIP graph; prints one JSON line."""
    import torch
    R, max_ctx, W = case.num_rows, case.max_ctx, a.dcp
    ld = dsa.dsa_decode_scores_ld(max_ctx)
    scores = torch.empty((a.layers, R, ld), dtype=torch.float32, device=dev)
    for l in range(a.layers):
        dsa.dsa_indexer_score(case.pool, case.layout, l, case.q_idx[l], case.q_idx_scale[l], case.w[l],
                              case.block_table, case.row_seq, case.row_ctx, max_ctx, scores[l], ld_scores=ld)
    idx = torch.empty((R, K), dtype=torch.int32, device=dev)
    mask = torch.empty((R,), dtype=torch.int32, device=dev)
    wsd = torch.empty(dsa.load_library().dsa_topk_dcp_workspace_bytes(R, max_ctx, K, W), dtype=torch.uint8, device=dev)
    wst = torch.empty(max(dsa.dsa_workspace_bytes(dsa.DSA_OP_TOPK, R, max_ctx, K), 256), dtype=torch.uint8, device=dev)

    def merge(l):
        dsa.dsa_topk_dcp(scores[l], case.row_ctx, max_ctx, K, W, idx=idx, resend_mask=mask, workspace=wsd,
                         ld_scores=ld)

    def plain(l):
        dsa.dsa_topk(scores[l], case.row_ctx, max_ctx, K, idx=idx, workspace=wst, ld_scores=ld)

    def timed(fn):
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cap):
            for l in range(a.layers):
                fn(l)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for l in range(a.layers):
                fn(l)
        reps = max(1, a.steps // a.layers)
        for _ in range(max(1, a.warmup // a.layers)):
            g.replay()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / (reps * a.layers), reps * a.layers

    us_dcp, n = timed(merge)
    us_plain, _ = timed(plain)
    resend = [int(m) & 0xFFFFFFFF for m in mask.tolist()]
    print(json.dumps({
        "metric": "exact top-k merge over emulated context-parallel shards",
        "value": round(1e6 / us_dcp, 1),
        "unit": "merges/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": a.warmup,
        "ms_per_step": round(us_dcp / 1000.0, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"top-{K} of batch {R} rows of {a.ctx} indexer scores, {W} token-strided shards "
                               f"each sending ceil(1.5 k / W) BF16-keyed words, {a.layers} layers rotated",
                   "batch": R, "ctx": a.ctx, "k": K, "shards": W, "layers_rotated": a.layers,
                   "launch": "HIP graph replay, one merge per layer"},
        "plain_topk_us": round(us_plain, 3),
        "merge_us": round(us_dcp, 3),
        "resend_mask_last_layer": resend,
    }), flush=True)


def build_workload(a, dev):
    """The synthetic case of the chosen workload, its rows_per_seq hint and its name."""
    from synth import (make_case, config_small, config_batch16, config_prefill_append, config_mixed_mxfp4)
    if a.config == "headline":
        key_desc = "FP8 index keys (132 B/token)" if a.index_fmt == "fp8" else "MXFP4 index keys (68 B/token)"
        lat_desc = ("FP8 latents (576 B + fp32 scale)" if a.latent_fmt == "fp8"
                    else "NVFP4 latents (352 B + fp32 scale)")
        case = make_case([a.ctx] * a.batch, block_size=a.block_size, num_layers=a.layers, seed=a.seed, device=dev,
                         k=K, index_fmt=a.index_fmt, latent_fmt=a.latent_fmt,
                         name="decode_b%d_ctx%d_x%dlayers" % (a.batch, a.ctx, a.layers))
        return case, 1, (f"DSA decode, batch {a.batch}, context {a.ctx} tokens, top-{K}, block size {a.block_size}, "
                         f"{key_desc} and {lat_desc}, {a.layers} independent layers rotated")
    if a.config == "small":
        return (config_small(seed=a.seed, device=dev), 1,
                "DSA decode, batch 1, context 8,192 tokens, top-2048, block size 64, FP8 keys and latents, one layer")
    if a.config == "batch16":
        return (config_batch16(seed=a.seed, device=dev), 1,
                "DSA decode, batch 16, contexts uniform on [16,384, 65,536], pages shuffled in one pool, top-2048, "
                "block size 64, FP8 keys and latents, one layer")
    if a.config == "long1m":
        case = make_case([1 << 20], block_size=64, num_layers=2, seed=a.seed, device=dev, plant=2048,
                         name="decode_b1_ctx1m_planted_x2layers")
        return (case, 1, "DSA decode, batch 1, context 1,048,576 tokens with 2,048 planted keys, top-2048, block "
                         "size 64, FP8 keys and latents, 2 independent layers rotated")
    if a.config == "prefill":
        return (config_prefill_append(seed=a.seed, device=dev), 2048,
                "DSA prefill-append, 2,048 query rows on a 150,000-token prefix (row r sees tokens <= 150,000 + r), "
                "top-2048 per row, block size 64, FP8 keys and latents, one layer")
    if a.config == "verify":
        S, T, L = 16, 4, 65536
        row_seq = [b for b in range(S) for _ in range(T)]
        row_ctx = [L - T + j + 1 for _ in range(S) for j in range(T)]
        case = make_case(row_ctx, row_seq=row_seq, ctx_lens_are_rows=True, block_size=128, seed=a.seed, device=dev,
                         k=K, index_fmt=a.index_fmt, name="verify_16x4_ctx64k")
        return (case, T, f"DSA speculative verification: 16 sequences x 4 query rows (row j sees {L - T} + j + 1 "
                         f"tokens of its sequence), top-2048 per row, block size 128, "
                         f"{'MXFP4' if a.index_fmt == 'mxfp4' else 'FP8'} index keys, FP8 latents, one layer")
    return (config_mixed_mxfp4(seed=a.seed, device=dev), 1,
            "DSA decode, batch 64, contexts log-uniform on [4,096, 262,144], top-2048, block size 128, MXFP4 index "
            "keys and FP8 latents, 24 layers in one packed row, rotated")


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (the path is single-GPU, "
              f"multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_attention_decode_paged_amd as dsa
    from sparse_attention_decode_paged_amd import accounting as A
    from synth import make_case

    dev = torch.device("cuda:0")
    dsa.load_library()
    if a.cpu_configs:
        return cpu_configs(dev)
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 5}))
        return

    t0 = time.time()
    case, rows_per_seq, workload = build_workload(a, dev)
    if a.rows_per_seq > 0:
        rows_per_seq = a.rows_per_seq
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    a.layers = case.layout.num_layers
    a.index_fmt, a.latent_fmt, a.block_size = case.layout.index_fmt, case.layout.latent_fmt, case.layout.block_size
    R, max_ctx = case.num_rows, case.max_ctx
    if a.dcp:
        return bench_dcp(a, dsa, case, dev)
    ws = torch.empty(dsa.dsa_workspace_bytes(dsa.DSA_OP_DECODE_STEP, R, max_ctx, K), dtype=torch.uint8, device=dev)
    idx = torch.empty((R, K), dtype=torch.int32, device=dev)
    out = torch.empty((R, 96, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, 96), dtype=torch.float32, device=dev)

    def step(i):
        l = i % a.layers
        dsa.dsa_decode_step(case.pool, case.layout, l, case.q_idx[l], case.q_idx_scale[l], case.w[l], case.q_lat[l],
                            case.block_table, case.row_seq, case.row_ctx, max_ctx, K, case.sm_scale,
                            idx=idx, out=out, lse=lse, workspace=ws, rows_per_seq=rows_per_seq)

    # One launch form for any --steps: the timed region is one replay of a HIP graph that
    # holds exactly `steps` layer-steps, rotating over the layers (layer i % layers), so no
    # host launch cost falls inside it. Warm-up: eager steps before capture, then one replay
    # of a graph of `warmup` steps (and one of the timed graph).
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        for i in range(2 * a.layers):  # eager warm-up before capture
            step(i)
    torch.cuda.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for i in range(n):
                step(i)
        return g

    g_steps = capture(a.steps)
    if a.warmup > 0:
        g_warm = capture(a.warmup)
        g_warm.replay()
        del g_warm
    g_steps.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g_steps.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps

    # spread: more replays of the same graph, each timed alone
    nrep = 9
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nrep + 1)]
    ev[0].record(stream)
    for i in range(nrep):
        g_steps.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(1000.0 * ev[i].elapsed_time(ev[i + 1]) / a.steps for i in range(nrep))
    spread = {"p10": round(per[int(0.1 * (nrep - 1))], 3), "p50": round(per[(nrep - 1) // 2], 3),
              "p90": round(per[int(0.9 * (nrep - 1))], 3), "replays": nrep, "steps_per_replay": a.steps}
    del g_steps
    # the read ceiling needs a buffer far beyond the 256 MB last-level cache
    pool_bytes = case.pool.numel() * case.pool.element_size()
    ceiling = hbm_read_ceiling(dsa, case.pool) if pool_bytes >= (1 << 30) else None

    # each kernel of the step timed alone (the step's own launches, on its workspace)
    reps = max(2, min(a.steps, 480) // 24)
    bufs = (idx, out, lse)
    # (the select and the attention are timed together: for batches of up to 4 rows with FP8
    # latents the step runs them as one launch, select_mla_kernel)
    st_us = {name: timed_stage_us(dsa, case, ws, bufs, a.layers, max_ctx, bit, reps, rows_per_seq)
             for name, bit in (("indexer", dsa.DSA_STAGE_INDEXER),
                               ("select_attention", dsa.DSA_STAGE_TOPK | dsa.DSA_STAGE_ATTENTION),
                               ("merge", dsa.DSA_STAGE_MERGE))}
    fused_sel = a.latent_fmt == "fp8" and R <= 4
    ix_us = st_us["indexer"]
    ctxs = [int(c) for c in case.row_ctx.tolist()]
    ix_kernel = {("fp8", False): "indexer_fp8_kernel<PAGED32, SEND=true>", ("fp8", True): "indexer_fp8_rows_kernel",
                 ("mxfp4", False): "indexer_mxfp4_kernel<PAGED32, SEND=true>",
                 ("mxfp4", True): "indexer_mxfp4_rows_kernel"}.get(
        (a.index_fmt, rows_per_seq > 1), "indexer")
    if max_ctx <= 16384:
        ix_kernel = ix_kernel.replace("SEND=true", "SEND=false")
    if a.config == "verify":
        # a few rows per sequence: each key is read once for its sequence's rows, so the
        # scan stays bound by the key bytes of the sequences
        step_bytes = None
        seqs = {}
        for q, c in zip(case.row_seq.tolist(), ctxs):
            seqs[q] = max(seqs.get(q, 0), c)
        ix_bytes = sum(A.indexer_bytes(c, a.index_fmt) for c in seqs.values()) + \
            (len(ctxs) - len(seqs)) * (A.Q_IDX if a.index_fmt == "fp8" else A.Q_IDX_MX)
        ix_gbps = ix_bytes / (ix_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ix_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ix_gbps / PEAK_HBM_GBPS, 4), "traffic": None, "algorithmic_bytes_per_launch": ix_bytes}
    elif rows_per_seq > 1:
        # rows share one sequence's keys: bytes are not the bound, the contraction is
        step_bytes = None
        ix_flops = A.indexer_flops(ctxs)
        roof = {"bound": "mfma", "achieved": round(ix_flops / (ix_us * 1e-6) / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ix_flops / (ix_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "algorithmic_flops_per_launch": ix_flops}
    else:
        step_bytes = A.layer_step_bytes(ctxs, K, a.index_fmt, a.latent_fmt)
        ix_bytes = sum(A.indexer_bytes(c, a.index_fmt) for c in ctxs)
        ix_gbps = ix_bytes / (ix_us * 1e-6) / 1e9
        traffic = (traffic_for(INDEXER_SRCS) if a.index_fmt == "fp8" and a.config == "headline" and a.batch == 1
                   and a.ctx == CTX and a.block_size == BS else None)
        roof = {"bound": "hbm", "achieved": round(ix_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ix_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic, "algorithmic_bytes_per_launch": ix_bytes,
                "frac_of_measured_read_ceiling": round(ix_gbps / ceiling["gbps"], 4) if ceiling else None}
        if ceiling:
            # the same bytes read by the streaming probe in one graph-launched kernel: the
            # launch's ramp and drain at this size, which no kernel of this size avoids
            same = size_matched_read(dsa, case.pool, ix_bytes)
            if same:
                roof["size_matched_read"] = dict(same, kernel="hbm_read_kernel")
                roof["frac_of_size_matched_read"] = round(same["us"] / ix_us, 4)
    step_gbps = step_bytes / (ms * 1e-3) / 1e9 if step_bytes else None
    # the other kernels of the step against their own algorithmic bytes (select: the 4 B
    # per token of scores it decides over; attention: the gathered latents, query, indices
    # and output); latency-bound at one row, reported for what they cost
    sel_bytes = 4 * sum(ctxs)
    att_bytes = sum(A.attention_bytes(c, K, a.latent_fmt) for c in ctxs)
    sa_bytes = sel_bytes + att_bytes
    sa_us = st_us["select_attention"]
    kernels = {
        "select_attention": {
            "kernels": "select_mla_kernel<CAND> (one launch)" if fused_sel
            else "topk_select_kernel<CAND>, then sparse_mla_kernel<NV, G> or sparse_mla32_kernel (the "
                 "split plan's choice)",
            "avg_us": round(sa_us, 3), "algorithmic_bytes": sa_bytes,
            "achieved_gbps": round(sa_bytes / (sa_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(sa_bytes / (sa_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)},
        "split_merge": {"avg_us": round(st_us["merge"], 3)},
    }

    res = {
        "metric": METRIC,
        "value": round(1000.0 / ms, 1),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "name": a.config,
            "batch": R, "ctx": max_ctx, "k": K, "block_size": a.block_size, "layers_rotated": a.layers,
            "index_fmt": a.index_fmt, "latent_fmt": a.latent_fmt, "rows_per_seq": rows_per_seq,
            "launch": "one HIP graph replay of exactly `steps` decode steps, layer i % layers for step i",
        },
        "step_us": spread,
        "step_hbm_gbps": round(step_gbps, 1) if step_gbps else None,
        "step_hbm_frac": round(step_gbps / PEAK_HBM_GBPS, 4) if step_gbps else None,
        "step_algorithmic_bytes": step_bytes,
        "roofline": dict({"kernel": ix_kernel + " (the step's indexer launch, with the top-k candidate stage)"},
                         **roof, avg_launch_us=round(ix_us, 3)),
        "step_kernels": kernels,
        "hbm_read_ceiling": ceiling,
        "gen_seconds": round(gen_s, 1),
    }
    if not a.no_cpu_baseline and a.config == "headline":
        res["cpu_baseline"] = cpu_baseline(case, min(a.cpu_layers, a.layers), K)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
