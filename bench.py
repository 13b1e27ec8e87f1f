#!/usr/bin/env python3
"""DSA decode benchmark on one MI355X.

One step = one dsa_decode_step call (lightning indexer -> causal top-2048 ->
absorbed sparse MLA attention) over one batch of decode rows whose inputs are
already resident in HBM.  Default workload: 64 sequences x 32,768 positions,
one query row each (batched decode), seeded synthetic bf16 N(0,1) inputs.

Prints ONE JSON line on stdout; progress goes to stderr.

Roofline: for decode batches (one query row per sequence) the dominant kernel
is the indexer (it streams 256 bytes of index key per visible position).  Its
average launch duration is measured here with HIP events around back-to-back
launches of the same call on the same stream; achieved = algorithmic bytes per
launch / that duration, against the 8 TB/s HBM3E peak.  Algorithmic bytes per
row = 256 n (keys) + 8192 (q) + 128 (w).  The roofline object's `step` entry
prices the whole step the same way: algorithmic bytes of the path per step
(256 n + 1152 min(n, 2048) + 221,312 per row) over the measured step time.

The default run (the batched-decode workload) also measures the 8,192-token
causal prefill (`prefill_c2`): the step, the indexer and the attention, each
timed alone with HIP events, in FLOPs against the bf16 matrix-core peak; and
the long-context decode step, 16 sequences x 202,752 positions
(`long_decode_c4`), in algorithmic bytes against the HBM peak.

Workloads whose rows share a sequence (a prefill chunk) read each key once per
32-row block and are matrix-core work: there the indexer (8,192 FLOP per row
and visible position) and the attention (139,264 FLOP per row and selected
position) are priced in FLOPs against the 2.5 PFLOP/s bf16 peak, and the
roofline object names the attention kernel, timed alone in the same way.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

METRIC = "DSA decode tokens/s (indexer+top2048+sparse MLA) & % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16 matrix-core peak, TFLOP/s
K_TOP = 2048


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # Fifty warmup steps: for the first few milliseconds of load the chip runs
    # a c3 step at ~158 us, settling to ~152 us after (measured with 3 and
    # with 50 or 100 warmup steps).
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--config", default="c3", help="workload: c1 | c2 | c3 | c4 | c5")
    p.add_argument("--no-prefill", dest="prefill", action="store_false",
                   help="skip the 8,192-token prefill measurement that accompanies a decode workload")
    p.add_argument("--no-long", dest="long", action="store_false",
                   help="skip the long-context decode step (16 x 202,752) that accompanies the default workload")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU baseline budget (oracle)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-paged", dest="paged", action="store_false",
                   help="skip timing the step over paged caches")
    p.add_argument("--no-index-share", dest="index_share", action="store_false",
                   help="skip timing a 4-layer IndexShare group (1 full + 3 shared layers)")
    p.add_argument("--mode", default="decode", choices=["decode", "copy"],
                   help="copy: a plain device-to-device copy of --copy-mib MiB, repeated --steps times, to "
                        "calibrate HBM byte counters against a kernel of known traffic")
    p.add_argument("--copy-mib", type=int, default=1024)
    return p.parse_args()


def src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(REPO, "sparse_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workload_label(w):
    vis = w.visible_len
    if w.name == "c3":
        return "batched decode: 64 sequences x 32,768 positions, one query row each, top-2048"
    if w.name == "c4":
        return "long-context decode: 16 sequences x 202,752 positions, one query row each, top-2048"
    if w.name == "c1":
        return "decode: 1 sequence x 4,096 positions, top-2048"
    return f"{w.description} ({len(vis)} rows)"


def traffic_from_profiles(kernel, workload, current_hash):
    """HBM bytes per launch from committed rocprofv3 counter summaries, only if
    they were taken on the current kernel source."""
    path = os.path.join(REPO, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != current_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, x, budget_s):
    import oracle
    from sparse_attention_amd import workloads as wl

    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)

    def run(rows):
        y = {k: v for k, v in x.items()}
        for key in ("q_idx", "w", "q_abs", "visible_len", "row_cache_base"):
            y[key] = x[key][rows]
        t = time.perf_counter()
        oracle.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"], y["k_idx"], y["q_abs"],
                           y["kv_latent"], K_TOP, wl.INDEX_SCALE, wl.SOFTMAX_SCALE)
        return time.perf_counter() - t

    R = w.num_rows
    # Rows spread evenly over the batch; the sample grows (and then repeats)
    # until it has cost about budget_s of wall time on all host cores.
    t1 = run([0])
    m = int(max(1, min(R, budget_s / max(t1, 1e-3) * 0.5)))
    rows = np.unique(np.linspace(0, R - 1, m).astype(np.int64))
    done, dt, passes = 0, 0.0, 0
    while dt < budget_s and passes < 1000:
        dt += run(rows)
        done += len(rows)
        passes += 1
    res = {"value": done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{len(rows)} of {R} decode rows of the same workload x {passes} passes (full rows: indexer "
                     f"over every visible position, top-{K_TOP}, 64-head attention), fp64, {dt:.1f} s"}
    # The same oracle on one thread, over the first rows of the sample, for
    # about a third of the budget.
    oracle.set_threads(1)
    t1 = run(rows[:1])
    m1 = int(max(1, min(len(rows), budget_s / 3 / max(t1, 1e-3))))
    dt1 = t1 + (run(rows[1:m1]) if m1 > 1 else 0.0)
    oracle.set_threads(cores)
    res["single_thread"] = {"value": m1 / dt1, "unit": "tokens/s", "cores": 1,
                            "sample": f"{m1} of the rows above, once, {dt1:.1f} s"}
    return res


def measure_prefill(dsa, wl, torch, dev, stream, steps, warmup, name="c2"):
    """Step, indexer and attention of a prefill workload, each timed alone
    over `steps` back-to-back launches (HIP events on the launch stream), in
    FLOPs against the bf16 peak."""
    w = wl.config(name)
    log(f"[bench] generating {w.name}: {w.num_rows} rows")
    x = w.generate()

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    R, maxv = w.num_rows, w.max_visible
    q_idx, wts, k_idx = bf(x["q_idx"]), torch.from_numpy(x["w"]).to(dev), bf(x["k_idx"])
    q_abs, kv = bf(x["q_abs"]), bf(x["kv_latent"])
    rows = dsa.Rows(torch.from_numpy(x["visible_len"]).to(dev), torch.from_numpy(x["row_cache_base"]).to(dev), maxv)
    idx = torch.empty((R, K_TOP), dtype=torch.int32, device=dev)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, 64), dtype=torch.float32, device=dev)
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, maxv, K_TOP), dev)
    ld = (maxv + 3) // 4 * 4
    scores = torch.empty((R, ld), dtype=torch.float32, device=dev)
    ws_at = dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, K_TOP), dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_step = timed(lambda: dsa.dsa_decode_step(rows, q_idx, wts, k_idx, wl.INDEX_SCALE, q_abs, kv, wl.SOFTMAX_SCALE,
                                                 K_TOP, idx, out, lse, ws, stream=stream))
    ms_idx = timed(lambda: dsa.dsa_indexer_scores(rows, q_idx, wts, k_idx, wl.INDEX_SCALE, scores, stream=stream))
    ms_attn = timed(lambda: dsa.dsa_sparse_mla_attn(rows, q_abs, kv, idx, K_TOP, wl.SOFTMAX_SCALE, out, lse, ws_at,
                                                    stream=stream))
    n = x["visible_len"].astype(np.int64)
    idx_flops = int(8192 * np.sum(n))
    attn_flops = int(139264 * np.sum(np.minimum(n, K_TOP)))

    def mfma_entry(ms, flops):
        tfs = flops / (ms * 1e-3) / 1e12
        return {"us": round(ms * 1e3, 2), "alg_flops": flops, "tflops": round(tfs, 2),
                "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}

    res = {"workload": workload_label(w), "rows": R, "us_per_step": round(ms_step * 1e3, 2),
           "rows_per_s": round(R / (ms_step * 1e-3), 1),
           "indexer": mfma_entry(ms_idx, idx_flops), "attention": mfma_entry(ms_attn, attn_flops),
           "step_alg_flops": idx_flops + attn_flops,
           "step_mfma_frac": round((idx_flops + attn_flops) / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)}
    log(f"[bench] {w.name} prefill: step {ms_step * 1e3:.1f} us, indexer {ms_idx * 1e3:.1f} us "
        f"({res['indexer']['mfma_frac']:.3f} of bf16 peak), attention {ms_attn * 1e3:.1f} us "
        f"({res['attention']['mfma_frac']:.3f})")
    del q_idx, wts, k_idx, q_abs, kv, idx, out, lse, ws, scores, ws_at
    return res


def measure_long_decode(dsa, wl, torch, dev, stream, steps, warmup, name="c4"):
    """The whole decode step of the long-context workload, timed over `steps`
    back-to-back launches (HIP events on the launch stream), in algorithmic
    bytes against the HBM peak."""
    w = wl.config(name)
    log(f"[bench] generating {w.name}: {w.num_rows} rows, {w.cache_rows} cache rows")
    x = w.generate()

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    R, maxv = w.num_rows, w.max_visible
    q_idx, wts, k_idx = bf(x["q_idx"]), torch.from_numpy(x["w"]).to(dev), bf(x["k_idx"])
    q_abs, kv = bf(x["q_abs"]), bf(x["kv_latent"])
    del x
    rows = dsa.Rows(torch.from_numpy(w.visible_len).to(dev), torch.from_numpy(w.row_cache_base).to(dev), maxv,
                    flags=dsa.ROWS_DISTINCT_SEQUENCES)
    idx = torch.empty((R, K_TOP), dtype=torch.int32, device=dev)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, 64), dtype=torch.float32, device=dev)
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, maxv, K_TOP), dev)

    def step():
        dsa.dsa_decode_step(rows, q_idx, wts, k_idx, wl.INDEX_SCALE, q_abs, kv, wl.SOFTMAX_SCALE, K_TOP, idx, out, lse,
                            ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n = w.visible_len.astype(np.int64)
    nbytes = int(np.sum(256 * n + 1152 * np.minimum(n, K_TOP) + 82048 + 139264))
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": workload_label(w), "rows": R, "us_per_step": round(ms * 1e3, 2),
           "tokens_per_s": round(R / (ms * 1e-3), 1), "step_alg_bytes": nbytes, "achieved_gbs": round(gbs, 1),
           "step_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    log(f"[bench] {w.name} decode: {ms * 1e3:.1f} us/step, {res['step_hbm_frac']:.3f} of HBM peak")
    del q_idx, wts, k_idx, q_abs, kv, idx, out, lse, ws
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): the library has "
              f"no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_amd as dsa
    from sparse_attention_amd import workloads as wl

    if args.mode == "copy":
        dev = torch.device("cuda:0")
        nbytes = args.copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                          "launches": args.warmup + args.steps}), flush=True)
        return

    dsa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.config(args.config)
    log(f"[bench] generating {w.name}: {w.num_rows} rows, {w.cache_rows} cache rows")
    t = time.perf_counter()
    x = w.generate()
    log(f"[bench] inputs ready in {time.perf_counter() - t:.1f} s")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    R, maxv = w.num_rows, w.max_visible
    q_idx, wts, k_idx = bf(x["q_idx"]), torch.from_numpy(x["w"]).to(dev), bf(x["k_idx"])
    q_abs, kv = bf(x["q_abs"]), bf(x["kv_latent"])
    # Decode batches promise one query row per sequence (a performance hint).
    distinct = len(np.unique(x["row_cache_base"])) == R
    rows = dsa.Rows(torch.from_numpy(x["visible_len"]).to(dev), torch.from_numpy(x["row_cache_base"]).to(dev), maxv,
                    flags=dsa.ROWS_DISTINCT_SEQUENCES if distinct else 0)
    idx = torch.empty((R, K_TOP), dtype=torch.int32, device=dev)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, 64), dtype=torch.float32, device=dev)
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, maxv, K_TOP), dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        dsa.dsa_decode_step(rows, q_idx, wts, k_idx, wl.INDEX_SCALE, q_abs, kv, wl.SOFTMAX_SCALE, K_TOP, idx, out,
                            lse, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"[bench] decode step: {ms_step * 1e3:.1f} us/step over {args.steps} steps")

    # The same steps one by one (an event pair around each): the median step.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms_median = float(np.median([a.elapsed_time(b) for a, b in ev]))

    # Small workloads fit the 256 MB last-level cache, so the steps above run
    # warm; here a 512 MB buffer is written before each step (untimed) to
    # evict the inputs first.
    cold = None
    cache_bytes = w.cache_rows * (128 + 576) * 2
    if cache_bytes < (256 << 20):
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ts = []
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            a, b = ev[i]
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        cold = {"median_us": round(float(np.median(ts)) * 1e3, 2), "flush_bytes": 512 << 20}
        log(f"[bench] cold step (512 MB flushed before each): {cold['median_us']:.1f} us median")
        del flush

    # Dominant kernel alone: the indexer, same rows and launch configuration.
    ld = (maxv + 3) // 4 * 4
    scores = torch.empty((R, ld), dtype=torch.float32, device=dev)

    def idx_launch():
        dsa.dsa_indexer_scores(rows, q_idx, wts, k_idx, wl.INDEX_SCALE, scores, stream=stream)

    for _ in range(args.warmup):
        idx_launch()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        idx_launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_idx = e0.elapsed_time(e1) / args.steps
    n = x["visible_len"].astype(np.int64)
    alg_bytes = int(np.sum(256 * n + 8192 + 128))
    achieved = alg_bytes / (ms_idx * 1e-3) / 1e9
    if distinct:
        log(f"[bench] indexer: {ms_idx * 1e3:.1f} us/launch, {achieved:.0f} GB/s algorithmic")
    else:
        log(f"[bench] indexer: {ms_idx * 1e3:.1f} us/launch")

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # Decode batches: the other two kernels of the step, each timed alone on
    # the step's own data (the indexer's scores, the step's index lists), in
    # algorithmic bytes against the HBM peak.  Top-k: 4 B per visible score
    # read + the index lists written.  Attention (with its split combine):
    # 1152 B per selected latent row + q_abs, out_latent, lse and the index
    # lists per row.
    decode_kernels = None
    if distinct:
        ws_tk = dsa.workspace(dsa.dsa_topk_workspace_size(R, maxv, K_TOP), dev)
        idx_tk = torch.empty_like(idx)
        ms_tk = timed(lambda: dsa.dsa_topk_select(rows, scores, K_TOP, idx_tk, ws_tk, stream=stream))
        ws_at = dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, K_TOP), dev)
        ms_at = timed(lambda: dsa.dsa_sparse_mla_attn(rows, q_abs, kv, idx, K_TOP, wl.SOFTMAX_SCALE, out, lse, ws_at,
                                                      stream=stream))
        tk_bytes = int(4 * np.sum(n) + 4 * R * K_TOP)
        at_bytes = int(1152 * np.sum(np.minimum(n, K_TOP)) + R * (73728 + 131072 + 256 + 4 * K_TOP))

        def hbm_entry(ms, nbytes):
            gbs = nbytes / (ms * 1e-3) / 1e9
            return {"us": round(ms * 1e3, 2), "alg_bytes": nbytes, "gbs": round(gbs, 1),
                    "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}

        decode_kernels = {"topk": hbm_entry(ms_tk, tk_bytes), "attention_with_combine": hbm_entry(ms_at, at_bytes)}
        log(f"[bench] top-k: {ms_tk * 1e3:.1f} us, attention + combine: {ms_at * 1e3:.1f} us")
        del ws_tk, idx_tk, ws_at

    # Prefill-type workloads: both big kernels in FLOPs (see the module notes).
    prefill = None
    if not distinct:
        ws_at = dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, K_TOP), dev)
        ms_attn = timed(lambda: dsa.dsa_sparse_mla_attn(rows, q_abs, kv, idx, K_TOP, wl.SOFTMAX_SCALE, out, lse,
                                                        ws_at, stream=stream))
        idx_flops = int(8192 * np.sum(n))
        attn_flops = int(139264 * np.sum(np.minimum(n, K_TOP)))

        def mfma_entry(ms, flops):
            tfs = flops / (ms * 1e-3) / 1e12
            return {"us": round(ms * 1e3, 2), "alg_flops": flops, "tflops": round(tfs, 2),
                    "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}

        prefill = {"indexer": mfma_entry(ms_idx, idx_flops), "attention": mfma_entry(ms_attn, attn_flops),
                   "step_alg_flops": idx_flops + attn_flops,
                   "step_mfma_frac": round((idx_flops + attn_flops) / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
                                           4)}
        log(f"[bench] prefill: indexer {prefill['indexer']['tflops']:.0f} TFLOP/s, attention "
            f"{prefill['attention']['tflops']:.0f} TFLOP/s ({ms_attn * 1e3:.1f} us)")
        del ws_at

    # IndexShare: a 4-layer group in which one "full" layer runs the whole path
    # and three "shared" layers reuse its top-2048 list for their attention
    # (each with its own absorbed queries and latent cache).  Decode configs only.
    share = None
    if args.index_share and R <= 1024:
        n_shared = 3
        # Each shared layer's queries and latent cache: N(0,1) in bf16, drawn on
        # the device (only timed here; parity of this composition is a test).
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000)
        extra = [(torch.randn(q_abs.shape, generator=gen, device=dev).to(torch.bfloat16),
                  torch.randn(kv.shape, generator=gen, device=dev).to(torch.bfloat16)) for _ in range(n_shared)]
        ws_a = dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, K_TOP), dev)
        out_s = torch.empty_like(out)
        lse_s = torch.empty_like(lse)

        def group():
            step()
            for qa_l, kv_l in extra:
                dsa.dsa_sparse_mla_attn(rows, qa_l, kv_l, idx, K_TOP, wl.SOFTMAX_SCALE, out_s, lse_s, ws_a,
                                        stream=stream)

        for _ in range(args.warmup):
            group()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            group()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_group = e0.elapsed_time(e1) / args.steps
        share = {"layers_per_group": 1 + n_shared, "us_per_group": round(ms_group * 1e3, 2),
                 "tokens_per_s_per_group": round(R / (ms_group * 1e-3), 1),
                 "us_per_layer": round(ms_group * 1e3 / (1 + n_shared), 2),
                 "us_if_every_layer_ran_the_indexer": round(ms_step * 1e3 * (1 + n_shared), 2)}
        log(f"[bench] IndexShare group (1 full + {n_shared} shared layers): {ms_group * 1e3:.1f} us, "
            f"{R / (ms_group * 1e-3):.0f} tokens/s per group")
        del extra

    # Paged caches: the same step over pools of 64-position blocks scattered by
    # a random permutation (block tables per sequence).  Workloads whose
    # sequence lengths are all multiples of the block size.
    paged = None
    PB = 64
    if args.paged and np.all(w.seq_len % PB == 0):
        nblk = int(w.cache_rows // PB)
        gen_p = torch.Generator(device=dev)
        gen_p.manual_seed(2024)
        perm = torch.randperm(nblk, generator=gen_p, device=dev)
        kpool = torch.empty_like(k_idx).view(nblk, PB, 128)
        lpool = torch.empty_like(kv).view(nblk, PB, 576)
        kpool[perm] = k_idx.view(nblk, PB, 128)
        lpool[perm] = kv.view(nblk, PB, 576)
        nb = int(w.seq_len.max() // PB)
        bt = torch.zeros((len(w.seq_len), nb), dtype=torch.int32, device=dev)
        for s_, (b0, T) in enumerate(zip(w.seq_base, w.seq_len)):
            bt[s_, :T // PB] = perm[b0 // PB: (b0 + T) // PB].to(torch.int32)
        seq_of_row = np.searchsorted(w.seq_base, x["row_cache_base"], side="right") - 1
        prow = dsa.Rows(rows.visible_len, torch.from_numpy(seq_of_row.astype(np.int64)).to(dev), maxv,
                        flags=rows.flags)
        pg = dsa.Paged(bt, PB)
        ws_p = dsa.workspace(dsa.dsa_decode_step_paged_workspace_size(R, maxv, K_TOP), dev)
        idx_p = torch.empty_like(idx)
        ms_paged = timed(lambda: dsa.dsa_decode_step_paged(prow, pg, q_idx, wts, kpool, wl.INDEX_SCALE, q_abs, lpool,
                                                           wl.SOFTMAX_SCALE, K_TOP, idx_p, out, lse, ws_p,
                                                           stream=stream))
        paged = {"block_size": PB, "us_per_step": round(ms_paged * 1e3, 2),
                 "tokens_per_s": round(R / (ms_paged * 1e-3), 1), "vs_packed": round(ms_step / ms_paged, 4)}
        log(f"[bench] paged step (blocks of {PB}): {ms_paged * 1e3:.1f} us/step")
        del kpool, lpool

    # The projections on either side of the path (query absorption before it,
    # V up-projection after it), timed alone at this workload's row count
    # (at most 8192 rows), with synthetic kv_b_proj weights.
    Rp = min(R, 8192)
    px = wl.projection_inputs(Rp)
    qn, qp, kvb = bf(px["q_nope"]), bf(px["q_pe"]), bf(px["kv_b"])
    o_lat = torch.from_numpy(px["o"]).to(dev)
    qa_p = torch.empty((Rp, 64, 576), dtype=torch.bfloat16, device=dev)
    up = torch.empty((Rp, 64, 256), dtype=torch.float32, device=dev)

    ms_ab = timed(lambda: dsa.dsa_absorb_queries(qn, qp, kvb, qa_p, stream=stream))
    ms_up = timed(lambda: dsa.dsa_v_up_proj(o_lat, kvb, up, stream=stream))
    ab_bytes = 64 * 192 * 512 * 2 + Rp * 64 * (192 + 64 + 576) * 2
    up_bytes = 64 * 256 * 512 * 2 + Rp * 64 * (512 * 4 + 256 * 4)
    ab_flops = 2 * Rp * 64 * 192 * 512
    up_flops = 2 * Rp * 64 * 512 * 256

    def proj_entry(ms, nbytes, flops):
        gbs = nbytes / (ms * 1e-3) / 1e9
        tfs = flops / (ms * 1e-3) / 1e12
        return {"us": round(ms * 1e3, 2), "alg_bytes": nbytes, "gbs": round(gbs, 1),
                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "tflops": round(tfs, 2),
                "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}

    projections = {"rows": Rp, "absorb_queries": proj_entry(ms_ab, ab_bytes, ab_flops),
                   "v_up_proj": proj_entry(ms_up, up_bytes, up_flops)}
    log(f"[bench] absorb_queries: {ms_ab * 1e3:.1f} us, v_up_proj: {ms_up * 1e3:.1f} us ({Rp} rows)")

    # The cache writers for this workload's new tokens (one per row, at most
    # 8192): both projections of the hidden state, the norms, RoPE and the
    # scatter into two caches of the same shape as the path's.
    Nw = min(R, 8192)
    cw = wl.cache_write_inputs(Nw, max_position=maxv, cache_rows=Nw)
    cw["slots"] = np.arange(Nw, dtype=np.int64)  # every token written
    cw_t = {k: (bf(v) if v.dtype == np.uint16 else torch.from_numpy(v).to(dev))
            for k, v in cw.items() if isinstance(v, np.ndarray)}
    kc_w = torch.empty((Nw, 128), dtype=torch.bfloat16, device=dev)
    lc_w = torch.empty((Nw, 576), dtype=torch.bfloat16, device=dev)
    ws_w = dsa.workspace(dsa.dsa_cache_write_workspace_size(Nw), dev)
    ms_cw = timed(lambda: dsa.dsa_cache_write(cw_t["hidden"], cw_t["wk"], cw_t["k_norm_weight"], cw_t["k_norm_bias"],
                                              1e-6, cw_t["kv_a"], cw_t["kv_norm_weight"], 1e-5, cw_t["positions"],
                                              cw_t["slots"], 1e6, kc_w, lc_w, ws_w, stream=stream))
    cw_bytes = 704 * 6144 * 2 + (128 * 2 + 512) * 4 + Nw * (6144 * 2 + 128 * 2 + 576 * 2 + 4 + 8)
    cw_flops = 2 * Nw * 6144 * 704
    cache_write = dict(tokens=Nw, **proj_entry(ms_cw, cw_bytes, cw_flops))
    log(f"[bench] cache_write: {ms_cw * 1e3:.1f} us ({Nw} tokens)")

    # Step-level algorithmic bytes (whole path).
    step_bytes = int(np.sum(256 * n + 1152 * np.minimum(n, K_TOP) + 82048 + 139264))
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # The 8,192-token causal prefill beside a decode workload (matrix-core
    # bound; timed alone, its inputs freed afterwards).
    prefill_c2 = None
    if args.prefill and prefill is None:
        prefill_c2 = measure_prefill(dsa, wl, torch, dev, stream, args.steps, args.warmup)
    # The long-context decode batch beside the default workload (HBM bound;
    # timed alone, its inputs freed afterwards).
    long_c4 = None
    if args.long and w.name == "c3":
        long_c4 = measure_long_decode(dsa, wl, torch, dev, stream, args.steps, args.warmup)
    traffic = traffic_from_profiles("indexer", w.name, src_hash(["indexer.hip", "dsa_device.h"]))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of rows")
        cpu = cpu_baseline(w, x, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']:.3f} tokens/s on {cpu['cores']} cores")

    value = R / (ms_step * 1e-3)
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "median_ms_per_step": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_label(w), "rows": R, "max_visible": maxv, "topk": K_TOP,
                   "index_heads": 32, "index_dim": 128, "heads": 64, "latent_row": 576},
        "roofline": ({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                      "kernel": "indexer_rows_kernel<false>", "kernel_us": round(ms_idx * 1e3, 2),
                      "alg_bytes_per_launch": alg_bytes,
                      "step": {"alg_bytes": step_bytes, "us": round(ms_step * 1e3, 2),
                               "achieved": round(step_gbs, 1), "frac": round(step_gbs / HBM_PEAK_GBS, 4)}}
                     if prefill is None else
                     {"bound": "mfma", "achieved": prefill["attention"]["tflops"], "peak": MFMA_BF16_PEAK_TFS,
                      "unit": "TFLOP/s", "frac": prefill["attention"]["mfma_frac"], "traffic": None,
                      "kernel": "sparse_mla_kernel<true>", "kernel_us": prefill["attention"]["us"],
                      "alg_flops_per_launch": prefill["attention"]["alg_flops"]}),
        "cpu_baseline": cpu,
        "projections": projections,
        "index_share": share,
        "cache_write": cache_write,
        "paged": paged,
        "decode_kernels": decode_kernels,
        "prefill": prefill,
        "prefill_c2": prefill_c2,
        "long_decode_c4": long_c4,
        "cold": cold,
        "step_alg_bytes": step_bytes if prefill is None else None,
        "step_hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if prefill is None else None,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
