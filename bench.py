"""Benchmark: linear-attention layer tokens/s per packed pass on one MI355X.

One step = one packed pass through la_scan_packed (all its launches: one for
d = 64 bf16 passes, else two or three, the form the library picks for the
pass, or --form) over one batch of synthetic input already resident in HBM.  The default workload
is one 7,400-token view with 8 branches of 48 tokens, H = 16, d = 64, bf16
(the pass size of the page "Serving 0.88M TPS from Two RTXs and Mac Minis",
section "Kernels", paragraph "One scan per pass").

Timing: W warm-up passes, then exactly K passes, both replayed as HIP graphs
on one stream and bracketed by torch.cuda.synchronize().  Inputs rotate over
enough copies (>= 1 GiB in total) that each pass reads its q/k/v from HBM
rather than from the 256 MB Infinity Cache.  The roofline line is the whole
pass (its algorithmic bytes over the pass time from HIP events on the
stream the launches run on; in the single-launch form the pass is one
kernel); multi-launch forms also report launch 3 alone.  HBM traffic and MFMA
busy cycles come from committed rocprofv3 counter summaries (profiles/),
used only when they were taken on the current kernel sources.  The fp64 CPU
oracle is timed on the host cores on the same workload (cpu_baseline).

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "view7400_br8x48_h16_d64_bf16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--block-chunks", type=int, default=None)
    ap.add_argument("--form", choices=["auto", "one", "two", "three"], default="auto",
                    help="scan form: one launch (d 64 bf16), two launches (no prefix "
                         "launch), three, or the library's choice for the pass shape")
    ap.add_argument("--rotate-gib", type=float, default=1.0,
                    help="total size of the rotated input copies")
    ap.add_argument("--eager", action="store_true",
                    help="plain stream launches instead of HIP graphs (for profilers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU work of the oracle baseline")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, --steps times "
                         "(reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--launch-floor", action="store_true",
                    help="only time three chained near-empty launches per step")
    ap.add_argument("--shards", type=int, default=0,
                    help="instead of the headline: split the workload's one request "
                         "into this many branch shards and time them with and without "
                         "the view-state cache against the unsplit pass")
    ap.add_argument("--split-fp32", action="store_true",
                    help="fp32 workloads: evaluate products as three bf16 MFMAs over hi/lo "
                         "operand splits (LA_F32_SPLIT) instead of fp32 MFMAs")
    ap.add_argument("--attention", action="store_true",
                    help="instead of the headline: time the tree-masked softmax attention "
                         "(la_attn_packed) of the workload against the bf16 MFMA peak")
    ap.add_argument("--cost-model", type=int, default=0,
                    help="instead of the headline: time this many random pass shapes and "
                         "fit the three-term cost model t = c0 + c1*sum(view) + c2*branches")
    return ap.parse_args()


def calibrate_copy(mib, steps):
    """A plain copy kernel of known size (torch elementwise add: reads mib MiB,
    writes mib MiB per launch), timed with HIP events over `steps` launches
    rotating over enough buffers (>= 1 GiB) to miss the Infinity Cache.  The
    same command under rocprofv3 --pmc gives the FETCH_SIZE / WRITE_SIZE
    readings of a known byte count."""
    import torch
    n = mib * 2**20 // 4
    nbuf = max(2, -(-2**30 // (2 * n * 4)))
    bufs = [(torch.ones(n, dtype=torch.float32, device="cuda:0"),
             torch.empty(n, dtype=torch.float32, device="cuda:0")) for _ in range(nbuf)]
    for a, b in bufs:
        torch.add(a, 1.0, out=b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        a, b = bufs[i % nbuf]
        torch.add(a, 1.0, out=b)      # one elementwise kernel: reads a, writes b
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4, "launches": steps,
                      "us_per_launch": us, "GBps": 2 * n * 4 / (us * 1e-6) / 1e9}), flush=True)


def launch_floor(steps, quiet=False, n_launches=3):
    """n_launches dependent launches of the library's smallest kernel (a
    64 KiB state export) per step, replayed as a HIP graph: the fixed cost of
    a pass of that many launches with no work in it.  Returns microseconds
    per step."""
    import torch
    import chunked_linear_attention_packed_amd as la
    src = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device="cuda:0")
    dst = torch.zeros((1, 64, 64), dtype=torch.float32, device="cuda:0")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        la.export_view_state(src, 0, dst, stream=st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for _ in range(steps):
            for _ in range(n_launches):
                la.export_view_state(src, 0, dst, stream=st)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(st):
        e0.record(st)
        g.replay()
        e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    if not quiet:
        print(json.dumps({"calibration": "launch floor", "launches_per_step": n_launches,
                          "us_per_step": us}), flush=True)
    return us


def _oracle_task(args):
    q, k, v, so, bp = args
    import oracle
    t = time.perf_counter()
    oracle.scan_recurrence(q, k, v, so, bp)
    return time.perf_counter() - t


def cpu_baseline(w, so, bp, target_s):
    """The fp64 oracle, unmodified, over the whole pass; heads are split across
    a process pool (heads are independent).  Repeated until about target_s
    seconds of CPU work; median wall time of the repeats."""
    import numpy as np
    import torch
    from concurrent.futures import ProcessPoolExecutor
    cores = min(len(os.sched_getaffinity(0)), 16, w.H)
    q, k, v = (x.to(torch.float32).numpy() for x in (w.q, w.k, w.v))
    bounds = np.linspace(0, w.H, cores + 1).astype(int)
    tasks = [(q[:, a:b], k[:, a:b], v[:, a:b], so, bp) for a, b in zip(bounds[:-1], bounds[1:])]
    walls, cpu = [], 0.0
    with ProcessPoolExecutor(max_workers=cores) as ex:
        while cpu < target_s or len(walls) < 3:
            t = time.perf_counter()
            parts = list(ex.map(_oracle_task, tasks))
            walls.append(time.perf_counter() - t)
            cpu += sum(parts)
            if len(walls) >= 20:
                break
    wall = float(np.median(walls))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": w.n_tokens / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host_cores": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"whole pass ({w.n_tokens} tokens x {w.H} heads), {len(walls)} repeats, "
                      f"median wall {wall:.3f} s, {cpu:.1f} s CPU work, {model}"}


def _graph_us(fn, steps, warmup, stream, eager=False):
    """Mean device time of fn() over `steps` calls replayed as one HIP graph
    (eager stream launches with eager=True), after `warmup` calls."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(max(warmup, 1)):
            fn()
    torch.cuda.synchronize()
    if eager:
        run = lambda: [fn() for _ in range(steps)]
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(steps):
                fn()
        run = g.replay
        with torch.cuda.stream(stream):
            run()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def shard_bench(a):
    """Branch shards of one long request on one GPU (section "Long Requests":
    shards each need the full view; cached view states avoid recomputing it).

    The workload's single request (view V, branches b_1..b_n) is scored three
    ways, each as one step of the graph-replayed timing:
      unsplit   one pass over the view and all branches;
      cached    shard 0 = view + its branches, its view state stored in a
                ViewStateCache, then shards 1..S-1 as branch-only passes
                seeded from the cache pool;
      uncached  every shard = view + its branches (the view recomputed S times).
    All passes use the unsplit pass's block size, so the shard outputs equal
    the unsplit ones bit for bit (checked here).  Inputs are already in HBM."""
    import numpy as np
    import torch
    import chunked_linear_attention_packed_amd as la
    import synth
    w = synth.workload(a.workload)
    if len(w.view_len) != 1 or w.view_len[0] < 1:
        raise SystemExit("--shards needs a workload with one request that has a view")
    V, lens, H, d = int(w.view_len[0]), np.asarray(w.branch_len), w.H, w.d
    n, S = len(lens), a.shards
    if not 1 <= S <= n:
        raise SystemExit(f"--shards must be between 1 and the {n} branches")
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    off = np.concatenate([[0], np.cumsum(np.concatenate([[V], lens]))]).astype(np.int64)
    plan_u = la.pack([V], [n], lens, heads=H, block_chunks=a.block_chunks)
    G = plan_u.info.block_chunks
    stream = torch.cuda.Stream(dev)

    def make(plan, qq, kk, vv, ext=None):
        qq, kk, vv = qq.contiguous(), kk.contiguous(), vv.contiguous()
        out = torch.empty_like(vv)
        fin = torch.empty((plan.info.n_views, H, d, d), dtype=torch.float32, device=dev)
        ws = la.new_workspace(plan, H, d, qq.dtype, dev)
        plan.device_plan(dev)
        return dict(plan=plan, q=qq, k=kk, v=vv, out=out, fin=fin, ws=ws, ext=ext)

    def run(p):
        la.scan_packed(p["q"], p["k"], p["v"], p["plan"], ext_state=p["ext"], out=p["out"],
                       final_state=p["fin"], workspace=p["ws"], stream=stream)

    unsplit = make(plan_u, q, k, v)
    cache = la.ViewStateCache(1, H, d, dev)
    row, _ = cache.reserve(0)
    parts = np.array_split(np.arange(n), S)
    cached, uncached = [], []
    for s, idx in enumerate(parts):
        b0, b1 = int(idx[0]), int(idx[-1]) + 1
        t0, t1 = int(off[1 + b0]), int(off[1 + b1])
        sel = torch.cat([torch.arange(0, V), torch.arange(t0, t1)]).to(dev)
        full = make(la.pack([V], [b1 - b0], lens[b0:b1], heads=H, block_chunks=G),
                    q[sel], k[sel], v[sel])
        uncached.append(full)
        if s == 0:
            cached.append(full)
        else:
            cached.append(make(la.pack([0], [b1 - b0], lens[b0:b1], heads=H, block_chunks=G,
                                       ext_row=[row]),
                               q[t0:t1], k[t0:t1], v[t0:t1], ext=cache.pool))

    def step_unsplit():
        run(unsplit)

    def step_cached():
        run(cached[0])
        la.export_view_state(cached[0]["fin"], 0, cache.pool[row], stream=stream)
        for p in cached[1:]:
            run(p)

    def step_uncached():
        for p in uncached:
            run(p)

    us_u = _graph_us(step_unsplit, a.steps, a.warmup, stream, a.eager)
    us_c = _graph_us(step_cached, a.steps, a.warmup, stream, a.eager)
    us_n = _graph_us(step_uncached, a.steps, a.warmup, stream, a.eager)
    # the shard outputs are the unsplit outputs, bit for bit
    match = True
    for s, idx in enumerate(parts):
        t0, t1 = int(off[1 + idx[0]]), int(off[1 + idx[-1] + 1])
        got = cached[s]["out"][V:] if s == 0 else cached[s]["out"]
        match &= bool(torch.equal(got, unsplit["out"][t0:t1]))
    T = int(off[-1])
    print(json.dumps({
        "experiment": "branch shards from a cached view state, one GPU",
        "workload": a.workload, "tokens": T, "view_tokens": V, "branches": n, "shards": S,
        "heads": H, "d": d, "dtype": w.dtype, "block_chunks": G,
        "launch": "eager" if a.eager else "hip_graph", "steps": a.steps,
        "unsplit_us": us_u, "cached_shards_us": us_c, "uncached_shards_us": us_n,
        "uncached_over_cached": us_n / us_c, "cached_over_unsplit": us_c / us_u,
        "tokens_per_s_cached": T / (us_c * 1e-6),
        "shard_outputs_equal_unsplit": match,
        "page_context": "the page reports shards without the cache taking 3.4x as long as "
                        "with it (whole model, 349 requests, older hardware)",
    }), flush=True)
    cache.close()


MFMA_BF16_PEAK_TFLOPS = 2500.0


def attention_bench(a):
    """The softmax-attention layer of the same packed pass (la_attn_packed):
    scores q.k and weighted values for every (token, attended key, head),
    4*d FLOPs each, against the dense bf16 MFMA peak.  Inputs rotate like the
    headline's; graph-replayed timing."""
    import numpy as np
    import torch
    import chunked_linear_attention_packed_amd as la
    import synth
    w = synth.workload(a.workload)
    if w.dtype != "bf16":
        raise SystemExit("--attention runs bf16 workloads")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H, block_chunks=1)
    so, bp = plan.seg_offsets, plan.branch_parent
    ap = la.attn_plan(so, bp)
    T, H, d = w.n_tokens, w.H, w.d
    pairs = 0
    for s_ in range(len(bp)):
        n = int(so[s_ + 1] - so[s_])
        p = int(bp[s_])
        lp = int(so[p + 1] - so[p]) if p >= 0 else 0
        pairs += n * lp + n * (n + 1) // 2
    flops = 4 * d * H * pairs
    dev = torch.device("cuda:0")
    set_bytes = 4 * T * H * d * 2
    n_sets = min(64, max(2, int(np.ceil(a.rotate_gib * 2**30 / set_bytes))))
    q0, k0, v0 = (x.to(dev) for x in (w.q, w.k, w.v))
    sets = [dict(q=q0.clone(), k=k0.clone(), v=v0.clone(), out=torch.empty_like(v0))
            for _ in range(n_sets)]
    del q0, k0, v0
    ap.device_items(dev)
    stream = torch.cuda.Stream(dev)
    ctr = [0]

    def fn():
        s_ = sets[ctr[0] % n_sets]
        ctr[0] += 1
        la.attn_packed(s_["q"], s_["k"], s_["v"], ap, 1.0, out=s_["out"], stream=stream)

    us = _graph_us(fn, a.steps, a.warmup, stream, a.eager)
    tf = flops / (us * 1e-6) / 1e12
    cpu = None
    if not a.no_cpu_baseline:
        # the fp64 attention oracle, unmodified, on a bounded sample: evenly
        # spaced query rows (all heads) until ~cpu_seconds of work; a row's
        # cost grows with its key count, so the sample spans the whole pass
        import numpy as np
        import oracle
        rows = np.linspace(0, T - 1, 4096).astype(int)
        done, t0 = 0, time.perf_counter()
        pairs_done = 0
        sizes = []
        for s_ in range(len(bp)):
            n = int(so[s_ + 1] - so[s_])
            p = int(bp[s_])
            lp = int(so[p + 1] - so[p]) if p >= 0 else 0
            sizes += [lp + i + 1 for i in range(n)]
        for start in range(0, len(rows), 64):
            chunk = rows[start:start + 64].tolist()
            oracle.attention_rows(w.q, w.k, w.v, so, bp, 1.0, chunk)
            done += len(chunk)
            pairs_done += sum(sizes[r] for r in chunk)
            if time.perf_counter() - t0 > a.cpu_seconds:
                break
        wall = time.perf_counter() - t0
        # scale by attended-key pairs: the sample's pairs/s over the pass's pairs
        rate = pairs_done / wall
        cpu = {"value": T * rate / pairs / 1.0, "unit": "tokens/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{done} evenly spaced query rows x {H} heads ({pairs_done} attended "
                         f"key pairs of {pairs}), {wall:.1f} s, one process; scaled to the "
                         f"whole pass by attended pairs"}
    print(json.dumps({
        "experiment": "tree-masked softmax attention over the packed pass",
        "workload": a.workload, "tokens": T, "heads": H, "d": d, "dtype": "bf16",
        "work_items": int(len(ap.items)), "launch": "eager" if a.eager else "hip_graph",
        "steps": a.steps, "us_per_pass": us, "tokens_per_s": T / (us * 1e-6),
        "algorithmic_flops": flops,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                     "kernel": "attn_kernel_bf16"},
        "cpu_baseline": cpu,
    }), flush=True)


def cost_model_bench(a):
    """Pass times of random pass shapes and the page's three-term cost model
    fitted to them (section "Cost Model").  Shapes: 1-8 requests, views
    log-uniform in [500, 18000] tokens, 1-64 branches of 24-128 tokens per
    request (the page's ranges), H = 16, d = 64, bf16 -- seed 2024.  Each
    pass is timed as `steps` graph-replayed passes after its warm-up.  The
    fit uses the even-numbered shapes; the odd ones are predicted (hold-out).
    The structural variant (ours) is fitted the same way from each pass's
    plan: tokens and rounds of workgroups (the single launch holds one
    workgroup per CU: its LDS); the longest view's 512-token block count is
    recorded with each sample."""
    import numpy as np
    import torch
    import chunked_linear_attention_packed_amd as la
    from chunked_linear_attention_packed_amd import cost_model as cm
    import synth
    rng = np.random.default_rng(2024)
    H, d = 16, 64
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rows, struct = [], []
    for i in range(a.cost_model):
        r = int(rng.integers(1, 9))
        vl = np.round(np.exp(rng.uniform(np.log(500), np.log(18000), size=r))).astype(np.int32)
        bc = rng.integers(1, 65, size=r).astype(np.int32)
        bl = rng.integers(24, 129, size=int(bc.sum())).astype(np.int32)
        plan = la.pack(vl, bc, bl, heads=H, block_chunks=a.block_chunks)
        T = plan.info.n_tokens
        q, k, v = (x.to(dev) for x in synth.draw_qkv(rng, T, H, d, "bf16"))
        out = torch.empty_like(v)
        fin = torch.empty((plan.info.n_views, H, d, d), dtype=torch.float32, device=dev)
        ws = la.new_workspace(plan, H, d, q.dtype, dev)
        plan.device_plan(dev)
        fn = lambda: la.scan_packed(q, k, v, plan, out=out, final_state=fin, workspace=ws,
                                    stream=stream)
        us = _graph_us(fn, a.steps, a.warmup, stream, a.eager)
        rows.append((vl.tolist(), bc.tolist(), int(bl.sum()), T, us))
        work = plan.info.piece_items * H
        chain = -(-int(vl.max()) // 512)
        struct.append({"work_items": int(work), "chain_blocks": int(chain)})
        print(f"pass {i}: requests {r} tokens {T} branches {int(bc.sum())} "
              f"block_chunks {plan.info.block_chunks} {us:.1f} us", file=sys.stderr, flush=True)
        del q, k, v, out, fin, ws
    X = np.array([cm.features(vl, bc) for vl, bc, _, _, _ in rows])
    Xt = np.array([[1.0, float(np.sum(vl)), float(bt)] for vl, _, bt, _, _ in rows])
    Xs = np.array([cm.features_structural(T, st["work_items"], cus)
                   for (_, _, _, T, _), st in zip(rows, struct)])
    t = np.array([us for *_, us in rows])
    tr, te = np.arange(0, len(t), 2), np.arange(1, len(t), 2)

    def holdout(Xm):
        f = cm.fit(Xm[tr], t[tr])
        rel = (Xm[te] @ np.array(f["c"]) - t[te]) / t[te]
        f["holdout_rel_rms"] = float(np.sqrt(np.mean(rel ** 2))) if len(te) else None
        f["holdout_rel_max"] = float(np.max(np.abs(rel))) if len(te) else None
        return f

    print(json.dumps({
        "experiment": "three-term pass cost model",
        "model": "t_us = c0 + c1 * sum(view tokens) + c2 * branch rows",
        "heads": H, "d": d, "dtype": "bf16", "passes": len(t), "steps_per_pass": a.steps,
        "launch": "eager" if a.eager else "hip_graph",
        "fit_all": cm.fit(X, t), "fit_even_holdout_odd": holdout(X),
        "variant_branch_tokens": {"model": "t_us = c0 + c1 * sum(view) + c2 * sum(branch tokens)",
                                  "fit_all": cm.fit(Xt, t), "fit_even_holdout_odd": holdout(Xt)},
        "variant_structural": {"model": "t_us = c0 + c1 * tokens + c2 * ceil(workgroups / CUs)",
                               "cus": cus,
                               "fit_all": cm.fit(Xs, t), "fit_even_holdout_odd": holdout(Xs)},
        "samples": [{"view_len": vl, "branches": int(np.sum(bc)), "branch_tokens": bt,
                     "tokens": T, "us": us, **st}
                    for (vl, bc, bt, T, us), st in zip(rows, struct)],
    }), flush=True)


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this scan runs on a single MI355X and has no "
              "multi-GPU path (requests shard across GPUs with no exchange; see DESIGN.md). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import chunked_linear_attention_packed_amd as la
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.calibrate_copy_mib:
        calibrate_copy(a.calibrate_copy_mib, a.steps)
        return
    if a.launch_floor:
        launch_floor(a.steps)
        return
    if a.shards:
        shard_bench(a)
        return
    if a.cost_model:
        cost_model_bench(a)
        return
    if a.attention:
        attention_bench(a)
        return
    la.load_library()
    dev = torch.device("cuda:0")
    w = synth.workload(a.workload)
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H,
                   block_chunks=a.block_chunks)
    info = plan.info
    T, H, d = w.n_tokens, w.H, w.d
    s_el = 2 if w.dtype == "bf16" else 4
    set_bytes = 4 * T * H * d * s_el
    n_sets = max(2, int(np.ceil(a.rotate_gib * 2**30 / set_bytes)))
    n_sets = min(n_sets, 64)
    q0, k0, v0 = (x.to(dev) for x in (w.q, w.k, w.v))
    sets = []
    for i in range(n_sets):
        sets.append(dict(q=q0.clone(), k=k0.clone(), v=v0.clone(), out=torch.empty_like(v0)))
    del q0, k0, v0
    fin = torch.empty((info.n_views, H, d, d), dtype=torch.float32, device=dev)
    ws = la.new_workspace(plan, H, d, w.q.dtype, dev)
    plan.device_plan(dev)
    stream = torch.cuda.Stream(dev)
    if a.split_fp32 and w.dtype != "f32":
        raise SystemExit("--split-fp32 applies to fp32 workloads")
    form = None if a.form == "auto" else a.form
    code = la.LA_F32_SPLIT if a.split_fp32 else (la.LA_BF16 if w.dtype == "bf16" else la.LA_F32)
    n_launches = {"one": 1, "two": 2, "three": 3}.get(a.form) or la.scan_launches(plan, H, d,
                                                                                  code)

    def step(i, stages=la.STAGE_ALL):
        s = sets[i % n_sets]
        la.scan_packed(s["q"], s["k"], s["v"], plan, out=s["out"], final_state=fin,
                       workspace=ws, stream=stream, stages=stages, split_fp32=a.split_fp32,
                       form=form)

    # first pass eagerly (also validates arguments)
    with torch.cuda.stream(stream):
        for i in range(n_sets):
            step(i)
    torch.cuda.synchronize()

    def make_graph(n, stages=la.STAGE_ALL):
        if a.eager:
            return lambda: [step(i, stages) for i in range(n)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                step(i, stages)
        return g.replay

    warm = make_graph(a.warmup)
    timed = make_graph(a.steps)
    with torch.cuda.stream(stream):
        warm()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        timed()
        ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_ms / a.steps

    # two independent passes in flight: even passes on `stream`, odd ones on a
    # second stream, each stream with its own workspace and final_state (a
    # node scoring several passes at once); reported beside the headline,
    # which stays single-stream
    two_stream = None
    if not a.eager:
        s1 = torch.cuda.Stream(dev)
        ws2 = [ws, torch.zeros_like(ws)]
        fin2 = [fin, torch.empty_like(fin)]

        def step2(i):
            s_ = sets[i % n_sets]
            st_ = stream if i % 2 == 0 else s1
            la.scan_packed(s_["q"], s_["k"], s_["v"], plan, out=s_["out"],
                           final_state=fin2[i % 2], workspace=ws2[i % 2], stream=st_,
                           split_fp32=a.split_fp32, form=form)

        def make_graph2(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                s1.wait_stream(stream)
                for i in range(n):
                    step2(i)
                stream.wait_stream(s1)
            return g.replay

        warm2, timed2 = make_graph2(max(a.warmup, 2)), make_graph2(a.steps)
        with torch.cuda.stream(stream):
            warm2()
        torch.cuda.synchronize()
        e4, e5 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e4.record(stream)
            timed2()
            e5.record(stream)
        torch.cuda.synchronize()
        us2 = e4.elapsed_time(e5) * 1e3 / a.steps
        two_stream = {"us_per_pass": us2, "tokens_per_s": T / (us2 * 1e-6)}

    # warm: the same input set back to back, so at this size q/k/v stay in the
    # 256 MB Infinity Cache; labelled, never the headline
    warm_same = None
    if not a.eager:
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=stream):
            for _ in range(a.steps):
                step(0)
        with torch.cuda.stream(stream):
            gw.replay()
        torch.cuda.synchronize()
        e6, e7 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e6.record(stream)
            gw.replay()
            e7.record(stream)
        torch.cuda.synchronize()
        usw = e6.elapsed_time(e7) * 1e3 / a.steps
        warm_same = {"us_per_pass": usw, "tokens_per_s": T / (usw * 1e-6),
                     "inputs": "one set reused (cache-warm)"}
        del gw

    # launch 3 alone (reads what the last full pass left in ws / final_state);
    # the single-launch form has no separate output launch
    l3_us = None
    if n_launches > 1:
        out_only = make_graph(a.steps, la.STAGE_OUTPUT)
        with torch.cuda.stream(stream):
            out_only()
        torch.cuda.synchronize()
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e2.record(stream)
            out_only()
            e3.record(stream)
        torch.cuda.synchronize()
        l3_us = e2.elapsed_time(e3) * 1e3 / a.steps

    # algorithmic bytes: q, k, v read once and out written once per token-head;
    # final states written once per view and head
    per_token_head = d * (3 * s_el + s_el)
    l3_bytes = T * H * per_token_head
    pass_bytes = l3_bytes + info.n_views * H * d * d * 4
    achieved = l3_bytes / (l3_us * 1e-6) / 1e9 if l3_us else None
    # algorithmic matrix work per chunk of c tokens and head: q.S (2 c d^2),
    # the causal scores and weighted values (c (c + 1) 2d), and the chunk's
    # own state K^T V (2 c d^2) where a later chunk needs it (every chunk but
    # the last of a segment)
    so = plan.seg_offsets
    flops = 0
    for s_ in range(len(plan.branch_parent)):
        n = int(so[s_ + 1] - so[s_])
        full, rem = divmod(n, 64)
        sizes = [64] * full + ([rem] if rem else [])
        flops += sum(2 * c * d * d + c * (c + 1) * 2 * d for c in sizes)
        flops += sum(2 * c * d * d for c in sizes[:-1])
    flops *= H
    from chunked_linear_attention_packed_amd.profile_summary import (kernel_source_hash,
                                                                     profile_record)
    src_hash = kernel_source_hash()
    form_tag = {1: "one", 2: "two", 3: "three"}[n_launches] + ("_split" if a.split_fp32 else "")
    tr = profile_record("traffic", a.workload, form_tag, src_hash)
    traffic = tr["bytes_per_pass"] if tr else None
    sq = profile_record("counters", a.workload, form_tag, src_hash)
    pass_us = gpu_ms * 1e3 / a.steps
    pass_achieved = pass_bytes / (pass_us * 1e-6) / 1e9

    # spread of single passes: each of `steps` eager passes bracketed by its own
    # events on the stream (eager launches add host submission gaps, so these
    # sit above the graph figure; they show the distribution, not the rate)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    with torch.cuda.stream(stream):
        for i, (e_a, e_b) in enumerate(evs):
            e_a.record(stream)
            step(i)
            e_b.record(stream)
    torch.cuda.synchronize()
    singles = np.array([e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in evs])
    floor_us = launch_floor(max(a.steps, 20), quiet=True, n_launches=n_launches)

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(w, plan.seg_offsets, plan.branch_parent, a.cpu_seconds)

    rec = {
        "metric": "linear-attn layer tokens/s per packed pass on 1 GPU + % of roofline",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": a.workload,
            "tokens": T, "heads": H, "d": d, "segments": info.n_segments,
            "views": info.n_views, "branches": info.n_branches,
            "chunk": info.chunk, "block_chunks": info.block_chunks,
            "work_blocks": info.n_blocks, "delta_blocks": info.n_delta,
            "launches": n_launches,
            "launch": "eager" if a.eager else "hip_graph",
            "precision": ("fp32 data, products as 3 bf16 MFMAs (hi.hi + hi.lo + lo.hi)"
                          if a.split_fp32 else
                          ("fp32 MFMA" if w.dtype == "f32" else "bf16 MFMA, fp32 accumulate")),
            "rotating_input_sets": n_sets,
            "gpu_us_per_pass": pass_us,
            "pass_algorithmic_bytes": pass_bytes,
            "pass_roofline_frac": pass_bytes / (pass_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "pass_algorithmic_flops": flops,
            "pass_mfma_frac": flops / (pass_us * 1e-6) / (
                2.5e15 if (w.dtype == "bf16" or a.split_fp32) else 157.3e12),
            "mfma_busy_frac_counters": (sq or {}).get("mfma_busy_frac"),
            "single_pass_us_eager": {"p10": float(np.percentile(singles, 10)),
                                     "median": float(np.median(singles)),
                                     "p90": float(np.percentile(singles, 90))},
            "launch_floor_us": floor_us,
            "two_passes_in_flight": two_stream,
            "warm_same_inputs": warm_same,
        },
        "roofline": {
            "bound": "hbm", "achieved": pass_achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": pass_achieved / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": ("piece_kernel, single launch: the whole pass" if n_launches == 1
                       else f"the whole pass ({n_launches} launches)"),
            "bytes_per_pass": pass_bytes,
            "traffic_source": tr.get("source") if tr else None,
        },
        "cpu_baseline": cpu,
    }
    if n_launches > 1:
        rec["launch3_roofline"] = {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "us": l3_us, "bytes_per_launch": l3_bytes,
            "kernel": ("output launch (in the two-launch form it also sums the block states "
                       "before its block)" if n_launches == 2 else "output launch"),
        }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
