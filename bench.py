"""Benchmark: sparse paged decode attention on one MI355X.

Default workload (the 128K decode configuration of the LServe write-up's
latency table, bqwf.cn "3.2", at Llama-3-8B attention shape): 4 sequences of
131072 tokens, 32 query / 8 KV heads, head_dim 128, logical pages of 16 inside
physical pages of 64 shuffled over the pool, KV heads 0-3 streaming (sink 64 +
window 2048), 4-7 dynamic with a 4096-token budget, page selection every C = 4
decode steps. `--workload single_256k` (one 262144-token sequence, logical
pages of 32 in physical pages of 256, selection every step) and `--workload
ragged_mha` (16 sequences of 16K-128K tokens, 32 KV heads, budget
min(4096, L/32), C = 4) time the other two long-context configurations.
Inputs are synthetic (seeded N(0,1) bf16) and resident in HBM.

A step is one pass of the whole hot path for one attention layer: append the
new token, refresh its page summary, select pages (on steps t with t % C == 0),
sparse decode attention for all heads. The append runs inside the attention
launch on steps without selection (spa_append_decode_attn) and inside the
selection's scoring launch on the others (spa_append_select_pages). To keep
the timing honest about HBM (a step of the 128K configuration touches 51-118
MB, less than the 256 MB last-level cache), the layer is replicated R times
with separate pools and consecutive steps cycle through the replicas, as the
layers of a model do.

Timing: one whole reuse cycle (C decode steps of every replica, R x C
layer-steps, exactly one in C of them selecting) is captured in a HIP graph
and replayed N >= 20 times, each replay between two events on the stream it
runs on; `value` is the median over the replays of the time per layer-step
(p10 / p90 beside it). The same is done for a graph of R selecting steps and
a graph of R non-selecting steps (select_step_us, plain_step_us), and for a
graph of R attention calls, the dominant kernel, for the roofline. A read
probe with the attention's access shape (whole 4 KiB pieces at scattered
places, each read once) gives the same GPU's measured ceiling.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode-attn µs/step + achieved HBM GB/s (% peak) at 128K ctx"
PEAK_GBPS = 8000.0
COPY_BYTES = 1 << 30          # calibration copy for the HBM byte counters
ATTN_KERNELS = "attn_kernel<16, 5, 4, false, false, false>|combine_kernel"    # one spa_sparse_decode_attn call
WRITE_KERNELS = "write_kernel<16>"                               # one spa_kv_pool_write call
ATTN_KERNELS_FP8 = "attn_kernel<16, 5, 4, false, false, true>|combine_kernel"
WRITE_KERNELS_FP8 = "write_kernel_q8<16>"
ROW_BYTES = {"bf16": 256, "fp8": 128 + 4}     # one stored key or value row: elements (+ its fp32 scale)
MIN_REPLAYS = 20
WRITE_REPS = 10                       # warm prompt writes timed

# per workload: layer replicas (each step's working set times R must exceed
# the 256 MB last-level cache), decode steps generated, a description
WORKLOADS = {
    "llama3_128k": dict(replicas=8, steps=16,
                        text="batch 4 x 131072 ctx (+1 token/step), 32 q / 8 kv heads, d 128, logical page 16 / "
                             "physical 64 shuffled, kv 0-3 streaming (sink 64 + window 2048), kv 4-7 dynamic "
                             "budget 4096, select every 4 steps"),
    "single_256k": dict(replicas=12, steps=2,
                        text="batch 1 x 262144 ctx (+1 token/step), 32 q / 8 kv heads, d 128, logical page 32 / "
                             "physical 256, kv 0-3 streaming (sink 64 + window 4096), kv 4-7 dynamic budget "
                             "4096, select every step, 32 planted pages"),
    "ragged_mha": dict(replicas=2, steps=8,
                       text="batch 16 x U[16384, 131072] ctx (+1 token/step), 32 q / 32 kv heads (MHA), d 128, "
                            "logical page 16 / physical 64 shuffled, kv 0-15 streaming (sink 64 + window 1024), "
                            "kv 16-31 dynamic budget min(4096, L/32), select every 4 steps"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl, L, select: bool, row: int = 256, tail: int = 0) -> dict:
    """Bytes the method must move in one layer-step, per part. L: the length
    of every sequence (an int) or one length per sequence. A stored K or V row
    is `row` bytes (256 for bf16; 128 codes + a 4-byte scale for fp8 pages),
    summaries 512 B per page; `tail`: tokens appended since the selection,
    which dynamic heads attend besides their selected pages."""
    lens = [int(L)] * wl.batch if np.isscalar(L) else [int(x) for x in L]
    D2 = wl.d * 2
    n_dyn = sum(wl.kind)
    n_str = wl.hkv - n_dyn
    B = wl.batch
    attn = sel = 0
    for Lb in lens:
        s0 = min(wl.sink, Lb)
        w0 = max(wl.sink, Lb - wl.window)
        t_stream = s0 + max(0, Lb - w0)
        n = -(-Lb // wl.p)
        k = min(n, max(1, wl.budget_at(Lb) // wl.p))
        t_dyn = k * wl.p + tail                 # selected pages are full pages here
        attn += (n_str * t_stream + n_dyn * t_dyn) * 2 * row + n_dyn * k * 4 + (Lb // wl.P + 1) * 4
        if select:
            sel += n_dyn * n * 2 * D2 + n_dyn * n * 4 * 2 + n_dyn * k * 4
    q_bytes = B * wl.hq * D2
    out_bytes = B * wl.hq * (wl.d * 4 + 4)
    attn += q_bytes + out_bytes
    if select:
        sel += q_bytes
    append = B * wl.hkv * 2 * (D2 + row)                   # read new bf16 rows, write them
    summary = B * n_dyn * (D2 + 2 * 2 * D2)                 # new key + read/write min/max
    return dict(attn=attn, append=append, summary=summary, select=sel,
                total=attn + append + summary + sel)


def bulk_write_bytes(wl, count: int, row: int = 256, ring: bool = False) -> int:
    """Bytes one prompt write of `count` tokens from position 0 must move: read
    the caller's bf16 K and V rows, write them into the pool (`row` bytes each
    stored), write the min/max summary of every logical page of the dynamic
    heads, read the page-table row. With `ring`, a streaming head keeps only
    the tokens of its sink pages and of the last ceil(window / P) + 1 physical
    pages (the rest would be overwritten within the same write), and only those
    are read and written."""
    n_dyn = sum(wl.kind)
    n_str = wl.hkv - n_dyn
    kept = count
    if ring and count > 0:
        sink_pages = -(-wl.sink // wl.P)
        win_pages = -(-wl.window // wl.P) + 1
        last = (count - 1) // wl.P
        kept = min(sink_pages * wl.P, count) + max(0, count - max(sink_pages, last - win_pages + 1) * wl.P)
    rows = n_dyn * count + n_str * kept
    return 2 * rows * (wl.d * 2 + row) + n_dyn * (-(-count // wl.p)) * 2 * wl.d * 2 + (-(-count // wl.P)) * 4


def host_info() -> dict:
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"nproc": os.cpu_count(), "affinity": aff, "cpu_model": model}


def cpu_baseline(wl, host_kv, replicas: int, budget_s: float = 15.0) -> dict:
    """The CPU oracle on a bounded sample of the same job: decode steps in the
    GPU's order (selections and reuse as scheduled, the queries the GPU steps
    use) over every layer replica, sequence and KV head, until about
    `budget_s` seconds of CPU work are done; scaled to microseconds per
    layer-step."""
    import oracle
    import workloads as W
    oracle.build()
    G = wl.G
    states = {(r, b, h): oracle.HeadState(wl.k_max)
              for r in range(replicas) for b in range(wl.batch) for h in range(wl.hkv)}
    t0 = time.perf_counter()
    n = n_sel = 0
    for i in range(wl.steps):
        for r in range(replicas):
            jobs = []
            for b in range(wl.batch):
                L = wl.seq_len(b, i)
                q = W.query(wl, b, i * replicas + r)
                K, V = host_kv[b]
                for h in range(wl.hkv):
                    jobs.append(dict(K=K[h, :L], V=V[h, :L], q=q[h * G:(h + 1) * G], dynamic=bool(wl.kind[h]),
                                     sink=wl.sink, window=wl.window, p=wl.p, budget=wl.budget_at(L),
                                     do_select=wl.selects_at(i), state=states[(r, b, h)]))
            oracle.decode_heads(jobs)
            n += 1
            n_sel += wl.selects_at(i)
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    info = host_info()
    return {"value": round(dt / n * 1e6, 1), "unit": "us/step", "cores": oracle.num_threads(),
            "kind": "oracle", **info,
            "sample": f"{n} layer-steps ({n_sel} with selection) in the GPU's step order over {replicas} layer "
                      f"replicas, all {wl.batch} sequences x {wl.hkv} KV heads each, fp64 oracle on "
                      f"{oracle.num_threads()} OpenMP threads, {dt:.1f} s total"}


def percentiles(xs) -> dict:
    a = np.sort(np.asarray(xs, np.float64))
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "n": int(a.size)}


def timing_plan(steps: int, warmup: int, replicas: int, reuse: int) -> tuple:
    """Replays of the one-cycle graph (reuse decode steps of every replica, the
    first of them selecting) that cover at least `steps` layer-steps and at
    least MIN_REPLAYS, and untimed replays after the eager first cycle that
    cover `warmup`. Every timed replay is a whole cycle, so the timed mix of
    selecting and plain steps is 1 : reuse - 1 whatever the arguments."""
    cycle = replicas * reuse
    replays = max(MIN_REPLAYS, -(-steps // cycle))
    warm_replays = max(1, -(-max(warmup - cycle, 0) // cycle))
    return replays, warm_replays


def time_graph(torch, build, replays: int, per: int) -> list:
    """Captures build() in a HIP graph, replays it once untimed, then `replays`
    times, each between two events on the current stream; returns the time
    of each timed replay divided by `per`, in microseconds."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        build()
    g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    return [1e3 * e0.elapsed_time(e1) / per for e0, e1 in evs]


def read_ceiling(torch, spa, chunks: int, replicas: int, replays: int) -> dict:
    """The read probe: `replicas` disjoint random sets of `chunks` 4 KiB
    pieces of a 2 GiB buffer (one set per launch, cycling like the layer
    replicas), for 4, 8 and 16 pieces per wave; the best is the ceiling.
    A launch over consecutive pieces gives the sequential figure."""
    total = (2 << 30) // 4096
    buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(7)
    perm = rng.permutation(total)[:chunks * replicas].astype(np.int32)
    sets = [torch.from_numpy(perm[i * chunks:(i + 1) * chunks].copy()).cuda() for i in range(replicas)]
    seq = [torch.arange(i * chunks, (i + 1) * chunks, dtype=torch.int32, device="cuda") for i in range(replicas)]
    sink = torch.empty(chunks, dtype=torch.int32, device="cuda")
    res = {}
    for name, ids in (("random", sets), ("sequential", seq)):
        for cpw in (4, 8, 16):
            us = time_graph(torch, lambda: [spa.probe_read_chunks(buf, i, cpw, sink) for i in ids], replays,
                            replicas)
            med = float(np.median(us))
            res[f"{name}_{cpw}"] = round(chunks * 4096 / (med * 1e-6) / 1e9, 1)
    del buf
    best = max(v for k, v in res.items() if k.startswith("random"))
    return {"GBps": best, "per_wave": res, "bytes_per_launch": chunks * 4096}


def prefill_flops(pf, dense: bool) -> int:
    """Algorithmic flops of one prefill call: 4 D per attended (query, key)
    pair (the q.k product and the weighted sum of v), summed over the query
    heads; the dynamic heads attend causally inside min(j + 1, kb) key blocks
    of query block j (dense: all of them), the streaming heads their sink and
    window."""
    L, b, D = pf.L, pf.block, pf.d
    t = np.arange(L, dtype=np.int64)
    s0 = np.minimum(pf.sink, t + 1)
    w_lo = np.maximum(pf.sink, t + 1 - pf.window)
    stream_pairs = int((s0 + np.maximum(0, t + 1 - w_lo)).sum())
    nb = -(-L // b)
    kb = nb if dense else min(max(1, pf.budget // b), nb)
    dyn_pairs = 0
    for j in range(nb):
        rows = min(b, L - j * b)
        earlier = min(j + 1, kb) - 1                       # full earlier key blocks
        dyn_pairs += rows * earlier * b + rows * (rows + 1) // 2
    n_dyn = sum(pf.kind)
    return 4 * D * pf.G * (n_dyn * dyn_pairs + (pf.hkv - n_dyn) * stream_pairs)


def bench_prefill(args) -> int:
    """spa_prefill_attn on a whole prompt: the time per call (median of
    timed calls with HIP events), the same prompt in dense mode, algorithmic
    MFMA throughput, and the oracle on sampled rows as the CPU baseline."""
    import torch
    import workloads as W
    import sparse_paged_attention_amd as spa
    spa.lib()
    torch.cuda.set_device(0)
    pf = W.PREFILLS[args.workload]
    t_setup = time.time()
    Qb = np.stack([W.prefill_rows(pf, "q", i) for i in range(pf.hq)])
    Kb = np.stack([W.prefill_rows(pf, "k", h) for h in range(pf.hkv)])
    Vb = np.stack([W.prefill_rows(pf, "v", h) for h in range(pf.hkv)])
    Wq, Wk = W.prefill_projection(pf, "q"), W.prefill_projection(pf, "k")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    q, k, v, wq, wk = dev(Qb), dev(Kb), dev(Vb), dev(Wq), dev(Wk)
    heads = spa.Heads(pf.hq, pf.kind, pf.sink, pf.window)
    out = torch.empty((pf.hq, pf.L, pf.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((pf.hq, pf.L), dtype=torch.float32, device="cuda")
    log(f"[bench] prefill setup {time.time() - t_setup:.1f}s")
    reps = max(5, min(args.steps, 20))

    def timed(cfg) -> dict:
        ws = torch.empty(spa.prefill_workspace_bytes(heads, pf.hkv, cfg, pf.L), dtype=torch.uint8, device="cuda")
        for _ in range(2):
            spa.prefill_attn(heads, cfg, q, k, v, wq, wk, out, lse, workspace=ws)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record()
            spa.prefill_attn(heads, cfg, q, k, v, wq, wk, out, lse, workspace=ws)
            e1.record()
        torch.cuda.synchronize()
        return percentiles([e0.elapsed_time(e1) for e0, e1 in evs])

    dense_mode = pf.L < pf.dense_below
    cfg = spa.Prefill(budget=pf.budget, dense_below=pf.dense_below)
    t = timed(cfg)
    flops = prefill_flops(pf, dense_mode)
    tflops = flops / (t["median"] * 1e-3) / 1e12
    dense = None
    if not dense_mode:
        td = timed(spa.Prefill(budget=pf.budget, dense_below=pf.L + 1))
        dflops = prefill_flops(pf, True)
        dense = {"ms": td, "flops": dflops, "TFLOPs": round(dflops / (td["median"] * 1e-3) / 1e12, 1),
                 "speedup_of_sparse": round(td["median"] / t["median"], 2)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build()
        rng = np.random.default_rng(3)
        G = pf.G
        sel_s = 0.0
        modes = []
        for h in range(pf.hkv):                     # the selection of every dynamic head (whole)
            dyn = bool(pf.kind[h])
            ts = time.perf_counter()
            if dyn and not dense_mode:
                S = oracle.prefill_block_scores(Qb[h * G:(h + 1) * G], Kb[h], Wq, Wk, pf.block)
                sel, cnt = oracle.prefill_select(S, max(1, pf.budget // pf.block))
                sel_s += time.perf_counter() - ts
                modes.append((oracle.PREFILL_SPARSE, dict(sel=sel, cnt=cnt)))
            else:
                modes.append((oracle.PREFILL_DENSE, {}) if dyn else
                             (oracle.PREFILL_STREAMING, dict(sink=pf.sink, window=pf.window)))
        t0 = time.perf_counter()
        n_rows = 0
        while time.perf_counter() - t0 < 10.0:       # uniformly sampled rows of every query head
            rows = np.sort(rng.integers(0, pf.L, 64)).astype(np.int64)
            for h in range(pf.hkv):
                mode, kw = modes[h]
                for g in range(G):
                    oracle.prefill_attend(Qb[h * G + g], Kb[h], Vb[h], pf.block, mode, rows=rows, **kw)
                    n_rows += rows.size
        row_s = (time.perf_counter() - t0) / n_rows
        dt = time.perf_counter() - t0
        est = sel_s + row_s * pf.L * pf.hq
        cpu = {"value": round(est * 1e3, 1), "unit": "ms", "cores": oracle.num_threads(), "kind": "oracle",
               **host_info(),
               "sample": f"block scores and selection of all {sum(pf.kind)} dynamic KV heads ({sel_s:.1f} s) and "
                         f"{n_rows} sampled query rows over all {pf.hq} query heads ({dt - sel_s:.1f} s), fp64 "
                         f"oracle, scaled to all {pf.L * pf.hq} rows"}

    res = {
        "metric": f"prefill block-sparse attention ms at {pf.L // 1024}K ctx (one layer, LServe write-up 3.1)",
        "value": t["median"],
        "unit": "ms",
        "n_gpus": 1,
        "steps": reps,
        "warmup": 2,
        "ms_per_step": t["median"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (fp32 accumulate, fp64 block scores)",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: one sequence of {pf.L} tokens, {pf.hq} q / {pf.hkv} kv heads, "
                               f"d {pf.d}, blocks of {pf.block}, kv heads "
                               f"{[h for h in range(pf.hkv) if not pf.kind[h]]} streaming (sink {pf.sink} + window "
                               f"{pf.window}), the others dynamic with {pf.budget} key tokens per query block, "
                               f"dense below {pf.dense_below} tokens ({'dense' if dense_mode else 'sparse'} here), "
                               f"random low-rank sketch d -> d/8 as W_q = W_k"},
        "timing": {"call_ms": t},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None, "flops_per_call": int(flops),
                     "kernel": "spa_prefill_attn (pool_kernel + select_kernel + attn_kernel), algorithmic flops "
                               "(4 d per attended query-key pair)"},
        "dense_mode": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64,
                    help="layer-steps to time at least (rounded up to whole reuse cycles of every replica, "
                         "and to at least 20 replays of one cycle)")
    ap.add_argument("--warmup", type=int, default=16, help="untimed layer-steps before (at least one cycle)")
    ap.add_argument("--workload", choices=tuple(WORKLOADS) + ("prefill_128k", "prefill_16k"), default="llama3_128k",
                    help="decode workloads, or prefill_128k / prefill_16k: block-sparse prefill attention")
    ap.add_argument("--replicas", type=int, default=0, help="layer replicas the steps cycle over (0: per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling probe")
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--storage", choices=("table", "ring", "compact"), default="table",
                    help="streaming heads' tokens: in the page table's pages like the dynamic heads, in a "
                         "ring of sink + window pages per sequence (window-only storage), or in rings with "
                         "the compact pool (page-table pages hold the dynamic heads only)")
    ap.add_argument("--kv", choices=("bf16", "fp8"), default="bf16",
                    help="pool format: bf16 rows, or fp8 pages (E4M3 codes with one fp32 scale per row)")
    ap.add_argument("--probe", action="store_true",
                    help="counter-collection mode: run the steps eagerly, then a plain copy of "
                         "COPY_BYTES for calibration; prints no result line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no multi-GPU "
              f"path; the sharding by KV head it would use moves no data between GPUs.", file=sys.stderr)
        return 2

    if args.workload.startswith("prefill"):
        return bench_prefill(args)

    import torch
    import workloads as W
    import sparse_paged_attention_amd as spa
    from sparse_paged_attention_amd.runner import DecodeLayer
    from sparse_paged_attention_amd.profiling import source_hash

    spa.lib()
    torch.cuda.set_device(0)
    spec = WORKLOADS[args.workload]
    wl = W.WORKLOADS[args.workload].scaled(steps=spec["steps"])
    R = args.replicas or spec["replicas"]
    C = wl.reuse
    cycle = R * C                                # layer-steps in one reuse cycle of every replica
    if wl.steps < 2 * C:
        raise SystemExit("the workload needs two reuse cycles of decode steps")

    t_setup = time.time()
    pt = W.page_table(wl)
    layers = [DecodeLayer(hq=wl.hq, hkv=wl.hkv, p=wl.p, P=wl.P, kind=wl.kind, sink=wl.sink,
                          window=wl.window, page_table=pt, num_phys_pages=wl.num_phys_pages,
                          k_max=wl.k_max, window_only=args.storage != "table",
                          compact=args.storage == "compact", kv_format=args.kv) for _ in range(R)]
    row = ROW_BYTES[args.kv]
    host_kv = []
    write_events = []
    newk = np.zeros((wl.steps, wl.batch, wl.hkv, wl.d), np.uint16)
    newv = np.zeros_like(newk)
    for b in range(wl.batch):
        K = W.kv_all(wl, b, "k", args.threads)
        V = W.kv_all(wl, b, "v", args.threads)
        pre = wl.contexts[b] - 1
        Kd = torch.from_numpy(K[:, :pre].view(np.int16)).cuda().view(torch.bfloat16)
        Vd = torch.from_numpy(V[:, :pre].view(np.int16)).cuda().view(torch.bfloat16)
        torch.cuda.synchronize()
        for layer in layers:                    # prompt write + summaries of the dynamic heads, one pass
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            layer.write_tokens(b, 0, Kd, Vd)
            e1.record()
            write_events.append((e0, e1, pre))
        if b == 0:
            first_prompt = (Kd, Vd, pre)        # kept for the warm timing of the write below
        del Kd, Vd
        newk[:, b] = K[:, pre:pre + wl.steps].transpose(1, 0, 2)
        newv[:, b] = V[:, pre:pre + wl.steps].transpose(1, 0, 2)
        host_kv.append((K, V))
        log(f"[bench] sequence {b} written to {R} pools")
    for layer in layers:
        layer.set_lengths([c - 1 for c in wl.contexts])
        layer.set_budget([wl.budget_at(c) for c in wl.contexts])
    torch.cuda.synchronize()
    # the set-up writes are the first into freshly allocated pools; the prompt
    # write is timed warm, as the steps are: sequence 0's prompt written again
    # into layer 0 (the same bytes, so the pool does not change)
    cold_sel = [(e0, e1, n) for e0, e1, n in write_events if n == write_events[0][2]]
    cold_us = sorted(1e3 * e0.elapsed_time(e1) for e0, e1, _ in cold_sel)
    Kd, Vd, pre0 = first_prompt
    write_us = []
    for _ in range(WRITE_REPS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layers[0].write_tokens(0, 0, Kd, Vd)
        e1.record()
        write_us.append((e0, e1))
    torch.cuda.synchronize()
    write_us = sorted(1e3 * e0.elapsed_time(e1) for e0, e1 in write_us)
    del Kd, Vd, first_prompt
    write_med = write_us[len(write_us) // 2]
    write_bytes = bulk_write_bytes(wl, pre0, row, ring=args.storage != "table")

    def dev(a, dtype=torch.bfloat16):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(dtype)

    # per decode step: lengths, new tokens; per layer-step: q
    lens = [torch.tensor([wl.seq_len(b, t) for b in range(wl.batch)], dtype=torch.int32, device="cuda")
            for t in range(wl.steps)]
    kn = [dev(newk[t]) for t in range(wl.steps)]
    vn = [dev(newv[t]) for t in range(wl.steps)]
    qs = [dev(np.stack([W.query(wl, b, t * R + r) for b in range(wl.batch)]))
          for t in range(wl.steps) for r in range(R)]
    pool0 = layers[0].pool
    pool_bytes = sum(t.numel() * t.element_size() for t in (pool0.k, pool0.v, pool0.k_scale, pool0.v_scale)
                     if t is not None)
    log(f"[bench] setup {time.time() - t_setup:.1f}s; {R} replicas x {pool_bytes / 2**30:.2f} GiB K+V")

    def layer_step(t: int, r: int):
        layer = layers[r]
        s = t * R + r
        layer.use_lengths(lens[t])
        if wl.selects_at(t):                    # append inside the scoring launch
            layer.append_select(qs[s], kn[t], vn[t])
            layer.attend(qs[s])
        else:                                   # append inside the attention launch
            layer.append_attend(qs[s], kn[t], vn[t])

    # warm-up: the first reuse cycle of every replica, eagerly (decode steps
    # 0 .. C-1); the timed cycle is the next one (steps C .. 2C-1)
    for t in range(C):
        for r in range(R):
            layer_step(t, r)
    torch.cuda.synchronize()
    t0 = C

    if args.probe:
        for t in range(t0, t0 + C):
            for r in range(R):
                layer_step(t, r)
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] probe done: {cycle} steps, copy of {COPY_BYTES} bytes")
        return 0

    replays, warm_replays = timing_plan(args.steps, args.warmup, R, C)

    def run_cycle():
        for t in range(t0, t0 + C):
            for r in range(R):
                layer_step(t, r)

    # the cycle graph: warm replays untimed, then the timed replays. A replay
    # re-appends the same tokens at the same positions and does the same work
    # (a selection can differ where a scoring wave reads the summary of the
    # page receiving the token, which an earlier replay already filled
    # further; the attention reads k pages per dynamic head whichever they are)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_cycle()
    for _ in range(warm_replays):
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    wall0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_us = [1e3 * e0.elapsed_time(e1) / cycle for e0, e1 in evs]
    cyc = percentiles(step_us)
    del g

    # selecting steps alone and non-selecting steps alone (R layer-steps each)
    sel_us = percentiles(time_graph(torch, lambda: [layer_step(t0, r) for r in range(R)], replays, R))
    plain_us = None
    if C > 1:
        plain_us = percentiles(time_graph(torch, lambda: [layer_step(t0 + 1, r) for r in range(R)], replays, R))
    weighted = (sel_us["median"] + (C - 1) * plain_us["median"]) / C if plain_us else sel_us["median"]

    # the dominant kernel: spa_sparse_decode_attn (attn_kernel + combine_kernel)
    # over the replicas at the last decode step of the cycle, R calls a replay
    t_last = t0 + C - 1

    def attn_calls():
        for r in range(R):
            layers[r].use_lengths(lens[t_last])
            layers[r].attend(qs[t_last * R + r])
    attn = percentiles(time_graph(torch, attn_calls, replays, R))
    lens_last = [wl.seq_len(b, t_last) for b in range(wl.batch)]
    attn_bytes_call = algorithmic_bytes(wl, lens_last, False, row, tail=C - 1)["attn"]

    # algorithmic bytes per layer-step over the timed cycle
    tot = 0
    for t in range(t0, t0 + C):
        tot += R * algorithmic_bytes(wl, [wl.seq_len(b, t) for b in range(wl.batch)], wl.selects_at(t), row,
                                     tail=t % C)["total"]
    bytes_per_step = tot / cycle
    gbps = bytes_per_step / (cyc["median"] * 1e-6) / 1e9
    attn_gbps = attn_bytes_call / (attn["median"] * 1e-6) / 1e9

    ceiling = None
    if not args.no_ceiling:
        ceiling = read_ceiling(torch, spa, max(1, attn_bytes_call // 4096), R, replays)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, host_kv, R)

    def stored_traffic(name: str, kernels: str):
        """HBM bytes per launch from a committed counter summary, if it was
        taken on the kernels as they are now built."""
        tpath = os.path.join(ROOT, "profiles", name)
        if not os.path.exists(tpath):
            return None
        tr = json.load(open(tpath))
        return tr.get("bytes_per_launch") if tr.get("kernel_source_hash") == source_hash(kernels) else None

    fp8 = args.kv == "fp8"
    attn_kernels = ATTN_KERNELS_FP8 if fp8 else ATTN_KERNELS
    write_kernels = WRITE_KERNELS_FP8 if fp8 else WRITE_KERNELS
    tag = ("fp8_" if fp8 else "") + args.workload
    traffic = stored_traffic(f"attn_{tag}_traffic.json", attn_kernels)
    write_traffic = stored_traffic(f"bulk_write_{tag}_traffic.json", write_kernels)

    res = {
        "metric": METRIC,
        "value": round(cyc["median"], 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": replays * cycle,
        "warmup": cycle + warm_replays * cycle,
        "ms_per_step": round(cyc["median"] * 1e-3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 pages (bf16 q, fp32 accumulate)" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec['text']}, {R} layer replicas",
                   "batch": wl.batch, "context": list(wl.contexts) if wl.batch > 1 and len(set(wl.contexts)) > 1
                   else wl.contexts[0], "replicas": R, "reuse": C,
                   "streaming_storage": {"table": "page table", "ring": "ring of sink + window pages per sequence",
                                         "compact": "rings, page-table pages holding the dynamic heads only"}[
                       args.storage],
                   "kv_format": {"bf16": "bf16 rows", "fp8": "fp8 pages: E4M3 codes + one fp32 scale per row"}[
                       args.kv],
                   "pool_gib_per_layer": round(pool_bytes / 2**30, 3)},
        "timing": {"what": f"{replays} replays of a graph of one reuse cycle ({C} decode steps x {R} replicas = "
                           f"{cycle} layer-steps, one in {C} selecting); per replay: time / {cycle}",
                   "step_us": cyc, "select_step_us": sel_us, "plain_step_us": plain_us,
                   "c_weighted_us": round(weighted, 3), "steps_requested": args.steps,
                   "warmup_requested": args.warmup},
        "achieved_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_GBPS, 4),
        "bytes_per_step": int(bytes_per_step),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": f"spa_sparse_decode_attn ({attn_kernels.replace('|', ' + ')})",
                     "achieved": round(attn_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / PEAK_GBPS, 4), "traffic": traffic,
                     "avg_launch_us": attn["median"], "launch_us": attn, "bytes_per_launch": int(attn_bytes_call),
                     "measured_ceiling_GBps": ceiling["GBps"] if ceiling else None,
                     "frac_of_measured_ceiling": round(attn_gbps / ceiling["GBps"], 4) if ceiling else None},
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
        "bulk_write": {"what": f"spa_kv_pool_write of one {pre0}-token prompt (all {wl.hkv} KV heads"
                               + (", the streaming heads' sink and last window pages only"
                                  if args.storage != "table" else "")
                               + f", summaries of the {sum(wl.kind)} dynamic heads in the same pass)",
                       "median_us": round(write_med, 1), "bytes": int(write_bytes),
                       "achieved": round(write_bytes / (write_med * 1e-6) / 1e9, 1), "unit": "GB/s",
                       "frac": round(write_bytes / (write_med * 1e-6) / 1e9 / PEAK_GBPS, 4),
                       "traffic": write_traffic, "calls": len(write_us),
                       "first_writes_median_us": round(cold_us[len(cold_us) // 2], 1),
                       "timing": "median of warm rewrites of sequence 0's prompt into one layer (the same bytes); "
                                 "first_writes_median_us: the set-up's first writes into the fresh pools"},
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
