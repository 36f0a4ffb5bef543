"""Benchmark: sparse paged decode attention at 128K context on one MI355X.

Workload (the 128K decode configuration of the LServe write-up's latency
table, bqwf.cn "3.2", at Llama-3-8B attention shape): 4 sequences of 131072
tokens, 32 query / 8 KV heads, head_dim 128, logical pages of 16 inside
physical pages of 64 shuffled over the pool, KV heads 0-3 streaming (sink 64 +
window 2048), 4-7 dynamic with a 4096-token budget, page selection every 4
decode steps. Inputs are synthetic (seeded N(0,1) bf16) and resident in HBM.

A step is one pass of the whole hot path for one attention layer: append the
new token, refresh its page summary, select pages (every 4th decode step),
sparse decode attention for all heads. The append runs inside the attention
launch on steps without selection (spa_append_decode_attn) and inside the
selection's scoring launch on the others (spa_append_select_pages). To keep the timing honest about HBM
(a step touches 51-118 MB, less than the 256 MB last-level cache), the layer
is replicated R times with separate pools and consecutive steps cycle through
the replicas, as the layers of a model do; the timed steps are replayed from
a HIP graph.

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
WORKLOAD = "llama3_128k"
ATTN_KERNELS = "attn_kernel<16, 5, 4, false, false, false>|combine_kernel"    # one spa_sparse_decode_attn call
WRITE_KERNELS = "write_kernel<16>"                               # one spa_kv_pool_write call
ATTN_KERNELS_FP8 = "attn_kernel<16, 5, 4, false, false, true>|combine_kernel"
WRITE_KERNELS_FP8 = "write_kernel_q8<16>"
ROW_BYTES = {"bf16": 256, "fp8": 128 + 4}     # one stored key or value row: elements (+ its fp32 scale)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl, L: int, select: bool, row: int = 256) -> dict:
    """Bytes the method must move in one layer-step, per part (all sequences
    at length L). A stored K or V row is `row` bytes (256 for bf16; 128 codes +
    a 4-byte scale for fp8 pages), summaries 512 B per page."""
    D2 = wl.d * 2
    n_dyn = sum(wl.kind)
    n_str = wl.hkv - n_dyn
    B = wl.batch
    s0 = min(wl.sink, L)
    w0 = max(wl.sink, L - wl.window)
    t_stream = s0 + max(0, L - w0)
    n = -(-L // wl.p)
    k = min(n, max(1, wl.budget_at(L) // wl.p))
    t_dyn = k * wl.p                        # selected pages are full pages here
    q_bytes = B * wl.hq * D2
    out_bytes = B * wl.hq * (wl.d * 4 + 4)
    attn = B * (n_str * t_stream + n_dyn * t_dyn) * 2 * row + q_bytes + out_bytes \
        + B * n_dyn * k * 4 + B * (L // wl.P + 1) * 4
    append = B * wl.hkv * 2 * (D2 + row)                   # read new bf16 rows, write them
    summary = B * n_dyn * (D2 + 2 * 2 * D2)                 # new key + read/write min/max
    sel = 0
    if select:
        sel = B * n_dyn * n * 2 * D2 + q_bytes + B * n_dyn * n * 4 * 2 + B * n_dyn * k * 4
    return dict(attn=attn, append=append, summary=summary, select=sel,
                total=attn + append + summary + sel)


def bulk_write_bytes(wl, count: int, row: int = 256) -> int:
    """Bytes one prompt write of `count` tokens must move: read the caller's
    bf16 K and V rows, write them into the pool (`row` bytes each stored),
    write the min/max summary of every logical page of the dynamic heads, read
    the page-table row."""
    n_dyn = sum(wl.kind)
    rows = wl.hkv * count
    return 2 * rows * (wl.d * 2 + row) + n_dyn * (-(-count // wl.p)) * 2 * wl.d * 2 + (-(-count // wl.P)) * 4


def cpu_baseline(wl, host_kv, replicas: int, sample_steps: int = 16) -> dict:
    """The CPU oracle on a bounded sample of the same job: the first
    `sample_steps` decode steps (selections and reuse as scheduled) of every
    layer replica, sequence and KV head, with the queries the GPU steps use,
    scaled to microseconds per layer-step."""
    import oracle
    import workloads as W
    oracle.build()
    G = wl.G
    states = {(r, b, h): oracle.HeadState(wl.k_max)
              for r in range(replicas) for b in range(wl.batch) for h in range(wl.hkv)}
    t0 = time.perf_counter()
    for i in range(sample_steps):
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
    dt = time.perf_counter() - t0
    n = sample_steps * replicas
    n_sel = sum(1 for i in range(sample_steps) if wl.selects_at(i))
    return {"value": round(dt / n * 1e6, 1), "unit": "us/step", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{sample_steps} decode steps ({n_sel} with selection) x {replicas} layer replicas = "
                      f"{n} layer-steps over all {wl.batch} sequences x {wl.hkv} KV heads, fp64 oracle, "
                      f"{dt:.1f} s total"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed layer-steps")
    ap.add_argument("--warmup", type=int, default=16, help="untimed layer-steps before")
    ap.add_argument("--replicas", type=int, default=8, help="layer replicas the steps cycle over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path keeps every "
              f"head on its own GPU and has no multi-GPU run.", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    import sparse_paged_attention_amd as spa
    from sparse_paged_attention_amd.runner import DecodeLayer
    from sparse_paged_attention_amd.profiling import source_hash

    spa.lib()
    torch.cuda.set_device(0)
    wl = W.WORKLOADS[WORKLOAD]
    R = args.replicas
    total_steps = args.warmup + args.steps
    n_decode = -(-total_steps // R)
    if n_decode > wl.steps:
        raise SystemExit(f"at most {wl.steps * R} layer-steps with {R} replicas")

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
        del Kd, Vd
        newk[:, b] = K[:, pre:pre + wl.steps].transpose(1, 0, 2)
        newv[:, b] = V[:, pre:pre + wl.steps].transpose(1, 0, 2)
        host_kv.append((K, V))
        log(f"[bench] sequence {b} written to {R} pools")
    for layer in layers:
        layer.set_lengths([c - 1 for c in wl.contexts])
        layer.set_budget([wl.budget_at(c) for c in wl.contexts])
    torch.cuda.synchronize()
    write_us = sorted(1e3 * e0.elapsed_time(e1) for e0, e1, _ in write_events)
    write_med = write_us[len(write_us) // 2]
    write_bytes = bulk_write_bytes(wl, write_events[0][2], row)

    def dev(a, dtype=torch.bfloat16):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(dtype)

    # per decode step: lengths, new tokens; per layer-step: q
    lens = [torch.tensor([wl.seq_len(b, t) for b in range(wl.batch)], dtype=torch.int32, device="cuda")
            for t in range(n_decode)]
    kn = [dev(newk[t]) for t in range(n_decode)]
    vn = [dev(newv[t]) for t in range(n_decode)]
    qs = [dev(np.stack([W.query(wl, b, t * R + r) for b in range(wl.batch)]))
          for t in range(n_decode) for r in range(R)]
    pool0 = layers[0].pool
    pool_bytes = sum(t.numel() * t.element_size() for t in (pool0.k, pool0.v, pool0.k_scale, pool0.v_scale)
                     if t is not None)
    log(f"[bench] setup {time.time() - t_setup:.1f}s; {R} replicas x {pool_bytes / 2**30:.2f} GiB K+V")

    def layer_step(s: int):
        t, r = divmod(s, R)
        layer = layers[r]
        layer.use_lengths(lens[t])
        if wl.selects_at(t):                    # append inside the scoring launch
            layer.append_select(qs[s], kn[t], vn[t])
            layer.attend(qs[s])
        else:                                   # append inside the attention launch
            layer.append_attend(qs[s], kn[t], vn[t])

    # warm-up (eager, also compiles nothing: kernels are prebuilt)
    for s in range(args.warmup):
        layer_step(s)
    torch.cuda.synchronize()

    if args.probe:
        for s in range(args.warmup, total_steps):
            layer_step(s)
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] probe done: {args.steps} steps, copy of {COPY_BYTES} bytes")
        return 0

    # capture the timed steps once; a replay re-appends the same tokens at the
    # same positions and does the same work per step (a selection can differ
    # where a scoring wave reads the summary of the page receiving the token,
    # which an earlier run already filled further; the attention reads k
    # pages per dynamic head whichever they are)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(args.warmup, total_steps):
            layer_step(s)
    g.replay()                                  # one untimed replay
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps

    # per-call time of the attention entry point (attn_kernel + combine_kernel):
    # a graph of `steps` attention calls cycling over the replicas at the
    # state the timed steps left (last decode step's lengths and selections),
    # replayed between two events on the capturing stream
    t_last = (total_steps - 1) // R
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for i in range(args.steps):
            r = i % R
            layers[r].use_lengths(lens[t_last])
            layers[r].attend(qs[t_last * R + r])
    ga.replay()
    torch.cuda.synchronize()
    ea0, ea1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea0.record()
    ga.replay()
    ea1.record()
    torch.cuda.synchronize()
    attn_avg_us = 1e3 * ea0.elapsed_time(ea1) / args.steps
    attn_bytes_call = algorithmic_bytes(wl, wl.seq_len(0, t_last), False, row)["attn"]

    # algorithmic bytes over the timed steps
    tot = 0
    for s in range(args.warmup, total_steps):
        t = s // R
        tot += algorithmic_bytes(wl, wl.seq_len(0, t), wl.selects_at(t), row)["total"]
    bytes_per_step = tot / args.steps
    gbps = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    attn_gbps = attn_bytes_call / (attn_avg_us * 1e-6) / 1e9

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
    tag = "fp8_" if fp8 else ""
    traffic = stored_traffic(f"attn_{tag}llama3_128k_traffic.json", attn_kernels)
    write_traffic = stored_traffic(f"bulk_write_{tag}llama3_128k_traffic.json", write_kernels)

    res = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: batch 4 x 131072 ctx (+1 token/step), 32 q / 8 kv heads, "
                               f"d 128, logical page 16 / physical 64 shuffled, kv 0-3 streaming "
                               f"(sink 64 + window 2048), kv 4-7 dynamic budget 4096, select every 4 "
                               f"steps, {R} layer replicas",
                   "batch": wl.batch, "context": wl.contexts[0], "replicas": R,
                   "streaming_storage": {"table": "page table", "ring": "ring of sink + window pages per sequence",
                                         "compact": "rings, page-table pages holding the dynamic heads only"}[
                       args.storage],
                   "kv_format": {"bf16": "bf16 rows", "fp8": "fp8 pages: E4M3 codes + one fp32 scale per row"}[
                       args.kv],
                   "pool_gib_per_layer": round(pool_bytes / 2**30, 3)},
        "achieved_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_GBPS, 4),
        "bytes_per_step": int(bytes_per_step),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": f"spa_sparse_decode_attn ({attn_kernels.replace('|', ' + ')})",
                     "achieved": round(attn_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / PEAK_GBPS, 4), "traffic": traffic,
                     "avg_launch_us": round(attn_avg_us, 2), "bytes_per_launch": int(attn_bytes_call)},
        "cpu_baseline": cpu,
        "bulk_write": {"what": f"spa_kv_pool_write of one {write_events[0][2]}-token prompt (all {wl.hkv} KV heads, "
                               f"summaries of the {sum(wl.kind)} dynamic heads in the same pass)",
                       "median_us": round(write_med, 1), "bytes": int(write_bytes),
                       "achieved": round(write_bytes / (write_med * 1e-6) / 1e9, 1), "unit": "GB/s",
                       "frac": round(write_bytes / (write_med * 1e-6) / 1e9 / PEAK_GBPS, 4),
                       "traffic": write_traffic, "calls": len(write_us)},
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
