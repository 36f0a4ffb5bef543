"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs. Every test here needs an MI355X and the built library."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import ParityRun, assert_reports, bits_to_bf16, log, seed_range

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_paged_attention_amd as spa
    spa.lib()
    oracle.build()


def run(wl, steps=None, check=None, fused=False, window_only=False, compact=False):
    log(f"[parity] {wl.name} B={wl.batch} hq={wl.hq} hkv={wl.hkv} p={wl.p} P={wl.P} "
        f"contexts={wl.contexts[:4]} steps={wl.steps if steps is None else steps} window_only={window_only} "
        f"compact={compact}")
    pr = ParityRun(wl, check_heads=check, fused=fused, window_only=window_only, compact=compact)
    reps = pr.run(steps)
    assert_reports(reps)
    return pr, reps


# ------------------------------------------------------------ pool layout

def test_pool_write_append_and_summaries_bit_exact():
    wl = W.WORKLOADS["toy_4k"].scaled(contexts=(300, 77, 1), batch=3, steps=3, permute=True,
                                      kind=(1, 1), planted=None)
    pr = ParityRun(wl, check_heads=[])
    layer = pr.layer
    for i in range(wl.steps):
        q, kn, vn = pr.step_inputs(i)
        layer.set_lengths([wl.seq_len(b, i) for b in range(wl.batch)])
        layer.append(bits_to_bf16(kn), bits_to_bf16(vn))
    torch.cuda.synchronize()
    kp = layer.pool.k.view(torch.int16).cpu().numpy().view(np.uint16)
    vp = layer.pool.v.view(torch.int16).cpu().numpy().view(np.uint16)
    sp = layer.pool.summary.view(torch.int16).cpu().numpy().view(np.uint16)
    pt = W.page_table(wl)
    p, P, r = wl.p, wl.P, wl.P // wl.p
    for b in range(wl.batch):
        L = wl.final_len(b)
        for h in range(wl.hkv):
            K = W.kv(wl, b, h, "k")[:L]
            V = W.kv(wl, b, h, "v")[:L]
            t = np.arange(L)
            phys = pt[b, t // P]
            slot = t % P
            np.testing.assert_array_equal(kp[phys, h, slot], K)
            np.testing.assert_array_equal(vp[phys, h, slot // p, :, slot % p], V)
            kmin, kmax = oracle.page_summary(K, p)
            j = np.arange(kmin.shape[0])
            np.testing.assert_array_equal(sp[pt[b, j // r], h, j % r, 0], kmin)
            np.testing.assert_array_equal(sp[pt[b, j // r], h, j % r, 1], kmax)


@pytest.mark.parametrize("p,P", [(16, 64), (32, 256), (64, 128)])
def test_bulk_write_in_chunks_builds_summaries(p, P):
    """spa_kv_pool_write with the head kinds, in chunks whose edges fall inside
    logical pages: the pool holds every token where the page table puts it,
    each dynamic head's summaries equal the oracle's min/max pooling of its
    keys (LServe write-up "2.1"), bit for bit, streaming heads' summaries are
    not touched, and rebuilding the summaries from the pool changes nothing."""
    from sparse_paged_attention_amd.runner import DecodeLayer
    wl = W.WORKLOADS["toy_4k"].scaled(contexts=(300, 77, 1, 2 * P + 3), batch=4, steps=1, permute=True,
                                      p=p, P=P, hkv=4, hq=8, kind=(1, 0, 1, 0), planted=None, name="bulk_write")
    log(f"[parity] bulk write p={p} P={P} contexts={wl.contexts}")
    pt = W.page_table(wl)
    layer = DecodeLayer(hq=wl.hq, hkv=wl.hkv, p=p, P=P, kind=wl.kind, sink=wl.sink, window=wl.window,
                        page_table=pt, num_phys_pages=wl.num_phys_pages, k_max=wl.k_max)
    layer.pool.summary.view(torch.int16).fill_(0x7F7F)           # a pattern no write produces here
    src = []
    for b in range(wl.batch):
        L = wl.contexts[b]
        K = np.stack([W.kv(wl, b, h, "k")[:L] for h in range(wl.hkv)])
        V = np.stack([W.kv(wl, b, h, "v")[:L] for h in range(wl.hkv)])
        src.append((K, V))
        edges = sorted({0, L, *[e for e in (37, 38, 38 + p, 2 * P + 1) if e < L]})
        for a, e in zip(edges[:-1], edges[1:]):
            layer.write_tokens(b, a, bits_to_bf16(np.ascontiguousarray(K[:, a:e])).cuda(),
                               bits_to_bf16(np.ascontiguousarray(V[:, a:e])).cuda())
    layer.set_lengths(list(wl.contexts))
    torch.cuda.synchronize()

    def host(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    kp, vp, sp = host(layer.pool.k), host(layer.pool.v), host(layer.pool.summary)
    r = P // p
    for b in range(wl.batch):
        K, V = src[b]
        L = wl.contexts[b]
        t = np.arange(L)
        phys, slot = pt[b, t // P], t % P
        j = np.arange(-(-L // p))
        for h in range(wl.hkv):
            np.testing.assert_array_equal(kp[phys, h, slot], K[h])
            np.testing.assert_array_equal(vp[phys, h, slot // p, :, slot % p], V[h])
            got = sp[pt[b, j // r], h, j % r]
            if wl.kind[h]:
                kmin, kmax = oracle.page_summary(K[h], p)
                np.testing.assert_array_equal(got[:, 0], kmin)
                np.testing.assert_array_equal(got[:, 1], kmax)
            else:
                assert (got == 0x7F7F).all()
    layer.rebuild_summaries()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(layer.pool.summary), sp)


# ------------------------------------------------------ the five workloads

def test_toy_4k():
    run(W.WORKLOADS["toy_4k"])


def test_llama3_32k_massive_activations():
    run(W.WORKLOADS["llama3_32k"])


def test_single_256k_p32():
    run(W.WORKLOADS["single_256k"])


def test_llama3_128k_reuse_small():
    """The 128K workload's shape and step schedule at small contexts: batch 4,
    shuffled pool, selection every 4 steps, 9 steps (tail of up to 3 tokens)."""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=9, budget=512,
                                           window=300)
    run(wl)


def test_ragged_mha_small():
    wl = W.WORKLOADS["ragged_mha"].scaled(contexts=(2500, 40, 1800, 3333, 700, 16, 1, 2049),
                                          batch=8, steps=6)
    run(wl)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (64, 8), (32, 2), (24, 8), (40, 8), (12, 2), (56, 8),
                                    (24, 2)])
def test_group_sizes(hq, hkv, fused):
    """Query groups of 1, 2, 8 and 16 heads (the benchmark's 4 elsewhere) and of
    3, 5, 6, 7 and 12 (scored by the kernel built for the next power of two,
    the extra query columns repeating the group's last query), on the separate
    entry points and on the launches with the append inside (for groups above
    4 the selection entry point runs the append first)."""
    kind = tuple(h % 2 for h in range(hkv))
    wl = W.Workload(f"g{hq // hkv}", 2000 + hq, 2, hq, hkv, 16, 64, (1500, 999), 5, 2, kind, 32, 200,
                    256, True)
    run(wl, fused=fused)


def test_p64_and_dense_budget():
    """p = 64 pages; the budget covers the context, so the dynamic head is dense."""
    wl = W.Workload("p64", 2100, 2, 8, 2, 64, 256, (700, 300), 3, 1, (0, 1), 8, 5000, 8192, True)
    run(wl)


def test_short_sequences_streaming_dense():
    """L <= sink + window: streaming heads attend everything."""
    wl = W.Workload("short", 2200, 3, 32, 8, 16, 64, (1, 30, 65), 4, 2, (0, 1) * 4, 64, 1024, 4096,
                    False)
    run(wl)


@pytest.mark.parametrize("fused", [True, False])
def test_llama3_128k_full_size(fused):
    """The configuration the benchmark times, at full size: 4 x 131072 + 16
    steps, shuffled pool, reuse every 4 steps. With `fused` the steps run the
    benchmark's launches (the append inside the selection / attention
    launches), checked on every (sequence, KV head); without it the separate
    entry points (the attention call the roofline is timed on), checked on
    sampled heads."""
    wl = W.WORKLOADS["llama3_128k"]
    run(wl, check=None if fused else [(0, 0), (0, 4), (1, 5), (2, 3), (3, 7)], fused=fused)


def test_ragged_mha_full_size():
    """The ragged continuous batch at full size: 16 sequences of 24842 ..
    127144 tokens, 32 KV heads (MHA) over one shuffled 20.5 GB pool, 16 steps
    with selection every 4, the benchmark's launches; checked on every head of
    the shortest and the longest sequences and of two others (128 of the 512
    (sequence, head) pairs, streaming 0-15 and dynamic 16-31)."""
    wl = W.WORKLOADS["ragged_mha"]
    short, long_ = int(np.argmin(wl.contexts)), int(np.argmax(wl.contexts))
    seqs = sorted({short, long_, 9, 13})
    run(wl, check=[(b, h) for b in seqs for h in range(wl.hkv)], fused=True)


# Top-k holds E scores per thread of a 1024-thread group, E the fewest of 8,
# 9, 12, 16, 24 and 32 that hold a row of n_max = max_pages * P / p scores.
# One context per band of E above 9 (p = 16, P = 64), planted pages, and an
# integer-valued case whose rows are full of exact score ties.
TOPK_BANDS = {
    "E12": (150_000, 9216, 12288, False),
    "E16": (200_000, 12288, 16384, False),
    "E24": (300_000, 16384, 24576, False),
    "E32": (500_000, 24576, 32768, False),
    "E32_ties": (520_000, 24576, 32768, True),
}


@pytest.mark.parametrize("band", list(TOPK_BANDS))
def test_topk_row_sizes(band):
    """Selections over rows of 9376 .. 32500 logical pages (contexts of 150K
    to 520K tokens): every top-k row size above the benchmark's, checked id for
    id against the oracle (strict: the scores are bit-identical), with the
    outputs; two selecting steps each."""
    L, lo, hi, quantized = TOPK_BANDS[band]
    wl = W.Workload(f"topk_{band}", 2950 + L // 1000, 1, 8, 2, 16, 64, (L,), 2, 1, (0, 1), 64, 512, 4096,
                    True, planted=None if quantized else "aligned3", quantized=quantized)
    n_max = wl.max_pages * (wl.P // wl.p)
    assert lo < n_max <= hi, (band, n_max)
    log(f"[parity] top-k band {band}: n_max {n_max}")
    reps = ParityRun(wl, strict_ties=True).run()
    assert_reports(reps)
    assert all(r["sel_checked"] == 1 for r in reps)


def test_sparse_config_of_the_write_up():
    """The LServe write-up's example sparse configuration ("5.2 参数调优指南",
    tests/golden/sparse_config.json): logical pages of 32 tokens inside
    physical pages of 512, half the KV heads streaming, a 4096-token budget,
    selection reused for 4 steps; the benchmark's launches against the
    oracle."""
    import json
    import os
    cfg = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sparse_config.json")))
    hkv = 8
    n_stream = int(cfg["static_sparsity_ratio"] * hkv)
    kind = (0,) * n_stream + (1,) * (hkv - n_stream)
    wl = W.Workload("write_up_config", 3100, 3, 32, hkv, cfg["logical_page_size"], cfg["physical_page_size"],
                    (140_000, 9000, 33_000), 9, cfg["reuse_interval"], kind, 64, 2048,
                    cfg["dynamic_token_budget"], True)
    run(wl, fused=True)


def test_outputs_stay_inside_their_buffers():
    """Canary words around every buffer the library writes (out, lse,
    workspace, selection outputs, scores): a few decode steps of the 128K
    shape at small contexts, on both the separate and the append entry points,
    leave every guard word as it was, and the results still match the
    oracle."""
    GUARD = 1024

    def guarded(t, fill):
        n = t.numel()
        buf = torch.empty(n + 2 * GUARD, dtype=t.dtype, device=t.device)
        if t.dtype == torch.float32:
            buf.view(torch.int32).fill_(fill)
        else:
            buf.fill_(fill)
        return buf, buf[GUARD:GUARD + n].view(t.shape)

    for fused in (False, True):
        wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=6, budget=512, window=300)
        pr = ParityRun(wl, fused=fused)
        layer = pr.layer
        bufs = {}
        for name, fill in (("out", 0x7FC0DEAD), ("lse", 0x7FC0BEEF), ("workspace", 0xA5),
                           ("sel_pages", 0x5A5A5A5A), ("sel_count", 0x5A5A5A5B), ("sel_len", 0x5A5A5A5C),
                           ("sel_phys", 0x5A5A5A5D)):
            t = getattr(layer, name)
            full, view = guarded(t, fill if t.dtype != torch.uint8 else fill)
            view.copy_(t)
            setattr(layer, name, view)
            bufs[name] = (full, full.clone())
        full, view = guarded(pr.scores, 0x7FC0F00D)
        view.copy_(pr.scores)
        pr.scores = view
        bufs["scores"] = (full, full.clone())
        assert_reports(pr.run())
        torch.cuda.synchronize()
        for name, (full, before) in bufs.items():
            for part in (slice(0, GUARD), slice(full.numel() - GUARD, full.numel())):
                a, b = full[part], before[part]
                if a.dtype == torch.float32:
                    a, b = a.view(torch.int32), b.view(torch.int32)
                assert torch.equal(a, b), f"fused={fused}: a guard word of {name} was overwritten"


def test_graph_replay_matches_eager():
    """The benchmark's path: decode steps (the append inside the selection /
    attention launches, selection every 4 steps) captured in a HIP graph and
    replayed. From the same pool state, every replay gives the eager run's
    outputs, lse and selections bit for bit; eager work and synchronisations
    run between the replays. (The pool is restored before each run: a replay
    re-appends the same tokens, but the summary of the page receiving a token
    may be read before its rewrite, and after an earlier run it already holds
    later tokens.)"""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=8, budget=512, window=300)
    log(f"[parity] graph replay {wl.name} contexts={wl.contexts} steps={wl.steps}")
    pr = ParityRun(wl, check_heads=[])
    layer = pr.layer
    layer.set_budget([wl.budget_at(wl.seq_len(b, 0)) for b in range(wl.batch)])
    pool = [layer.pool.k, layer.pool.v, layer.pool.summary]
    snap = [t.clone() for t in pool]
    steps = []
    for i in range(wl.steps):
        q, kn, vn = pr.step_inputs(i)
        lens = torch.tensor([wl.seq_len(b, i) for b in range(wl.batch)], dtype=torch.int32, device="cuda")
        steps.append((lens, bits_to_bf16(q), bits_to_bf16(kn), bits_to_bf16(vn), wl.selects_at(i)))

    def buffers():
        return [(torch.empty_like(layer.out), torch.empty_like(layer.lse), torch.empty_like(layer.sel_pages),
                 torch.empty_like(layer.sel_count)) for _ in steps]

    def run_steps(rec):
        for (lens, q, kn, vn, sel), (o, l, sp, sc) in zip(steps, rec):
            layer.use_lengths(lens)
            if sel:
                layer.append_select(q, kn, vn)
                layer.attend(q)
            else:
                layer.append_attend(q, kn, vn)
            o.copy_(layer.out)
            l.copy_(layer.lse)
            sp.copy_(layer.sel_pages)
            sc.copy_(layer.sel_count)

    def restore():
        for t, s0 in zip(pool, snap):
            t.copy_(s0)
        torch.cuda.synchronize()

    eager = buffers()
    restore()
    run_steps(eager)
    torch.cuda.synchronize()
    replayed = buffers()
    g = torch.cuda.CUDAGraph()
    restore()
    with torch.cuda.graph(g):
        run_steps(replayed)
    for rep in range(3):
        restore()
        noise = torch.randn(1 << 20, device="cuda").sum()        # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        for i, (a, b) in enumerate(zip(eager, replayed)):
            for x, y, what in zip(a, b, ("out", "lse", "sel_pages", "sel_count")):
                assert torch.equal(x, y), f"replay {rep} step {i}: {what} differs from the eager run"
    # and the eager run itself is the oracle's (same steps, same state)
    pr2 = ParityRun(wl, fused=True)
    assert_reports(pr2.run())


def test_pages_mapped_from_the_free_list_as_sequences_grow():
    """The serving flow: each sequence's prompt pages come from the host free
    list (spa_alloc_*), and a new physical page is taken and entered into the
    device page table exactly when a step's token opens it (every sequence
    crosses a page boundary during the steps; the entries of earlier pages,
    which selections refer to, never change). Checked against the oracle every
    step; all pages go back to the free list at the end."""
    import sparse_paged_attention_amd as spa
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(1020, 126, 2047, 64), steps=12, budget=512, window=300,
                                           permute=False)
    P = wl.P
    alloc = spa.Allocator(wl.num_phys_pages)
    pt = np.full((wl.batch, wl.max_pages), -1, np.int32)
    for b in range(wl.batch):
        n = -(-(wl.contexts[b] - 1) // P)
        pt[b, :n] = alloc.alloc(n)
    log(f"[parity] pages from the free list {wl.name} contexts={wl.contexts}")
    pr = ParityRun(wl, fused=True, page_table=pt)
    opened = 0
    for i in range(wl.steps):
        for b in range(wl.batch):
            t = wl.seq_len(b, i) - 1
            if t % P == 0:                       # the token opens a physical page
                assert pt[b, t // P] == -1
                pt[b, t // P] = alloc.alloc(1)[0]
                pr.layer.page_table[b, t // P] = int(pt[b, t // P])
                opened += 1
        assert_reports([pr.run_step(i)])
    assert opened == wl.batch
    alloc.free([int(x) for x in pt[pt >= 0]])
    assert alloc.num_free == wl.num_phys_pages


# ------------------------------------------ window-only streaming storage

WINDOW_ONLY_CASES = {
    "toy_4k": lambda: W.WORKLOADS["toy_4k"].scaled(steps=6, reuse=2),
    "128k_small": lambda: W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=9,
                                                           budget=512, window=300),
    "ragged_small": lambda: W.WORKLOADS["ragged_mha"].scaled(contexts=(2500, 40, 1800, 3333, 700, 16, 1, 2049),
                                                             batch=8, steps=6),
    "p32_P256": lambda: W.WORKLOADS["single_256k"].scaled(contexts=(9000,), steps=5, window=700, sink=40),
    "p64": lambda: W.Workload("p64_ring", 2480, 2, 8, 2, 64, 256, (2000, 700), 6, 2, (0, 1), 8, 600, 512, True),
}


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", list(WINDOW_ONLY_CASES))
def test_window_only_storage(case, fused):
    """Streaming heads kept in a ring of sink + window pages per sequence
    (the window's pages reused as it moves; LServe write-up "2.1": streaming
    heads attend the sink and the window only): the same results as the
    oracle, on the separate entry points and on the benchmark's launches."""
    run(WINDOW_ONLY_CASES[case](), fused=fused, window_only=True)


def test_window_only_matches_page_table_layout():
    """The ring changes where streaming heads' rows live, nothing else: step
    by step, outputs, lse and selections are bit-identical to the page-table
    layout, and no streaming head's row is ever written into a page of the
    page table (those pages stay zero there)."""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=9, budget=512, window=300)
    log(f"[parity] ring vs page table {wl.name} contexts={wl.contexts}")
    a = ParityRun(wl, check_heads=[], fused=True)
    b = ParityRun(wl, check_heads=[], fused=True, window_only=True)
    for i in range(wl.steps):
        a.run_step(i)
        b.run_step(i)
        for x, y, what in ((a.layer.out, b.layer.out, "out"), (a.layer.lse, b.layer.lse, "lse"),
                           (a.layer.sel_pages, b.layer.sel_pages, "sel_pages"),
                           (a.layer.sel_count, b.layer.sel_count, "sel_count")):
            assert torch.equal(x, y), f"step {i}: {what} differs"
    pt = W.page_table(wl)
    used = np.unique(pt[pt >= 0])
    stream = [h for h in range(wl.hkv) if not wl.kind[h]]
    k = b.layer.pool.k[torch.from_numpy(used).cuda()][:, stream]
    v = b.layer.pool.v[torch.from_numpy(used).cuda()][:, stream]
    assert not k.view(torch.int16).any() and not v.view(torch.int16).any()


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", list(WINDOW_ONLY_CASES))
def test_compact_pool(case, fused):
    """The compact layout of window-only storage: the page table's pages hold
    only the dynamic heads and the rings only the streaming heads (each in its
    rank among the heads of its kind); the same results as the oracle."""
    run(WINDOW_ONLY_CASES[case](), fused=fused, compact=True)


def test_compact_pool_matches_page_table_layout():
    """The compact pool gives, step by step, the page-table layout's outputs,
    lse and selections bit for bit, with half the head slots per page."""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=9, budget=512, window=300)
    log(f"[parity] compact vs page table {wl.name} contexts={wl.contexts}")
    a = ParityRun(wl, check_heads=[], fused=True)
    b = ParityRun(wl, check_heads=[], fused=True, compact=True)
    assert b.layer.pool.k.shape[1] * 2 == a.layer.pool.k.shape[1]
    for i in range(wl.steps):
        a.run_step(i)
        b.run_step(i)
        for x, y, what in ((a.layer.out, b.layer.out, "out"), (a.layer.lse, b.layer.lse, "lse"),
                           (a.layer.sel_pages, b.layer.sel_pages, "sel_pages"),
                           (a.layer.sel_count, b.layer.sel_count, "sel_count")):
            assert torch.equal(x, y), f"step {i}: {what} differs"


def test_compact_pool_128k_full_size_sampled():
    """The benchmark's configuration at full size in the compact layout (half
    the pool), the benchmark's launches, sampled heads."""
    run(W.WORKLOADS["llama3_128k"], check=[(0, 1), (1, 6), (2, 4), (3, 3)], fused=True, compact=True)


def test_window_only_128k_full_size_sampled():
    """The benchmark's configuration at full size with the streaming heads in
    rings (4 x 131072 + 16 steps, the benchmark's launches), sampled heads."""
    run(W.WORKLOADS["llama3_128k"], check=[(0, 0), (1, 3), (2, 5), (3, 2)], fused=True, window_only=True)


@pytest.mark.parametrize("bpi", [4, 5, 6, 7, 8, 9, 10, 12, 16])
def test_every_item_size(bpi):
    """Each attention work-item size (odd sizes pad the last block pair):
    the 128K shape at small contexts with a 3-token tail, and p = 64 pages."""
    import sparse_paged_attention_amd as spa
    spa.set_attn_blocks_per_item(bpi)
    try:
        run(W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=5, budget=512,
                                              window=300))
        run(W.Workload(f"p64_bpi{bpi}", 2400 + bpi, 2, 8, 2, 64, 256, (2000, 700), 3, 2, (0, 1), 8, 600,
                       512, True))
    finally:
        spa.set_attn_blocks_per_item(0)


def test_append_inside_attention_pool_bit_exact():
    """spa_append_decode_attn and spa_append_select_pages write the same pool
    (keys, values, summaries) as spa_kv_pool_append: four steps alternating
    the two, new pages opened on the way."""
    wl = W.WORKLOADS["toy_4k"].scaled(contexts=(300, 77, 1, 33), batch=4, steps=4, permute=True,
                                      kind=(1, 0), planted=None)
    pr = ParityRun(wl, check_heads=[])
    layer = pr.layer
    layer.set_budget([256] * wl.batch)
    for i in range(wl.steps):
        q, kn, vn = pr.step_inputs(i)
        layer.set_lengths([wl.seq_len(b, i) for b in range(wl.batch)])
        if i % 2 == 0:
            layer.append_select(bits_to_bf16(q), bits_to_bf16(kn), bits_to_bf16(vn))
        else:
            layer.append_attend(bits_to_bf16(q), bits_to_bf16(kn), bits_to_bf16(vn))
    torch.cuda.synchronize()
    kp = layer.pool.k.view(torch.int16).cpu().numpy().view(np.uint16)
    vp = layer.pool.v.view(torch.int16).cpu().numpy().view(np.uint16)
    sp = layer.pool.summary.view(torch.int16).cpu().numpy().view(np.uint16)
    pt = W.page_table(wl)
    p, P, r = wl.p, wl.P, wl.P // wl.p
    for b in range(wl.batch):
        L = wl.final_len(b)
        for h in range(wl.hkv):
            K = W.kv(wl, b, h, "k")[:L]
            V = W.kv(wl, b, h, "v")[:L]
            t = np.arange(L)
            phys = pt[b, t // P]
            slot = t % P
            np.testing.assert_array_equal(kp[phys, h, slot], K)
            np.testing.assert_array_equal(vp[phys, h, slot // p, :, slot % p], V)
            if wl.kind[h]:
                kmin, kmax = oracle.page_summary(K, p)
                j = np.arange(kmin.shape[0])
                np.testing.assert_array_equal(sp[pt[b, j // r], h, j % r, 0], kmin)
                np.testing.assert_array_equal(sp[pt[b, j // r], h, j % r, 1], kmax)


def test_append_inside_attention_128k_small():
    """The 128K shape at small contexts, steps without selection appending in
    the attention launch (selection every 4 steps, tails of up to 3 tokens)."""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=9, budget=512,
                                           window=300)
    run(wl, fused=True)


def test_append_inside_attention_edges():
    """Appending in the attention launch: a second token (the dynamic heads'
    tail is the new token alone), tokens inside the sink, tokens opening a
    new block and a new page, ragged MHA heads, p = 64 pages."""
    wl = W.Workload("fused_edges", 2700, 6, 16, 4, 16, 64, (1, 2, 16, 33, 64, 1090), 4, 3, (0, 1, 1, 0),
                    32, 64, 256, True)
    run(wl, fused=True)
    run(W.WORKLOADS["ragged_mha"].scaled(contexts=(2500, 40, 1800, 3333, 700, 16, 1, 2049), batch=8,
                                         steps=5), fused=True)
    run(W.Workload("fused_p64", 2800, 2, 8, 2, 64, 256, (2000, 700), 5, 2, (0, 1), 8, 600, 512, True),
        fused=True)


@pytest.mark.parametrize("bpi", [4, 5, 7, 16])
def test_append_inside_attention_item_sizes(bpi):
    """Every head's last item carries the appended token, whatever the item size."""
    import sparse_paged_attention_amd as spa
    spa.set_attn_blocks_per_item(bpi)
    try:
        run(W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=5, budget=512,
                                              window=300), fused=True)
    finally:
        spa.set_attn_blocks_per_item(0)


def test_score_ranges_of_every_fill():
    """Scoring works on ranges of 128 pages in passes of 16, a head's last
    range taking one pass more: contexts whose last range holds 1, 17, 33,
    113, 128 and 132 pages (1 to 9 live passes) and one that ends inside a
    page."""
    n_pages = (129, 145, 161, 241, 256, 260, 227)
    ctx = tuple(16 * n for n in n_pages[:-1]) + (16 * n_pages[-1] - 5,)
    wl = W.Workload("score_fill", 2600, len(ctx), 16, 4, 16, 64, ctx, 2, 1, (1, 0, 1, 1), 16, 100, 512,
                    True)
    run(wl)


def test_attention_resolving_pages_through_the_page_table():
    """spa_sparse_decode_attn without the selection's physical pages (looks the
    selected pages up in the page table itself): same results."""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=6, budget=512, window=300)
    log(f"[parity] {wl.name} through the page table")
    assert_reports(ParityRun(wl, resolve_at_selection=False).run())


def test_selection_exact_ties_go_to_lowest_page_id():
    """Integer-valued keys and queries: many pages share a score exactly, and
    the selection must still match the oracle id for id (lowest ids win)."""
    wl = W.Workload("ties", 2300, 3, 32, 8, 16, 64, (3000, 777, 5000), 3, 1, (0, 1) * 4, 16, 128, 512,
                    True, quantized=True)
    log(f"[parity] {wl.name}")
    pr = ParityRun(wl, strict_ties=True)
    assert_reports(pr.run())


def random_workload(seed: int, groups=(1, 8)):
    """A seeded random small configuration: KV heads, group size (in the range
    `groups`), page sizes, batch and lengths, head kinds, sink and window,
    budget, reuse interval, page layout, pool format, storage and launch
    path."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.integers(groups[0], groups[1] + 1))
    p = int(rng.choice([16, 32, 64]))
    P = p * int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 5))
    contexts = tuple(int(x) for x in rng.integers(1, 3000, batch))
    kind = tuple(int(x) for x in rng.integers(0, 2, hkv))
    sink = int(rng.integers(0, 100))
    window = int(rng.integers(1, 600))
    budget = int(rng.integers(p, 1025))
    wl = W.Workload(f"random{seed}", 7000 + seed, batch, hkv * G, hkv, p, P, contexts, int(rng.integers(3, 7)),
                    int(rng.integers(1, 5)), kind, sink, window, budget, bool(rng.integers(0, 2)),
                    quantized=bool(rng.random() < 0.2))
    storage = str(rng.choice(["table", "ring", "compact"]))
    return wl, dict(kv_format=str(rng.choice(["bf16", "fp8"])), fused=bool(rng.integers(0, 2)),
                    window_only=storage != "table", compact=storage == "compact")


@pytest.mark.parametrize("seed", seed_range("SPA_RANDOM_SEEDS", 48))
def test_random_configurations(seed):
    """Forty-eight seeded random small configurations (random_workload) through
    the whole step against the oracle: every step's outputs, scores and
    selections, on whichever pool format, storage and launch path the seed
    draws. SPA_RANDOM_SEEDS=a:b runs seeds a .. b - 1 instead (a wider
    sweep)."""
    wl, opts = random_workload(seed)
    log(f"[parity] random {seed}: B={wl.batch} hq={wl.hq} hkv={wl.hkv} p={wl.p} P={wl.P} kind={wl.kind} "
        f"contexts={wl.contexts} sink={wl.sink} window={wl.window} budget={wl.budget} reuse={wl.reuse} "
        f"permute={wl.permute} quantized={wl.quantized} {opts}")
    pr = ParityRun(wl, **opts)
    assert_reports(pr.run())


@pytest.mark.parametrize("seed", seed_range("SPA_RANDOM_LARGE_GROUP_SEEDS", 12))
def test_random_configurations_large_groups(seed):
    """Twelve seeded random small configurations whose query groups hold 9 to
    16 heads: the scoring kernel built for 16 queries with the group's last
    query repeated, and the step's append launched before the selection."""
    wl, opts = random_workload(5000 + seed, groups=(9, 16))
    log(f"[parity] random large group {seed}: B={wl.batch} hq={wl.hq} hkv={wl.hkv} p={wl.p} P={wl.P} "
        f"kind={wl.kind} contexts={wl.contexts} budget={wl.budget} {opts}")
    assert_reports(ParityRun(wl, **opts).run())
