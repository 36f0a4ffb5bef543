"""GPU parity for fp8 pages (E4M3 codes with one fp32 scale per row, bf16
summaries of the dequantized keys rounded outward): the pool bytes the HIP
writes produce against the oracle's quantizer bit for bit, and whole decode
steps against the oracle's fp8 decode step. Every test needs an MI355X and the
built library."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import ParityRun, assert_reports, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_paged_attention_amd as spa
    spa.lib()
    oracle.build()


def run(wl, steps=None, fused=False, window_only=False, compact=False, check=None):
    log(f"[fp8 parity] {wl.name} B={wl.batch} hq={wl.hq} hkv={wl.hkv} p={wl.p} P={wl.P} "
        f"contexts={wl.contexts[:4]} steps={wl.steps if steps is None else steps} fused={fused} "
        f"window_only={window_only} compact={compact}")
    pr = ParityRun(wl, check_heads=check, fused=fused, window_only=window_only, compact=compact,
                   kv_format="fp8")
    reps = pr.run(steps)
    assert_reports(reps)
    return pr, reps


@pytest.mark.parametrize("p,P", [(16, 64), (32, 256), (64, 64)])
def test_fp8_pool_bytes_bit_exact(p, P):
    """Prompt write (spa_kv_pool_write) then appended tokens (spa_kv_pool_append):
    every code, every scale and every summary equal the oracle's quantization of
    the same bf16 rows; then the summaries rebuilt from the pool
    (spa_page_summary_update) are the same bytes."""
    wl = W.Workload(f"fp8_bytes_p{p}", 3100 + p, 2, 8, 2, p, P, (1500, 333), 5, 2, (0, 1), 8, 400,
                    256, True)
    pr = ParityRun(wl, kv_format="fp8")
    for i in range(wl.steps):
        pr.layer.set_lengths([wl.seq_len(b, i) for b in range(wl.batch)])
        _, kn, vn = pr.step_inputs(i)
        from parity import bits_to_bf16
        pr.layer.append(bits_to_bf16(kn), bits_to_bf16(vn))
    torch.cuda.synchronize()
    pool = pr.layer.pool

    def check(where):
        k, v = pool.k.cpu().numpy(), pool.v.cpu().numpy()
        ks, vs = pool.k_scale.cpu().numpy(), pool.v_scale.cpu().numpy()
        summ = pool.summary.view(torch.int16).cpu().numpy().view(np.uint16)
        pt = pr.layer.page_table.cpu().numpy()
        for b in range(wl.batch):
            L = wl.seq_len(b, wl.steps - 1)
            t = np.arange(L)
            phys, slot = pt[b, t // P], t % P
            lp, i = slot // p, slot % p
            for h in range(wl.hkv):
                (Kc, Ks), (Vc, Vs) = pr.K[(b, h)], pr.V[(b, h)]
                assert np.array_equal(k[phys, h, slot], Kc[:L]), (where, b, h, "key codes")
                assert np.array_equal(ks[phys, h, slot], Ks[:L]), (where, b, h, "key scales")
                assert np.array_equal(v[phys, h, lp, :, i], Vc[:L]), (where, b, h, "value codes")
                assert np.array_equal(vs[phys, h, slot], Vs[:L]), (where, b, h, "value scales")
                if wl.kind[h]:
                    kmin, kmax = oracle.page_summary_q8(Kc[:L], Ks[:L], p)
                    j = np.arange(kmin.shape[0])
                    jp = pt[b, (j * p) // P]
                    jl = ((j * p) % P) // p
                    assert np.array_equal(summ[jp, h, jl, 0], kmin), (where, b, h, "summary min")
                    assert np.array_equal(summ[jp, h, jl, 1], kmax), (where, b, h, "summary max")

    check("written")
    pool.summary.zero_()
    pr.layer.rebuild_summaries()
    torch.cuda.synchronize()
    check("rebuilt")


def test_fp8_toy_4k():
    run(W.WORKLOADS["toy_4k"])


def test_fp8_llama3_32k_massive_activations():
    run(W.WORKLOADS["llama3_32k"])


@pytest.mark.parametrize("fused", [False, True])
def test_fp8_llama3_128k_reuse_small(fused):
    """Batch 4, shuffled pool, selection every 4 steps; fused: the append entry
    points (on fp8 pools they run the append as a launch of its own first)."""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=9, budget=512,
                                           window=300)
    run(wl, fused=fused)


def test_fp8_llama3_128k_full_size_sampled():
    """The benchmark's configuration at full size on fp8 pages: 4 x 131072 + 16
    steps, shuffled pool, reuse every 4 steps, the benchmark's launches (the
    append entry points); checked on sampled heads of both kinds."""
    run(W.WORKLOADS["llama3_128k"], check=[(0, 0), (0, 4), (1, 5), (2, 3), (3, 7)], fused=True)


def test_fp8_ragged_mha_small():
    wl = W.WORKLOADS["ragged_mha"].scaled(contexts=(2500, 40, 1800, 3333, 700, 16, 1, 2049),
                                          batch=8, steps=6)
    run(wl)


def test_fp8_p32_P256():
    run(W.WORKLOADS["single_256k"].scaled(contexts=(9000,), steps=5, window=700, sink=40))


@pytest.mark.parametrize("fused", [False, True])
def test_fp8_group_of_7(fused):
    """A group of 7 query heads per KV head (28 / 4), scored by the kernel built
    for 8, on fp8 pages."""
    run(W.Workload("fp8_g7", 3207, 2, 28, 4, 16, 64, (1500, 999), 5, 2, (1, 0, 1, 0), 32, 200, 256, True),
        fused=fused)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("compact", [False, True])
def test_fp8_window_only_storage(compact, fused):
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=9, budget=512,
                                           window=300)
    run(wl, window_only=True, compact=compact, fused=fused)


def test_fp8_append_inside_attention_pool_bytes():
    """spa_append_decode_attn and spa_append_select_pages on fp8 pages write the
    same codes, scales and summaries as spa_kv_pool_append followed by the
    plain calls, and give results within the tolerances."""
    wl = W.WORKLOADS["llama3_128k"].scaled(contexts=(1000, 333, 64, 17), steps=3, budget=256, window=200,
                                           reuse=100)
    a = ParityRun(wl, kv_format="fp8")
    b = ParityRun(wl, kv_format="fp8", fused=True)
    for i in range(wl.steps):
        assert_reports([a.run_step(i)])
        assert_reports([b.run_step(i)])
    torch.cuda.synchronize()
    for name in ("k", "v", "k_scale", "v_scale", "summary"):
        x, y = getattr(a.layer.pool, name), getattr(b.layer.pool, name)
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), name


def test_fp8_degenerate_rows_bit_exact():
    """Rows that exercise the quantizer's edges, through the prompt write of a
    fp8 pool: all zeros, all -0, a lone smallest bf16 subnormal, subnormals only
    (the scale is then an fp32 subnormal), a row reaching the largest bf16,
    mixed signs across 60 decades; codes, scales and summaries equal the
    oracle's quantization of the same rows."""
    import sparse_paged_attention_amd as spa
    rng = np.random.default_rng(77)
    p, P, count = 16, 64, 64
    X = np.empty((2, 2, count, 128), np.uint16)          # [K/V][head][token][channel]
    for kv in range(2):
        for h in range(2):
            x = (rng.standard_normal((count, 128)) * 10.0 ** rng.integers(-30, 30, (count, 1))).astype(np.float32)
            rows = W.to_bf16_bits(x)
            rows[0] = 0
            rows[1] = 0x8000
            rows[2] = 0
            rows[2, 5] = 0x0001
            rows[3] = rng.integers(1, 0x80, 128).astype(np.uint16) | (rng.integers(0, 2, 128).astype(np.uint16) << 15)
            rows[4, 9] = 0x7F7F                           # the largest finite bf16
            X[kv, h] = rows
    pool = spa.Pool.empty(2, p, P, 4, kv_format="fp8")
    heads = spa.Heads(8, (0, 1), 8, 64)
    row = torch.arange(4, dtype=torch.int32, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    spa.kv_pool_write(pool, row, 0, dev(X[0]), dev(X[1]), heads=heads)
    torch.cuda.synchronize()
    k, v = pool.k.cpu().numpy(), pool.v.cpu().numpy()
    ks, vs = pool.k_scale.cpu().numpy(), pool.v_scale.cpu().numpy()
    summ = pool.summary.view(torch.int16).cpu().numpy().view(np.uint16)
    t = np.arange(count)
    phys, slot = t // P, t % P
    for h in range(2):
        Kc, Ks = oracle.quantize_rows(X[0, h])
        Vc, Vs = oracle.quantize_rows(X[1, h])
        assert np.array_equal(ks[phys, h, slot].view(np.uint32), Ks.view(np.uint32)), (h, "key scales")
        assert np.array_equal(k[phys, h, slot], Kc), (h, "key codes")
        assert np.array_equal(vs[phys, h, slot].view(np.uint32), Vs.view(np.uint32)), (h, "value scales")
        assert np.array_equal(v[phys, h, slot // p, :, slot % p], Vc), (h, "value codes")
        if h == 1:
            kmin, kmax = oracle.page_summary_q8(Kc, Ks, p)
            j = np.arange(count // p)
            assert np.array_equal(summ[(j * p) // P, h, ((j * p) % P) // p, 0], kmin), "summary min"
            assert np.array_equal(summ[(j * p) // P, h, ((j * p) % P) // p, 1], kmax), "summary max"


@pytest.mark.parametrize("p,P", [(16, 64), (32, 256), (64, 128)])
def test_fp8_bulk_write_in_chunks_bit_exact(p, P):
    """spa_kv_pool_write into fp8 pages in chunks whose edges fall inside
    logical pages (and inside the 16-row groups the kernel quantizes together):
    every code and scale equals the oracle's quantization of the whole rows,
    and each dynamic head's summaries, built across the chunks (tokens before
    a chunk's start read back from the pool), equal the oracle's outward-rounded
    min / max of the dequantized keys."""
    from parity import bits_to_bf16
    from sparse_paged_attention_amd.runner import DecodeLayer
    wl = W.WORKLOADS["toy_4k"].scaled(contexts=(300, 77, 1, 2 * P + 3), batch=4, steps=1, permute=True,
                                      p=p, P=P, hkv=4, hq=8, kind=(1, 0, 1, 0), planted=None,
                                      name="fp8_bulk_write_chunks")
    log(f"[fp8 parity] chunked write p={p} P={P} contexts={wl.contexts}")
    pt = W.page_table(wl)
    layer = DecodeLayer(hq=wl.hq, hkv=wl.hkv, p=p, P=P, kind=wl.kind, sink=wl.sink, window=wl.window,
                        page_table=pt, num_phys_pages=wl.num_phys_pages, k_max=wl.k_max, kv_format="fp8")
    src = []
    for b in range(wl.batch):
        L = wl.contexts[b]
        K = np.stack([W.kv(wl, b, h, "k")[:L] for h in range(wl.hkv)])
        V = np.stack([W.kv(wl, b, h, "v")[:L] for h in range(wl.hkv)])
        src.append((K, V))
        edges = sorted({0, L, *[e for e in (5, 37, 38, 38 + p, 2 * P + 1) if e < L]})
        for a, e in zip(edges[:-1], edges[1:]):
            layer.write_tokens(b, a, bits_to_bf16(np.ascontiguousarray(K[:, a:e])).cuda(),
                               bits_to_bf16(np.ascontiguousarray(V[:, a:e])).cuda())
    torch.cuda.synchronize()
    pool = layer.pool
    k, v = pool.k.cpu().numpy(), pool.v.cpu().numpy()
    ks, vs = pool.k_scale.cpu().numpy(), pool.v_scale.cpu().numpy()
    summ = pool.summary.view(torch.int16).cpu().numpy().view(np.uint16)
    r = P // p
    for b in range(wl.batch):
        K, V = src[b]
        L = wl.contexts[b]
        t = np.arange(L)
        phys, slot = pt[b, t // P], t % P
        for h in range(wl.hkv):
            Kc, Ks = oracle.quantize_rows(K[h])
            Vc, Vs = oracle.quantize_rows(V[h])
            assert np.array_equal(k[phys, h, slot], Kc), (b, h, "key codes")
            assert np.array_equal(ks[phys, h, slot].view(np.uint32), Ks[:L].view(np.uint32)), (b, h, "key scales")
            assert np.array_equal(v[phys, h, slot // p, :, slot % p], Vc), (b, h, "value codes")
            assert np.array_equal(vs[phys, h, slot].view(np.uint32), Vs[:L].view(np.uint32)), (b, h, "value scales")
            if wl.kind[h]:
                kmin, kmax = oracle.page_summary_q8(Kc, Ks[:L], p)
                j = np.arange(kmin.shape[0])
                assert np.array_equal(summ[pt[b, j // r], h, j % r, 0], kmin), (b, h, "summary min")
                assert np.array_equal(summ[pt[b, j // r], h, j % r, 1], kmax), (b, h, "summary max")
