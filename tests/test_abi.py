"""Host-side checks of the C ABI: the library loads, exports every entry
point declared in include/spa.h, and rejects bad arguments on the host before
anything is launched (every call below fails validation, so no kernel runs and
no device memory is touched, with or without a GPU)."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def spa():
    import sparse_paged_attention_amd as spa
    if not os.path.exists(spa.LIB_PATH):
        from sparse_paged_attention_amd import _build
        _build.build_library()
    spa.lib()
    return spa


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(spa_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_exports_every_declared_function(spa):
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(spa.lib(), n), n
    assert set(names) == set(spa.EXPORTS)


def test_default_budget_matches_page_rule(spa):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "budget_rule.json")))
    for L, b in g["pairs"]:
        assert spa.default_budget(L) == b
    assert spa.default_budget(-5) == 0


def test_status_strings(spa):
    for s in range(6):
        assert spa.lib().spa_status_string(s)


def test_allocator_free_list(spa):
    a = spa.Allocator(8)
    assert a.num_free == 8
    ids = a.alloc(3)
    assert ids == [0, 1, 2]
    assert a.num_free == 5
    with pytest.raises(spa.PoolExhausted) as e:
        a.alloc(6)
    assert "No free pages" in str(e.value)
    assert a.num_free == 5                      # all-or-nothing
    a.free([1])
    assert a.alloc(1) == [1]                    # last freed is handed out first
    with pytest.raises(spa.SpaError):
        a.free([7])                             # not allocated
    with pytest.raises(spa.SpaError):
        a.free([0, 0])                          # twice in one call
    assert a.num_free == 5
    with pytest.raises(spa.SpaError):
        a.free([99])
    a.free([0, 1, 2])
    assert a.num_free == 8
    assert sorted(a.alloc(8)) == list(range(8))
    with pytest.raises(spa.SpaError):
        spa.Allocator(0)


FAKE = 0x1000   # never dereferenced: every call below fails validation first


def mkpool(spa, **kw):
    d = dict(num_kv_heads=8, head_dim=128, logical_page=16, physical_page=64, num_phys_pages=10,
             k_pool=FAKE, v_pool=FAKE, summary=FAKE)
    d.update(kw)
    return spa.c_pool(**d)


def mkheads(spa, hq=32, sink=64, window=1024, kind=(0, 0, 0, 0, 1, 1, 1, 1)):
    arr = (ctypes.c_uint8 * len(kind))(*kind)
    h = spa.c_heads(hq, sink, window, ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8)))
    h._keep = arr
    return h


def mkbatch(spa, B=1, mp=4, pt=FAKE, lens=FAKE):
    return spa.c_batch(B, mp, pt, lens)


def attn(spa, pool, heads, batch, q=FAKE, sel=FAKE, k_max=8, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return spa.lib().spa_sparse_decode_attn(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(batch),
                                            q, sel, sel, sel, None, k_max, out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=64), 2), (dict(head_dim=0), 1), (dict(logical_page=8), 2),
    (dict(logical_page=128, physical_page=256), 1), (dict(physical_page=40), 1),
    (dict(logical_page=16, physical_page=16 * 65), 1), (dict(num_phys_pages=0), 1),
    (dict(k_pool=None), 1), (dict(num_kv_heads=0), 1), (dict(num_kv_heads=200), 1),
    (dict(summary=None), 1), (dict(num_phys_pages=2**31 - 1), 2),
])
def test_pool_validation(spa, bad, status):
    pool = mkpool(spa, **bad)
    kind = (0,) * pool.num_kv_heads if pool.num_kv_heads in (0, 200) else (0, 0, 0, 0, 1, 1, 1, 1)
    heads = mkheads(spa, kind=kind[:8] if len(kind) >= 8 else kind)
    assert attn(spa, pool, heads, mkbatch(spa)) == status
    assert spa.lib().spa_last_error()


@pytest.mark.parametrize("bad,status", [
    (dict(hq=20), 1), (dict(hq=8 * 17), 2), (dict(hq=8 * 32), 2), (dict(hq=0), 1), (dict(sink=-1), 1),
    (dict(window=0), 1), (dict(kind=(0, 0, 0, 0, 1, 1, 1, 2)), 1),
])
def test_heads_validation(spa, bad, status):
    assert attn(spa, mkpool(spa), mkheads(spa, **bad), mkbatch(spa)) == status


def test_batch_and_buffer_validation(spa):
    pool, heads = mkpool(spa), mkheads(spa)
    assert attn(spa, pool, heads, mkbatch(spa, B=-1)) == 1
    assert attn(spa, pool, heads, mkbatch(spa, mp=0)) == 1
    assert attn(spa, pool, heads, mkbatch(spa, pt=None)) == 1
    assert attn(spa, pool, heads, mkbatch(spa), q=None) == 1
    assert attn(spa, pool, heads, mkbatch(spa), out=None) == 1
    assert attn(spa, pool, heads, mkbatch(spa), sel=None) == 1
    assert attn(spa, pool, heads, mkbatch(spa), k_max=0) == 1
    assert attn(spa, pool, heads, mkbatch(spa), ws_bytes=16) == 4
    assert attn(spa, pool, heads, mkbatch(spa), ws=None) == 4
    # an empty batch is a no-op that succeeds without touching anything
    assert attn(spa, pool, heads, mkbatch(spa, B=0, pt=None, lens=None)) == 0


def test_workspace_bytes(spa):
    pool, heads = mkpool(spa), mkheads(spa)
    n = spa.lib().spa_workspace_bytes(ctypes.byref(pool), ctypes.byref(heads), 4, 2049, 256)
    assert n >= 4 * 8 * 2049 * 4 * 4          # page scores of every head
    assert n % 256 == 0
    bad = mkpool(spa, head_dim=64)
    assert spa.lib().spa_workspace_bytes(ctypes.byref(bad), ctypes.byref(heads), 4, 2049, 256) == 0


def test_select_and_summary_validation(spa):
    L = spa.lib()
    pool, heads, batch = mkpool(spa), mkheads(spa), mkbatch(spa)
    args = lambda **o: [ctypes.byref(o.get("pool", pool)), ctypes.byref(heads), ctypes.byref(batch),
                        o.get("q", FAKE), o.get("budget", FAKE), o.get("k_max", 8), FAKE, FAKE, FAKE,
                        None, None, o.get("ws", FAKE), o.get("ws_bytes", 1 << 30), None]
    assert L.spa_select_pages(*args(k_max=0)) == 1
    assert L.spa_select_pages(*args(q=None)) == 1
    assert L.spa_select_pages(*args(budget=None)) == 1
    assert L.spa_select_pages(*args(ws_bytes=8)) == 4
    big = mkbatch(spa, mp=20000)
    assert L.spa_select_pages(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(big), FAKE, FAKE, 8,
                              FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == 2
    assert L.spa_page_summary_update(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(batch),
                                     None, 5, None) == 1
    assert L.spa_page_summary_update(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(batch),
                                     FAKE, 0, None) == 1
    assert L.spa_kv_pool_append(ctypes.byref(pool), None, ctypes.byref(batch), None, FAKE, None) == 1
    bad_heads = mkheads(spa, kind=(0, 0, 0, 0, 1, 1, 1, 3))
    assert L.spa_kv_pool_append(ctypes.byref(pool), ctypes.byref(bad_heads), ctypes.byref(batch), FAKE,
                                FAKE, None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(pool), None, FAKE, 4, -1, 250, 10, FAKE, FAKE, None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(pool), None, FAKE, 4, -1, -1, 1, FAKE, FAKE, None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(pool), None, None, 4, -1, 0, 1, FAKE, FAKE, None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(pool), None, FAKE, 4, -1, 0, 0, FAKE, FAKE, None) == 0
    assert L.spa_kv_pool_write(ctypes.byref(pool), ctypes.byref(bad_heads), FAKE, 4, -1, 0, 1, FAKE, FAKE,
                               None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(pool), ctypes.byref(heads), FAKE, 4, -1, 0, 0, FAKE, FAKE, None) == 0


def test_window_only_storage_validation(spa):
    """Rings of the streaming heads: ceil(sink / P) + ceil(window / P) + 1 pages,
    checked against the pool, and only usable together with the head kinds."""
    L = spa.lib()
    ring = lambda pool, heads: L.spa_stream_ring_pages(ctypes.byref(pool), ctypes.byref(heads))
    big_pool = mkpool(spa, num_phys_pages=1000)
    assert ring(big_pool, mkheads(spa, sink=64, window=1024)) == 1 + 16 + 1
    assert ring(big_pool, mkheads(spa, sink=65, window=1025)) == 2 + 17 + 1
    assert ring(big_pool, mkheads(spa, sink=0, window=1)) == 0 + 1 + 1
    assert ring(mkpool(spa, physical_page=256), mkheads(spa, sink=64, window=4096)) == 1 + 16 + 1
    assert ring(mkpool(spa, num_kv_heads=0), mkheads(spa)) == 0
    heads = mkheads(spa)                                     # ring of 18 pages
    small = mkpool(spa, num_phys_pages=17)
    ringed = spa.c_batch(1, 4, FAKE, FAKE, FAKE)
    assert attn(spa, small, heads, ringed) == 1              # the ring does not fit the pool
    assert L.spa_kv_pool_append(ctypes.byref(big_pool), None, ctypes.byref(ringed), FAKE, FAKE, None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(big_pool), None, FAKE, 4, 0, 0, 1, FAKE, FAKE, None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(big_pool), ctypes.byref(heads), FAKE, 4, 1000 - 17, 0, 1, FAKE,
                               FAKE, None) == 1
    assert L.spa_kv_pool_write(ctypes.byref(big_pool), ctypes.byref(heads), FAKE, 4, 1000 - 18, 0, 0, FAKE,
                               FAKE, None) == 0


def test_compact_pool_validation(spa):
    """head_slots: 0 or H_kv (one slot per head), or a compact layout holding
    the larger of the two head kinds, which needs the head kinds and rings."""
    L = spa.lib()
    heads = mkheads(spa)                                     # 4 streaming + 4 dynamic heads
    plain = mkbatch(spa)
    ringed = spa.c_batch(1, 4, FAKE, FAKE, FAKE)
    assert attn(spa, mkpool(spa, head_slots=9), heads, plain) == 1          # more slots than heads
    assert attn(spa, mkpool(spa, head_slots=-1), heads, plain) == 1
    assert attn(spa, mkpool(spa, num_phys_pages=100, head_slots=3), heads, ringed) == 1   # 4 heads of a kind
    assert attn(spa, mkpool(spa, num_phys_pages=100, head_slots=4), heads, plain) == 1    # no rings
    assert L.spa_kv_pool_append(ctypes.byref(mkpool(spa, num_phys_pages=100, head_slots=4)), None,
                                ctypes.byref(ringed), FAKE, FAKE, None) == 1               # no head kinds
    compact = mkpool(spa, num_phys_pages=100, head_slots=4)
    assert L.spa_kv_pool_write(ctypes.byref(compact), ctypes.byref(heads), FAKE, 4, -1, 0, 1, FAKE, FAKE,
                               None) == 1                                                  # no ring base
    assert L.spa_kv_pool_write(ctypes.byref(compact), ctypes.byref(heads), FAKE, 4, 50, 0, 0, FAKE, FAKE,
                               None) == 0
    all_dyn = mkheads(spa, kind=(1,) * 8)                    # no streaming head: no rings needed
    assert L.spa_kv_pool_write(ctypes.byref(mkpool(spa, head_slots=8)), ctypes.byref(all_dyn), FAKE, 4, -1, 0, 0,
                               FAKE, FAKE, None) == 0


def test_attn_blocks_per_item_setting(spa):
    """Accepted item sizes round-trip; anything else is rejected up front."""
    lib = spa.lib()
    for ok in (0, 4, 5, 6, 7, 8, 9, 10, 12, 16, 0):
        assert lib.spa_set_attn_blocks_per_item(ok) == 0
    for bad in (-1, 1, 2, 3, 11, 13, 17, 64):
        assert lib.spa_set_attn_blocks_per_item(bad) == 1
        assert b"blocks per item" in lib.spa_last_error()
    assert lib.spa_set_attn_blocks_per_item(0) == 0


def test_append_decode_attn_validation(spa):
    """The append-and-attend entry point checks its own inputs and then the
    attention's, before anything is launched."""
    L = spa.lib()
    pool, heads = mkpool(spa), mkheads(spa)

    def call(batch, k_new=FAKE, v_new=FAKE, q=FAKE, k_max=8, ws_bytes=1 << 30):
        return L.spa_append_decode_attn(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(batch), k_new,
                                        v_new, q, FAKE, FAKE, FAKE, None, k_max, FAKE, None, FAKE, ws_bytes,
                                        None)
    assert call(mkbatch(spa), k_new=None) == 1
    assert call(mkbatch(spa), v_new=None) == 1
    assert call(mkbatch(spa), q=None) == 1
    assert call(mkbatch(spa), k_max=0) == 1
    assert call(mkbatch(spa), ws_bytes=16) == 4
    assert call(mkbatch(spa, B=-1)) == 1
    assert call(mkbatch(spa, B=0, pt=None, lens=None), k_new=None, v_new=None) == 0


def test_append_select_pages_validation(spa):
    L = spa.lib()
    pool, heads = mkpool(spa), mkheads(spa)

    def call(batch, k_new=FAKE, v_new=FAKE, q=FAKE, k_max=8, ws_bytes=1 << 30):
        return L.spa_append_select_pages(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(batch), k_new,
                                         v_new, q, FAKE, k_max, FAKE, FAKE, FAKE, None, None, FAKE, ws_bytes,
                                         None)
    assert call(mkbatch(spa), k_new=None) == 1
    assert call(mkbatch(spa), v_new=None) == 1
    assert call(mkbatch(spa), q=None) == 1
    assert call(mkbatch(spa), k_max=0) == 1
    assert call(mkbatch(spa), ws_bytes=8) == 4
    assert call(mkbatch(spa, mp=20000), ws_bytes=1 << 40) == 2
    assert call(mkbatch(spa, B=0, pt=None, lens=None), k_new=None, v_new=None) == 0



def test_fp8_pool_validation(spa):
    """kv_format: SPA_KV_BF16 or SPA_KV_FP8; fp8 pages need both row-scale
    arrays. Checked on the host before anything is launched (a zero-token write
    launches nothing)."""
    L = spa.lib()
    heads = mkheads(spa)

    def write(pool):
        return L.spa_kv_pool_write(ctypes.byref(pool), ctypes.byref(heads), FAKE, 4, -1, 0, 0, FAKE, FAKE, None)

    assert write(mkpool(spa, kv_format=spa.SPA_KV_FP8, k_scale=FAKE, v_scale=FAKE)) == 0
    assert write(mkpool(spa, kv_format=spa.SPA_KV_BF16)) == 0          # scales unused
    for bad in (dict(kv_format=2), dict(kv_format=-1),
                dict(kv_format=spa.SPA_KV_FP8), dict(kv_format=spa.SPA_KV_FP8, k_scale=FAKE),
                dict(kv_format=spa.SPA_KV_FP8, v_scale=FAKE)):
        assert write(mkpool(spa, **bad)) == 1, bad
        assert b"kv_format" in L.spa_last_error() or b"scale" in L.spa_last_error()
    assert attn(spa, mkpool(spa, kv_format=spa.SPA_KV_FP8), heads, mkbatch(spa)) == 1


def launches(spa):
    """Kernel launches so far when the host-only stub build is loaded (see
    tests/asan/launch_stubs.cpp), else None."""
    f = getattr(spa.lib(), "spa_test_launch_count", None)
    return f() if f is not None else None


def test_fp8_append_select_checks_workspace_before_any_launch(spa):
    """On fp8 pools spa_append_select_pages runs the append as a launch of its
    own; a missing or short workspace (scores NULL) and missing selection
    outputs must be reported before that launch, so a failing call leaves the
    pool untouched."""
    L = spa.lib()
    pool = mkpool(spa, kv_format=spa.SPA_KV_FP8, k_scale=FAKE, v_scale=FAKE)
    heads = mkheads(spa)
    before = launches(spa)

    def call(ws=FAKE, ws_bytes=8, q=FAKE, sel=FAKE):
        return L.spa_append_select_pages(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(mkbatch(spa)), FAKE,
                                         FAKE, q, FAKE, 8, sel, FAKE, FAKE, None, None, ws, ws_bytes, None)
    assert call() == spa.SPA_ERR_WORKSPACE
    assert call(ws=None, ws_bytes=1 << 30) == spa.SPA_ERR_WORKSPACE
    assert call(ws_bytes=1 << 30, q=None) == spa.SPA_ERR_INVALID
    assert call(ws_bytes=1 << 30, sel=None) == spa.SPA_ERR_INVALID
    assert launches(spa) == before


def prefill(spa, heads=None, hkv=8, cfg=None, L=40000, q=FAKE, k=FAKE, v=FAKE, wq=FAKE, wk=FAKE, out=FAKE,
            ws=FAKE, ws_bytes=1 << 30, cfg_ptr=True):
    heads = heads or mkheads(spa)
    cfg = cfg or spa.Prefill().c()
    c = ctypes.byref(cfg) if cfg_ptr else None
    return spa.lib().spa_prefill_attn(ctypes.byref(heads), hkv, c, L, q, k, v, wq, wk, out, None, None, None,
                                      None, ws, ws_bytes, None)


def test_prefill_validation(spa):
    """spa_prefill_attn and spa_prefill_workspace_bytes reject bad arguments on
    the host: configuration, head shapes, lengths, pointers, workspace."""
    L = spa.lib()
    c = lambda **kw: spa.Prefill(**kw).c()
    assert prefill(spa, cfg_ptr=False) == 1                         # no configuration
    assert prefill(spa, hkv=0) == 1 and prefill(spa, hkv=200) == 1
    assert prefill(spa, cfg=c(head_dim=64)) == 2 and prefill(spa, cfg=c(head_dim=0)) == 1
    assert prefill(spa, cfg=c(block=32)) == 2 and prefill(spa, cfg=c(block=0)) == 1
    assert prefill(spa, cfg=c(budget=0)) == 1
    assert prefill(spa, L=-1) == 1
    assert prefill(spa, L=(1 << 24) + 1) == 2                       # positions past 2^24
    assert prefill(spa, heads=mkheads(spa, hq=12)) == 1             # H_q not a multiple of H_kv
    assert prefill(spa, heads=mkheads(spa, hq=8 * 32)) == 2         # a group of 32 is not built
    # a selection row holds at most 8192 blocks (sparse mode only; the dense
    # mode's acceptance is checked with the launch stubs below)
    assert prefill(spa, L=8193 * 64) == 2
    for name in ("q", "k", "v", "out"):
        assert prefill(spa, **{name: None}) == 1, name
    assert prefill(spa, wq=None) == 1 and prefill(spa, wk=None) == 1   # the dynamic heads select
    assert prefill(spa, ws=None) == 4
    hs = mkheads(spa)
    need = L.spa_prefill_workspace_bytes(ctypes.byref(hs), 8, ctypes.byref(c()), 40000)
    assert need > 0
    assert prefill(spa, ws_bytes=need - 1) == 4
    assert spa.lib().spa_last_error()
    # sizes: 0 for invalid shapes; the dense mode needs no selection workspace
    assert L.spa_prefill_workspace_bytes(ctypes.byref(hs), 0, ctypes.byref(c()), 40000) == 0
    assert L.spa_prefill_workspace_bytes(ctypes.byref(hs), 8, ctypes.byref(c(head_dim=64)), 40000) == 0
    dense = L.spa_prefill_workspace_bytes(ctypes.byref(hs), 8, ctypes.byref(c()), 1000)
    assert 0 < dense < need
    streaming = mkheads(spa, kind=(0,) * 8)
    assert L.spa_prefill_workspace_bytes(ctypes.byref(streaming), 8, ctypes.byref(c()), 40000) == dense


def test_every_failing_call_launches_nothing(spa):
    """With the stub build loaded, the validation failures of the calls above
    enqueue nothing, and a call that passes its checks launches."""
    if launches(spa) is None:
        pytest.skip("needs the host-only stub build (SPA_LIB_PATH)")
    before = launches(spa)
    test_batch_and_buffer_validation(spa)
    test_select_and_summary_validation(spa)
    test_append_decode_attn_validation(spa)
    test_append_select_pages_validation(spa)
    test_compact_pool_validation(spa)
    test_window_only_storage_validation(spa)
    assert launches(spa) == before
    assert attn(spa, mkpool(spa), mkheads(spa), mkbatch(spa)) == 0      # passes: one launch
    assert launches(spa) == before + 1
    test_prefill_validation(spa)
    assert launches(spa) == before + 1
    assert prefill(spa, L=0) == 0                                       # an empty prompt: nothing to do
    assert launches(spa) == before + 1
    assert prefill(spa) == 0                                            # sparse: passes, launches
    assert launches(spa) == before + 2
    assert prefill(spa, L=8193 * 64, cfg=spa.Prefill(dense_below=1 << 30).c()) == 0   # dense past 8192 blocks
    assert launches(spa) == before + 3


def test_sparse_config_of_the_write_up(spa):
    """The sparse configuration the LServe write-up gives as its example
    ("5.2 参数调优指南"; page sizes "2.2", largest logical page "5.3"), read
    from tests/golden/sparse_config.json: both page-size pairs and the largest
    logical page are accepted, a logical page past the largest is rejected,
    the static sparsity ratio maps onto half the KV heads streaming, and the
    token budget and reuse interval are those of the benchmark workload."""
    import workloads as W
    cfg = json.load(open(os.path.join(ROOT, "tests", "golden", "sparse_config.json")))
    L = spa.lib()
    heads = mkheads(spa)

    def ws(p, P):
        pool = mkpool(spa, logical_page=p, physical_page=P)
        return L.spa_workspace_bytes(ctypes.byref(pool), ctypes.byref(heads), 4, 256, 128)
    assert ws(cfg["logical_page_size"], cfg["physical_page_size"]) > 0
    assert ws(cfg["alt_logical_page_size"], cfg["alt_physical_page_size"]) > 0
    assert ws(cfg["max_logical_page_size"], 4 * cfg["max_logical_page_size"]) > 0
    assert ws(2 * cfg["max_logical_page_size"], 4 * cfg["max_logical_page_size"]) == 0
    wl = W.WORKLOADS["llama3_128k"]
    assert sum(1 for k in wl.kind if k == 0) == int(cfg["static_sparsity_ratio"] * wl.hkv)
    assert wl.budget == cfg["dynamic_token_budget"]
    assert wl.reuse == cfg["reuse_interval"]
    assert (wl.p, wl.P) == (cfg["alt_logical_page_size"], cfg["alt_physical_page_size"])


def test_noalloc_attention_scratch_limit(spa):
    """spa_sparse_decode_attn_noalloc checks its arguments like
    spa_sparse_decode_attn and rejects shapes whose partials exceed the
    static scratch (SPA_NOALLOC_SCRATCH_BYTES) before anything is enqueued
    (the scratch size check needs the stub build here: on a machine without a
    GPU the real library cannot look the scratch's address up)."""
    L = spa.lib()
    pool, heads = mkpool(spa), mkheads(spa)

    def call(batch, q=FAKE, k_max=256):
        return L.spa_sparse_decode_attn_noalloc(ctypes.byref(pool), ctypes.byref(heads), ctypes.byref(batch), q,
                                                FAKE, FAKE, FAKE, None, k_max, FAKE, None, None)
    assert call(mkbatch(spa), q=None) == spa.SPA_ERR_INVALID
    assert call(mkbatch(spa), k_max=0) == spa.SPA_ERR_INVALID
    assert call(mkbatch(spa, B=0, pt=None, lens=None)) == 0
    if launches(spa) is None:
        return
    before = launches(spa)
    assert call(mkbatch(spa, B=64)) == spa.SPA_ERR_WORKSPACE
    assert b"scratch" in L.spa_last_error()
    assert launches(spa) == before
    assert call(mkbatch(spa, B=4)) == 0
    assert launches(spa) == before + 1
