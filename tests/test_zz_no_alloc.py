"""spa_sparse_decode_attn_noalloc, the attention entry point that allocates
nothing (its split partials live in the library's static per-GPU scratch),
against spa_sparse_decode_attn with a workspace: two calls in a row, the
second on a smaller batch, through the C ABI; and the size limit of the
scratch reported before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import OUT_TOL, LSE_TOL, ParityRun, bits_to_bf16, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_paged_attention_amd as spa
    spa.lib()


def compare(pr: ParityRun, step: int) -> None:
    import sparse_paged_attention_amd as spa
    layer = pr.layer
    pr.run_step(step)                    # the step through the usual entry points, checked against the oracle
    q, _, _ = pr.step_inputs(step)
    qd = bits_to_bf16(q)
    out_ws, lse_ws = torch.full_like(layer.out, float("nan")), torch.full_like(layer.lse, float("nan"))
    out_na, lse_na = torch.full_like(layer.out, float("nan")), torch.full_like(layer.lse, float("nan"))
    spa.sparse_decode_attn(layer.pool, layer.heads, layer.batch, qd, layer.sel_pages, layer.sel_count,
                           layer.sel_len, layer.k_max, out_ws, lse_ws, workspace=layer.workspace,
                           sel_phys=layer.sel_phys)
    spa.sparse_decode_attn_noalloc(layer.pool, layer.heads, layer.batch, qd, layer.sel_pages, layer.sel_count,
                                   layer.sel_len, layer.k_max, out_na, lse_na, sel_phys=layer.sel_phys)
    torch.cuda.synchronize()
    err = float((out_na - out_ws).abs().max())
    lerr = float((lse_na - lse_ws).abs().max())
    log(f"[noalloc] {pr.wl.name} B={pr.wl.batch} step {step}: max |noalloc - workspace| out {err:.2e} "
        f"lse {lerr:.2e}")
    assert torch.isfinite(out_na).all() and torch.isfinite(lse_na).all()
    assert err <= OUT_TOL and lerr <= LSE_TOL
    assert torch.equal(out_na, out_ws) and torch.equal(lse_na, lse_ws)    # the same kernels and split


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    big = W.WORKLOADS["llama3_128k"].scaled(contexts=(4100, 3001, 1000, 17), steps=2, budget=512, window=300)
    small = W.WORKLOADS["llama3_128k"].scaled(contexts=(700, 33), batch=2, steps=2, budget=256, window=100)
    compare(ParityRun(big, check_heads=[(0, 0), (0, 5), (3, 6)]), 0)
    compare(ParityRun(small), 0)          # smaller input after a larger one: scratch holds stale partials


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """64 sequences x 8 KV heads x 256 selected pages need ~58 MB of partials,
    more than the 32 MiB scratch: SPA_ERR_WORKSPACE, nothing launched."""
    import sparse_paged_attention_amd as spa
    B, hkv, hq, k_max = 64, 8, 32, 256
    pool = spa.Pool.empty(hkv, 16, 64, 1)
    heads = spa.Heads(hq, (0, 0, 0, 0, 1, 1, 1, 1), 64, 2048)
    batch = spa.Batch(torch.zeros((B, 1), dtype=torch.int32, device="cuda"),
                      torch.zeros(B, dtype=torch.int32, device="cuda"))
    q = torch.zeros((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    sel = torch.zeros((B, hkv, k_max), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, hkv), dtype=torch.int32, device="cuda")
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.full((B, hq, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(spa.SpaError) as e:
        spa.sparse_decode_attn_noalloc(pool, heads, batch, q, sel, cnt, sl, k_max, out)
    assert e.value.status == spa.SPA_ERR_WORKSPACE and "scratch" in e.value.message
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
