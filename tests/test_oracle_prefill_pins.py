"""Pins of the prefill oracle (oracle/prefill_oracle.c) against what the
LServe write-up's "3.1 预填充阶段优化" and the mathematics fix, each computed
here another way:

  - the block score is the mean over a block pair of the low-rank logits
    (Q W_q)(K_i W_k)^T / sqrt(d), over every query head of the KV head's group:
    numpy forms the whole token-by-token matrix of each head and averages its
    blocks (the oracle pools first, then projects);
  - selection: numpy.lexsort on (score descending, block id ascending), the
    query's own block always kept, min(j + 1, budget / b) blocks in all;
  - attention: torch's scaled_dot_product_attention in fp64 with the mask
    each mode implies (causal; causal within the selected blocks; sink +
    window), and the closed cases that reduce to dense causal attention: the
    dense mode below the threshold, a budget covering the sequence, a
    one-block sequence.

Pure CPU; no GPU code involved."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as W

B = 64


def inputs(L, seed=5, tied=False, planted=0, D=128):
    """One query head (head 3, of KV head 1) and its KV head."""
    pf = W.Prefill("pin", seed, L, 4, 2, (0, 1), 16, 100, 512, 1 << 30, planted=planted, tied=tied)
    return (pf, W.prefill_rows(pf, "q", 3), W.prefill_rows(pf, "k", 1), W.prefill_rows(pf, "v", 1),
            W.prefill_projection(pf, "q"), W.prefill_projection(pf, "k"))


def group(pf):
    """The queries of KV head 1's group (query heads 2 and 3): [2][L][D]."""
    return np.stack([W.prefill_rows(pf, "q", h) for h in (2, 3)])


def f64(bits):
    return W.bf16_to_f32(bits).astype(np.float64)


def sdpa(Q, K, V, mask):
    """fp64 softmax(Q K^T / sqrt(d)) V with a boolean [L][L] mask; also lse."""
    q, k, v = (torch.from_numpy(f64(x)) for x in (Q, K, V))
    m = torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=m[None])[0]
    logits = (q @ k.T) / np.sqrt(q.shape[1])
    lse = torch.logsumexp(logits.masked_fill(~m, -np.inf), dim=1)
    return out.numpy(), lse.numpy()


def causal(L):
    return np.tril(np.ones((L, L), bool))


@pytest.mark.parametrize("L", [300, 512, 64 * 7 + 1])
def test_block_score_is_the_mean_low_rank_logit_of_the_pair(L):
    """Over every query row of the block in every query head of the group and
    every key row of the key block."""
    pf, Q, K, V, Wq, Wk = inputs(L)
    Qg = group(pf)
    S = orc.prefill_block_scores(Qg, K, Wq, Wk, B)
    C = f64(K) @ f64(Wk)
    logits = np.stack([(f64(q) @ f64(Wq)) @ C.T / np.sqrt(128) for q in Qg])     # [G][L][L]
    nb = -(-L // B)
    for j in range(nb):
        for i in range(nb):
            if i >= j:
                assert np.isnan(S[j, i])
                continue
            want = logits[:, j * B:(j + 1) * B, i * B:(i + 1) * B].mean()
            got = float(S[j, i])
            assert abs(got - want) <= 2 ** -23 * abs(want) + 1e-12, (j, i, got, want)


def test_block_score_uses_both_projections_in_their_roles():
    """Swapping W_q and W_k (or the query and key roles) changes the scores."""
    pf, Q, K, V, Wq, Wk = inputs(512)
    S = orc.prefill_block_scores(Q, K, Wq, Wk, B)
    assert not np.allclose(np.nan_to_num(S), np.nan_to_num(orc.prefill_block_scores(Q, K, Wk, Wq, B)))
    assert not np.allclose(np.nan_to_num(S), np.nan_to_num(orc.prefill_block_scores(K, Q, Wq, Wk, B)))


@pytest.mark.parametrize("kb", [1, 2, 5, 40])
def test_selection_is_the_diagonal_plus_the_best_earlier_blocks(kb):
    pf, Q, K, V, Wq, Wk = inputs(64 * 23 + 9)
    S = orc.prefill_block_scores(Q, K, Wq, Wk, B)
    sel, cnt = orc.prefill_select(S, kb)
    nb = S.shape[0]
    for j in range(nb):
        k = min(j, kb - 1)
        ids = np.arange(j)
        order = np.lexsort((ids, -S[j, :j].astype(np.float64)))
        want = sorted(order[:k].tolist()) + [j]
        assert cnt[j] == k + 1 == min(j + 1, kb)
        assert sel[j, :cnt[j]].tolist() == want


def test_selection_ties_go_to_the_lowest_block_id():
    S = np.full((6, 6), np.nan, np.float32)
    for j in range(6):
        S[j, :j] = 1.0                       # every earlier block scores the same
    S[5, 3] = 2.0
    sel, cnt = orc.prefill_select(S, 3)
    assert sel[5, :3].tolist() == [0, 3, 5]
    assert sel[4, :3].tolist() == [0, 1, 4]
    assert sel[1, :2].tolist() == [0, 1] and sel[0, :1].tolist() == [0]


@pytest.mark.parametrize("L", [1, 37, 64, 200])
def test_dense_mode_is_causal_attention(L):
    pf, Q, K, V, Wq, Wk = inputs(L)
    out, lse = orc.prefill_attend(Q, K, V, B, orc.PREFILL_DENSE)
    want, wlse = sdpa(Q, K, V, causal(L))
    np.testing.assert_allclose(out, want, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(lse, wlse, atol=1e-12, rtol=1e-10)


def test_budget_covering_the_sequence_is_dense_attention():
    L = 64 * 9 + 20
    pf, Q, K, V, Wq, Wk = inputs(L)
    Qg = group(pf)
    out, lse, sel, cnt, S = orc.prefill_head(Qg, K, V, Wq, Wk, b=B, dynamic=True, dense=False, budget=L + B)
    assert (cnt == np.arange(1, cnt.size + 1)).all()
    for g in range(2):
        want, wlse = sdpa(Qg[g], K, V, causal(L))
        np.testing.assert_allclose(out[g], want, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(lse[g], wlse, atol=1e-12, rtol=1e-10)


def test_one_block_sequence_is_dense_whatever_the_budget():
    pf, Q, K, V, Wq, Wk = inputs(50)
    out, lse, sel, cnt, S = orc.prefill_head(Q, K, V, Wq, Wk, b=B, dynamic=True, dense=False, budget=B)
    want, _ = sdpa(Q, K, V, causal(50))
    np.testing.assert_allclose(out[0], want, atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("budget", [64, 192, 320])
def test_sparse_attention_is_causal_attention_inside_the_selected_blocks(budget):
    L = 64 * 11 + 33
    pf, Q, K, V, Wq, Wk = inputs(L, planted=2)
    Qg = group(pf)
    out, lse, sel, cnt, S = orc.prefill_head(Qg, K, V, Wq, Wk, b=B, dynamic=True, dense=False, budget=budget)
    mask = np.zeros((L, L), bool)
    for t in range(L):
        for i in sel[t // B, :cnt[t // B]]:
            mask[t, i * B:min((i + 1) * B, t + 1)] = True
    assert (mask <= causal(L)).all() and mask[np.arange(L), np.arange(L)].all()
    for g in range(2):                       # both heads of the group use the KV head's selection
        want, wlse = sdpa(Qg[g], K, V, mask)
        np.testing.assert_allclose(out[g], want, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(lse[g], wlse, atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("sink,window", [(16, 100), (0, 1), (64, 64), (3, 500)])
def test_streaming_head_is_sink_plus_window_causal_attention(sink, window):
    L = 260
    pf, Q, K, V, Wq, Wk = inputs(L)
    out, lse = orc.prefill_attend(Q, K, V, B, orc.PREFILL_STREAMING, sink, window)
    t = np.arange(L)[:, None]
    s = np.arange(L)[None, :]
    mask = (s <= t) & ((s < sink) | (s >= t + 1 - window))
    want, wlse = sdpa(Q, K, V, mask)
    np.testing.assert_allclose(out, want, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(lse, wlse, atol=1e-12, rtol=1e-10)


def test_one_attended_key_gives_its_value():
    """Position 0 attends itself only: out = v_0 exactly, lse = q_0.k_0/sqrt(d)."""
    pf, Q, K, V, Wq, Wk = inputs(70)
    out, lse = orc.prefill_attend(Q, K, V, B, orc.PREFILL_DENSE)
    np.testing.assert_array_equal(out[0], f64(V[0]))
    assert abs(lse[0] - f64(Q[0]) @ f64(K[0]) / np.sqrt(128)) < 1e-12


def test_sampled_rows_equal_the_full_computation():
    L = 64 * 6 + 5
    pf, Q, K, V, Wq, Wk = inputs(L)
    S = orc.prefill_block_scores(Q, K, Wq, Wk, B)
    sel, cnt = orc.prefill_select(S, 3)
    rows = np.array([0, 63, 64, 200, L - 1])
    for mode, kw in ((orc.PREFILL_SPARSE, dict(sel=sel, cnt=cnt)), (orc.PREFILL_DENSE, {}),
                     (orc.PREFILL_STREAMING, dict(sink=8, window=70))):
        full, flse = orc.prefill_attend(Q, K, V, B, mode, **kw)
        part, plse = orc.prefill_attend(Q, K, V, B, mode, rows=rows, **kw)
        np.testing.assert_array_equal(part, full[rows])
        np.testing.assert_array_equal(plse, flse[rows])


def test_planted_blocks_are_selected():
    """Sanity (not parity): with the tied random sketch, key blocks pulled along
    the queries' shared direction are among the last query block's choices."""
    pf = W.Prefill("plant", 9, 64 * 40, 4, 2, (0, 1), 16, 100, 640, 1 << 30, planted=4, tied=True)
    Q, K = group(pf), W.prefill_rows(pf, "k", 1)
    Wq, Wk = W.prefill_projection(pf, "q"), W.prefill_projection(pf, "k")
    S = orc.prefill_block_scores(Q, K, Wq, Wk, B)
    sel, cnt = orc.prefill_select(S, 10)
    planted = set(W.prefill_planted_blocks(pf, 1).tolist())
    assert len(planted & set(sel[-1, :cnt[-1]].tolist())) >= 3
