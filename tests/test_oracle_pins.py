"""Pins for the CPU oracle: checks against things the pages and mathematics fix,
never against the oracle's own formulas retyped.

  - budget rule: values of the LServe write-up's rule (golden file)
  - page summaries: numpy's min / max along the page
  - page scores: exact rational arithmetic (Python Fractions) on the
    q+ . kmax + q- . kmin form (a second formula for the same bound), the
    upper-bound invariant, a one-token page's closed form, and hand-built
    rounding cases where a plain fp32 or fp64 sum rounds wrongly
  - top-k: numpy.lexsort, and brute force over every subset on tiny inputs
  - attended sets: the sink + recent index construction, page ranges
  - attention: torch's scaled_dot_product_attention in float64 on the CPU,
    with grouped heads expanded by repeat_interleave; one- and two-token
    closed forms
  - composition: a dynamic head whose budget covers the context equals dense
    attention; a streaming head equals dense attention under its mask; reuse
    keeps the selection and adds the tail.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def bf16_frac(bits) -> Fraction:
    return Fraction(float(W.bf16_to_f32(np.array([bits], np.uint16))[0]))


def rn32(x: Fraction) -> np.float32:
    """Nearest binary32 to the exact rational x, ties to even."""
    if x == 0:
        return np.float32(0.0)
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        return (abs(Fraction(float(c)) - x), int(np.array([c], np.float32).view(np.uint32)[0]) & 1)

    return min(cands, key=key)


def bf16(x) -> np.ndarray:
    return W.to_bf16_bits(np.asarray(x, np.float32))


def rand_bf16(rng, shape, scale=1.0):
    return bf16(rng.standard_normal(shape).astype(np.float32) * scale)


def sdpa(q_bits, K_bits, V_bits, mask=None):
    """Reference attention: torch SDPA in float64 on the CPU.
    q [H][D], K/V [Hkv][L][D]; heads grouped as in the GQA code of the
    long-context survey ("2.3": repeat_interleave of K/V over the group)."""
    q = torch.from_numpy(W.bf16_to_f32(q_bits).astype(np.float64))
    K = torch.from_numpy(W.bf16_to_f32(K_bits).astype(np.float64))
    V = torch.from_numpy(W.bf16_to_f32(V_bits).astype(np.float64))
    G = q.shape[0] // K.shape[0]
    K = K.repeat_interleave(G, dim=0)
    V = V.repeat_interleave(G, dim=0)
    m = None
    if mask is not None:
        m = torch.from_numpy(np.asarray(mask, bool)).reshape(1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], K, V, attn_mask=m)
    return out[:, 0, :].numpy()


# ------------------------------------------------------------- budget rule

def test_budget_rule_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "budget_rule.json")))
    for L, budget in g["pairs"]:
        assert orc.budget_tokens(L) == budget, L


def test_pages_to_select(orc):
    # budget in tokens over the page size, at least one page, at most all pages
    assert orc.pages_to_select(256, 1024, 16) == 64          # 1024 tokens = 64 pages of 16
    assert orc.pages_to_select(8193, 4096, 16) == 256
    assert orc.pages_to_select(8192, 4096, 32) == 128
    assert orc.pages_to_select(10, 4096, 16) == 10
    assert orc.pages_to_select(10, 0, 16) == 1
    assert orc.pages_to_select(10, 31, 16) == 1


# --------------------------------------------------------------- summaries

@pytest.mark.parametrize("L,p", [(1, 16), (16, 16), (37, 16), (200, 32), (129, 64)])
def test_page_summary_matches_numpy(orc, L, p):
    rng = np.random.default_rng(L * 7 + p)
    K = rand_bf16(rng, (L, 128))
    kmin, kmax = orc.page_summary(K, p)
    Kf = W.bf16_to_f32(K)
    n = -(-L // p)
    assert kmin.shape == (n, 128)
    for j in range(n):
        rows = Kf[j * p:min(L, j * p + p)]
        np.testing.assert_array_equal(W.bf16_to_f32(kmin[j]), rows.min(axis=0))
        np.testing.assert_array_equal(W.bf16_to_f32(kmax[j]), rows.max(axis=0))


def test_page_summary_signed_zero_total_order(orc):
    K = np.zeros((2, 128), np.uint16)
    K[0, :] = 0x8000            # -0
    K[1, :] = 0x0000            # +0
    kmin, kmax = orc.page_summary(K, 16)
    assert (kmin == 0x8000).all() and (kmax == 0x0000).all()


# ------------------------------------------------------------------ scores

def exact_score(q_rows, kmin_row, kmax_row) -> np.float32:
    """max over the query group of RN32(q+ . kmax + q- . kmin), exactly."""
    best = None
    for q in q_rows:
        acc = Fraction(0)
        for c in range(len(q)):
            qc = bf16_frac(q[c])
            acc += qc * (bf16_frac(kmax_row[c]) if qc > 0 else bf16_frac(kmin_row[c]))
        s = rn32(acc)
        best = s if best is None or s > best else best
    return best


@pytest.mark.parametrize("G", [1, 4])
def test_scores_exact_rational(orc, G):
    rng = np.random.default_rng(10 + G)
    L, p = 16 * 5 + 3, 16
    K = rand_bf16(rng, (L, 128))
    q = rand_bf16(rng, (G, 128))
    kmin, kmax = orc.page_summary(K, p)
    s = orc.page_scores(q, kmin, kmax)
    for j in range(kmin.shape[0]):
        want = exact_score(q, kmin[j], kmax[j])
        assert s[j].view(np.uint32) == np.float32(want).view(np.uint32), j


def test_scores_upper_bound_every_key(orc):
    rng = np.random.default_rng(3)
    L, p, G = 16 * 4 + 5, 16, 4
    K = rand_bf16(rng, (L, 128))
    q = rand_bf16(rng, (G, 128))
    kmin, kmax = orc.page_summary(K, p)
    s = orc.page_scores(q, kmin, kmax)
    for t in range(L):
        for g in range(G):
            dot = sum(bf16_frac(q[g, c]) * bf16_frac(K[t, c]) for c in range(128))
            assert s[t // p] >= rn32(dot), (t, g)


def test_score_of_one_token_page_is_its_dot(orc):
    rng = np.random.default_rng(4)
    p, G = 16, 4
    L = 2 * p + 1                      # the last page holds exactly one token
    K = rand_bf16(rng, (L, 128))
    q = rand_bf16(rng, (G, 128))
    kmin, kmax = orc.page_summary(K, p)
    s = orc.page_scores(q, kmin, kmax)
    want = max(rn32(sum(bf16_frac(q[g, c]) * bf16_frac(K[L - 1, c]) for c in range(128)))
               for g in range(G))
    assert s[-1] == want


def _one_page(values_q, values_k):
    """q and a one-token page whose key is values_k (both padded with zeros)."""
    q = np.zeros((1, 128), np.uint16)
    k = np.zeros((1, 128), np.uint16)
    q[0, :len(values_q)] = bf16(values_q)
    k[0, :len(values_k)] = bf16(values_k)
    return q, k


def test_score_rounding_is_exact_then_round(orc):
    # 1 + 2^-24 is the midpoint between 1 and 1 + 2^-23: ties to even gives 1
    q, k = _one_page([1.0, 2.0 ** -12], [1.0, 2.0 ** -12])
    kmin, kmax = orc.page_summary(k, 16)
    assert orc.page_scores(q, kmin, kmax)[0] == np.float32(1.0)
    # a term 2^-80 below fp64 resolution decides the rounding: exact sum is just
    # above the midpoint, so RN32 is 1 + 2^-23 (an fp64 sum would give 1)
    q, k = _one_page([1.0, 2.0 ** -12, 2.0 ** -40], [1.0, 2.0 ** -12, 2.0 ** -40])
    kmin, kmax = orc.page_summary(k, 16)
    assert orc.page_scores(q, kmin, kmax)[0] == np.float32(1.0 + 2.0 ** -23)
    # exact cancellation gives +0
    q, k = _one_page([1.0, 1.0], [1.0, -1.0])
    kmin, kmax = orc.page_summary(k, 16)
    s = orc.page_scores(q, kmin, kmax)[0]
    assert s == 0 and not np.signbit(s)


def test_score_picks_kmin_for_negative_query(orc):
    # two tokens: channel 0 in {-3, 2}; q = -1 reaches its bound at kmin = -3
    K = np.zeros((2, 128), np.uint16)
    K[0, 0], K[1, 0] = bf16([-3.0])[0], bf16([2.0])[0]
    q = np.zeros((1, 128), np.uint16)
    q[0, 0] = bf16([-1.0])[0]
    kmin, kmax = orc.page_summary(K, 16)
    assert orc.page_scores(q, kmin, kmax)[0] == np.float32(3.0)
    q[0, 0] = bf16([1.0])[0]
    assert orc.page_scores(q, kmin, kmax)[0] == np.float32(2.0)


def test_score_range_is_reported(orc):
    q, k = _one_page([2.0 ** 100, 2.0 ** -100], [2.0 ** 20, 2.0 ** -20])
    kmin, kmax = orc.page_summary(k, 16)
    with pytest.raises(orc.OracleError):
        orc.page_scores(q, kmin, kmax)


# ------------------------------------------------------------------- top-k

@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (300, 64), (8193, 256)])
def test_topk_matches_lexsort(orc, n, k):
    rng = np.random.default_rng(n)
    s = rng.integers(0, 40, n).astype(np.float32)    # many ties
    ids = orc.topk(s, k)
    want = np.sort(np.lexsort((np.arange(n), -s))[:k])
    np.testing.assert_array_equal(ids, want)


def test_topk_brute_force_subsets(orc):
    rng = np.random.default_rng(5)
    for trial in range(30):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, n + 1))
        s = rng.integers(0, 4, n).astype(np.float32)
        # the kept set is the one subset where every kept page beats every
        # dropped page in (higher score, then lower id)
        good = [S for S in itertools.combinations(range(n), k)
                if all((s[a] > s[b]) or (s[a] == s[b] and a < b)
                       for a in S for b in range(n) if b not in S)]
        assert len(good) == 1
        np.testing.assert_array_equal(orc.topk(s, k), np.array(good[0]))


# ---------------------------------------------------------- attended sets

@pytest.mark.parametrize("L,sink,window", [(1, 64, 512), (100, 64, 512), (576, 64, 512),
                                           (577, 64, 512), (4096, 64, 512), (4096, 0, 1),
                                           (50, 4, 10)])
def test_streaming_set_is_sink_plus_recent(orc, L, sink, window):
    mask = orc.attended_set(False, L, sink, window, 16)
    sink_idx = np.arange(min(sink, L))
    recent_idx = np.arange(max(L - window, 0), L)
    want = np.zeros(L, bool)
    want[np.union1d(sink_idx, recent_idx)] = True
    np.testing.assert_array_equal(mask, want)


def test_dynamic_set_pages_plus_tail(orc):
    L, p = 100, 16
    sel = np.array([0, 2, 6], np.int32)          # page 6 = positions 96..99 (partial)
    mask = orc.attended_set(True, L, 0, 0, p, sel, Ls=98)
    want = np.zeros(L, bool)
    for j in sel:
        want[j * p:min(L, j * p + p)] = True
    want[98:] = True
    np.testing.assert_array_equal(mask, want)
    mask = orc.attended_set(True, L, 0, 0, p, np.array([1], np.int32), Ls=90)
    want = np.zeros(L, bool)
    want[16:32] = True
    want[90:] = True
    np.testing.assert_array_equal(mask, want)


# -------------------------------------------------------------- attention

def test_attend_dense_equals_sdpa(orc):
    rng = np.random.default_rng(6)
    L = 77
    q = rand_bf16(rng, (1, 128))
    K = rand_bf16(rng, (L, 128))
    V = rand_bf16(rng, (L, 128))
    out, lse = orc.attend(q[0], K, V, np.ones(L, bool))
    np.testing.assert_allclose(out, sdpa(q, K[None], V[None])[0], rtol=0, atol=1e-12)
    x = W.bf16_to_f32(K).astype(np.float64) @ W.bf16_to_f32(q[0]).astype(np.float64) / math.sqrt(128)
    assert abs(lse - (x.max() + math.log(np.exp(x - x.max()).sum()))) < 1e-12


def test_attend_masked_equals_sdpa(orc):
    rng = np.random.default_rng(7)
    L = 90
    q = rand_bf16(rng, (1, 128), 3.0)
    K = rand_bf16(rng, (L, 128))
    V = rand_bf16(rng, (L, 128))
    mask = rng.random(L) < 0.3
    mask[5] = True
    out, _ = orc.attend(q[0], K, V, mask)
    np.testing.assert_allclose(out, sdpa(q, K[None], V[None], mask)[0], rtol=0, atol=1e-12)


def test_attend_one_and_two_tokens(orc):
    rng = np.random.default_rng(8)
    q = rand_bf16(rng, (128,))
    K = rand_bf16(rng, (3, 128))
    V = rand_bf16(rng, (3, 128))
    out, lse = orc.attend(q, K, V, np.array([0, 1, 0], bool))
    np.testing.assert_array_equal(out, W.bf16_to_f32(V[1]).astype(np.float64))
    x = [float(W.bf16_to_f32(q).astype(np.float64) @ W.bf16_to_f32(K[t]).astype(np.float64))
         / math.sqrt(128) for t in range(3)]
    assert abs(lse - x[1]) < 1e-12
    out, _ = orc.attend(q, K, V, np.array([1, 0, 1], bool))
    sig = 1.0 / (1.0 + math.exp(-(x[2] - x[0])))
    want = sig * W.bf16_to_f32(V[2]).astype(np.float64) + (1 - sig) * W.bf16_to_f32(V[0]).astype(np.float64)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


def test_attend_empty_set(orc):
    q = np.zeros(128, np.uint16)
    K = np.zeros((4, 128), np.uint16)
    out, lse = orc.attend(q, K, K, np.zeros(4, bool))
    assert (out == 0).all() and lse == -np.inf


# ------------------------------------------------------------- composition

def _head_inputs(seed, L, G=4):
    rng = np.random.default_rng(seed)
    return rand_bf16(rng, (L, 128)), rand_bf16(rng, (L, 128)), rand_bf16(rng, (G, 128))


@pytest.mark.parametrize("L", [1, 40, 333])
def test_dynamic_full_budget_is_dense(orc, L):
    K, V, q = _head_inputs(L, L)
    out, lse, _ = orc.decode_head(K, V, q, dynamic=True, sink=0, window=1, p=16,
                                  budget=L + 16, do_select=True)
    np.testing.assert_allclose(out, sdpa(q, K[None], V[None]), rtol=0, atol=1e-12)


def test_streaming_head_is_masked_dense(orc):
    L, sink, window = 700, 64, 512
    K, V, q = _head_inputs(11, L)
    out, _, _ = orc.decode_head(K, V, q, dynamic=False, sink=sink, window=window, p=16,
                                budget=0, do_select=False)
    mask = np.zeros(L, bool)
    mask[:sink] = True
    mask[L - window:] = True
    np.testing.assert_allclose(out, sdpa(q, K[None], V[None], mask), rtol=0, atol=1e-12)
    # short sequence: the streaming head is dense
    out, _, _ = orc.decode_head(K[:500], V[:500], q, dynamic=False, sink=sink, window=window,
                                p=16, budget=0, do_select=False)
    np.testing.assert_allclose(out, sdpa(q, K[None, :500], V[None, :500]), rtol=0, atol=1e-12)


def test_dynamic_selection_then_reuse(orc):
    p, budget = 16, 64                      # 4 pages kept
    L0 = 16 * 20 + 7
    K, V, q0 = _head_inputs(12, L0 + 3)
    st = orc.HeadState(32)
    out0, _, scores = orc.decode_head(K[:L0], V[:L0], q0, dynamic=True, sink=0, window=1, p=p,
                                      budget=budget, do_select=True, state=st, want_scores=True)
    sel0 = st.pages
    np.testing.assert_array_equal(sel0, np.sort(np.lexsort((np.arange(scores.size), -scores))[:4]))
    assert int(st.Ls[0]) == L0
    mask = np.zeros(L0, bool)
    for j in sel0:
        mask[j * p:(j + 1) * p] = True
    np.testing.assert_allclose(out0, sdpa(q0, K[None, :L0], V[None, :L0], mask[:L0]), atol=1e-12)
    # two more steps without selecting: same pages, plus the new tokens
    rng = np.random.default_rng(13)
    for extra in (1, 2):
        L = L0 + extra
        q = rand_bf16(rng, (4, 128))
        out, _, _ = orc.decode_head(K[:L], V[:L], q, dynamic=True, sink=0, window=1, p=p,
                                    budget=budget, do_select=False, state=st)
        np.testing.assert_array_equal(st.pages, sel0)
        m = np.zeros(L, bool)
        m[:L0] = mask
        m[L0:] = True
        for j in sel0:
            m[j * p:min(L, (j + 1) * p)] = True
        np.testing.assert_allclose(out, sdpa(q, K[None, :L], V[None, :L], m), atol=1e-12)


def test_planted_pages_are_selected(orc):
    wl = W.WORKLOADS["toy_4k"]
    K = W.kv(wl, 0, 1, "k")[:wl.contexts[0]]
    V = W.kv(wl, 0, 1, "v")[:wl.contexts[0]]
    q = W.query(wl, 0, 0)[4:8]
    st = orc.HeadState(64)
    orc.decode_head(K, V, q, dynamic=True, sink=0, window=1, p=16, budget=1024,
                    do_select=True, state=st)
    assert set(W.planted_pages(wl, 0, 1)) <= set(st.pages.tolist())
    assert st.pages.size == 64


def test_oracle_batch_matches_single(orc):
    jobs, singles = [], []
    for h in range(3):
        K, V, q = _head_inputs(20 + h, 300)
        st1, st2 = orc.HeadState(8), orc.HeadState(8)
        singles.append(orc.decode_head(K, V, q, dynamic=bool(h % 2), sink=16, window=64, p=16,
                                       budget=64, do_select=True, state=st1))
        jobs.append(dict(K=K, V=V, q=q, dynamic=bool(h % 2), sink=16, window=64, p=16,
                         budget=64, do_select=True, state=st2))
    res = orc.decode_heads(jobs)
    for (o1, l1, _), (o2, l2) in zip(singles, res):
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
