"""Pins for the oracle's fp8 pages, against what the E4M3 format and the
mathematics fix, never against the oracle's own formulas retyped:

  - E4M3 decoding of all 256 codes: torch's float8_e4m3fn (a library routine)
  - E4M3 encoding (nearest, ties to even): torch's float8_e4m3fn conversion on
    every code value, every midpoint and its fp32 neighbours, random values;
    saturation at 448 from the format's largest finite value
  - row quantization: the scale by numpy's fp32 division, the codes by torch's
    conversion of numpy's fp32 quotients, the largest code of a row at 448,
    and the format's rounding error bound
  - outward rounding to bf16: brute force over the sorted list of all finite
    bf16 values
  - summaries of fp8 pages: numpy min / max of dequantized keys (decoded by
    torch) rounded by that brute force; the bound on every q.k of the page
  - attention and whole decode steps over fp8 pages: torch SDPA in float64 on
    the dequantized rows; with power-of-two scales every dequantized value is
    a bf16 value, so each step equals the bf16 path on those values
"""
import numpy as np
import pytest
import torch

import workloads as W

E4M3_MAX = 448.0


def torch_decode(codes) -> np.ndarray:
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_bits(x) -> np.ndarray:
    return W.to_bf16_bits(np.asarray(x, np.float32))


def bf16_values(bits) -> np.ndarray:
    return W.bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


# every finite bf16 value, sorted, with one bit pattern for each
_ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
_FIN = _ALL[((_ALL >> 7) & 0xFF) != 0xFF]
_VALS = bf16_values(_FIN)
_ORDER = np.argsort(_VALS, kind="stable")
_SORTED = _VALS[_ORDER]


def brute_down(x: np.ndarray) -> np.ndarray:
    """Largest finite bf16 value <= x, by search over all of them."""
    i = np.searchsorted(_SORTED, x, side="right") - 1
    return _SORTED[i]


def brute_up(x: np.ndarray) -> np.ndarray:
    i = np.searchsorted(_SORTED, x, side="left")
    return _SORTED[i]


def dequant(codes, scales) -> np.ndarray:
    return torch_decode(codes) * np.asarray(scales, np.float64)[:, None]


def sdpa64(q, K, V, mask=None) -> np.ndarray:
    """Softmax attention in float64 (torch SDPA on the CPU): q [G][D], K/V [L][D]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, None, :]
    Kt = torch.from_numpy(np.asarray(K, np.float64))[None].expand(qt.shape[0], -1, -1)
    Vt = torch.from_numpy(np.asarray(V, np.float64))[None].expand(qt.shape[0], -1, -1)
    m = None if mask is None else torch.from_numpy(np.asarray(mask, bool)).reshape(1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m)[:, 0, :].numpy()


def rand_rows(rng, L, D=128, outliers=True):
    """Normal bf16 rows; two channels of the first row scaled x100 (the massive
    activation pattern of the 32K Llama-3 workload)."""
    x = rng.standard_normal((L, D)).astype(np.float32)
    if outliers and L:
        x[0, [7, 91]] *= 100.0
    return bf16_bits(x)


# ----------------------------------------------------------------- codes

def test_e4m3_decode_all_codes_match_torch(orc):
    ours = np.array([orc.e4m3_value(c) for c in range(256)])
    ref = torch_decode(np.arange(256))
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert ours[0x7E] == E4M3_MAX and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch(orc):
    vals = np.unique(np.abs(torch_decode(np.arange(0x7F))))          # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2                                  # ties
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)            # exact in fp32
    near = np.concatenate([np.nextafter(mids32, np.float32(0)),
                           np.nextafter(mids32, np.float32(np.inf))])
    rng = np.random.default_rng(3)
    rand = np.concatenate([rng.uniform(-463, 463, 20000),
                           rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
                           rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000)]).astype(np.float32)
    x = np.concatenate([vals, -vals, mids, -mids, near, -near, rand]).astype(np.float32)
    assert np.all(np.abs(x) < 464)                   # torch keeps these finite
    assert np.array_equal(orc.e4m3_encode(x), torch_encode(x))


def test_e4m3_encode_saturates(orc):
    x = np.array([448, 463.99, 464, 500, 1e4, 3.0e38, -448, -464, -1e30], np.float32)
    assert orc.e4m3_encode(x).tolist() == [0x7E] * 6 + [0xFE] * 3
    for bad in (np.inf, -np.inf, np.nan):
        with pytest.raises(orc.OracleError):
            orc.e4m3_encode(np.array([1.0, bad], np.float32))


# ----------------------------------------------------------- quantization

@pytest.mark.parametrize("L", [1, 16, 300])
def test_quantize_rows_scale_and_codes(orc, L):
    X = rand_rows(np.random.default_rng(L), L)
    codes, scales = orc.quantize_rows(X)
    x32 = W.bf16_to_f32(X)
    amax = np.abs(x32).max(axis=1).astype(np.float32)
    assert np.array_equal(scales, amax / np.float32(E4M3_MAX))        # one fp32 division
    quot = (x32 / scales[:, None]).astype(np.float32)                  # fp32 quotients
    assert np.array_equal(codes, torch_encode(quot))
    assert np.all(np.abs(torch_decode(codes)).max(axis=1) == E4M3_MAX)


def test_quantize_rows_error_bound(orc):
    """E4M3 keeps 3 fraction bits: a rounding error of at most 2^-4 relative in the
    normal range and 2^-10 absolute below 2^-6, both times the row's scale (plus
    the fp32 quotient's own rounding)."""
    X = rand_rows(np.random.default_rng(5), 500)
    codes, scales = orc.quantize_rows(X)
    x = bf16_values(X)
    y = x / scales[:, None]
    err = np.abs(y - torch_decode(codes))
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + np.abs(y) * 2.0 ** -23
    assert np.all(err <= bound)


def test_quantize_zero_and_tiny_rows(orc):
    X = np.zeros((3, 128), np.uint16)
    X[1, :] = 0x8000                                  # -0
    X[2, 5] = 0x0001                                  # the smallest bf16 subnormal
    codes, scales = orc.quantize_rows(X)
    assert scales[0] == 0 and scales[1] == 0 and not codes[:2].any()
    assert scales[2] == np.float32(bf16_values([1])[0]) / np.float32(448)
    assert scales[2] > 0 and torch_decode(codes[2:3])[0, 5] == E4M3_MAX
    bad = X.copy()
    bad[0, 0] = 0x7F80                                # +inf
    with pytest.raises(orc.OracleError):
        orc.quantize_rows(bad)


# ----------------------------------------------------------- bf16 rounding

def test_bf16_round_outward_brute_force(orc):
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        _SORTED[::97], np.nextafter(_SORTED[::89], np.inf),
                        np.nextafter(_SORTED[::83], -np.inf), [0.0, -0.0, 1e-45, -1e-45]])
    x = x[np.abs(x) < 3.0e38]
    down = bf16_values(orc.bf16_round_outward(x, down=True))
    up = bf16_values(orc.bf16_round_outward(x, down=False))
    assert np.array_equal(down, brute_down(x))
    assert np.array_equal(up, brute_up(x))


# ------------------------------------------------------------ summaries

@pytest.mark.parametrize("L,p", [(1, 16), (37, 16), (200, 32), (129, 64)])
def test_page_summary_q8_brute_force(orc, L, p):
    Kc, Ks = orc.quantize_rows(rand_rows(np.random.default_rng(L + p), L))
    kmin, kmax = orc.page_summary_q8(Kc, Ks, p)
    K = dequant(Kc, Ks)
    n = -(-L // p)
    lo = np.stack([K[j * p:(j + 1) * p].min(axis=0) for j in range(n)])
    hi = np.stack([K[j * p:(j + 1) * p].max(axis=0) for j in range(n)])
    assert np.array_equal(bf16_values(kmin), brute_down(lo))
    assert np.array_equal(bf16_values(kmax), brute_up(hi))


def test_page_scores_q8_bound_every_key(orc):
    rng = np.random.default_rng(21)
    L, p = 160, 16
    Kc, Ks = orc.quantize_rows(rand_rows(rng, L))
    q = bf16_bits(rng.standard_normal((4, 128)))
    kmin, kmax = orc.page_summary_q8(Kc, Ks, p)
    s = orc.page_scores(q, kmin, kmax)
    dots = bf16_values(q) @ dequant(Kc, Ks).T                          # [G][L]
    for j in range(L // p):
        assert np.float64(s[j]) >= dots[:, j * p:(j + 1) * p].sum(axis=0).max() * (1 - 1e-7)


def pow2_scaled(orc, rng, L):
    """Codes of rows quantized from bf16 data, with power-of-two scales instead of
    amax / 448: every dequantized value is then exactly a bf16 value."""
    Kc, _ = orc.quantize_rows(rand_rows(rng, L))
    Ks = (2.0 ** rng.integers(-6, 3, L)).astype(np.float32)
    K = dequant(Kc, Ks)
    Kb = bf16_bits(K)
    assert np.array_equal(bf16_values(Kb), K)
    return Kc, Ks, Kb


def test_page_summary_q8_exact_keys_equal_bf16_summary(orc):
    """With every dequantized key exactly a bf16 value, the fp8 summary is the
    bf16 summary of those keys bit for bit (the same totalOrder, -0 < +0)."""
    Kc, Ks, Kb = pow2_scaled(orc, np.random.default_rng(4), 100)
    Kc[5, :7] = 0x80                                  # -0 codes next to +0 ones
    Kc[6, :7] = 0x00
    Kc[21, 3] = 0x80
    Kb = bf16_bits(dequant(Kc, Ks))
    a = orc.page_summary_q8(Kc, Ks, 16)
    b = orc.page_summary(Kb, 16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _order(bits):
    """bf16 patterns -> keys ordered like IEEE totalOrder (-0 < +0)."""
    b = np.asarray(bits, np.uint32)
    return np.where(b & 0x8000, (~b) & 0xFFFF, b | 0x8000)


def test_page_summary_q8_grows_by_merging_the_new_key(orc):
    """Appending a key to a page changes its summary to the min / max (in
    totalOrder) of the old summary and the new key rounded outward -- what an
    append may do without re-reading the page. Pages mixing -0 and +0 keys,
    keys below the smallest bf16 subnormal, both signs."""
    rng = np.random.default_rng(31)
    for trial in range(12):
        p = 16
        rows = rand_rows(rng, p)
        if trial % 3 == 0:
            rows[rng.random((p, 128)) < 0.3] = 0x8000          # -0
        if trial % 3 == 1:
            rows[rng.random((p, 128)) < 0.3] = 0x0000
        Kc, Ks = orc.quantize_rows(rows)
        if trial % 4 == 2:                                      # scales far below the bf16 range
            Ks = (Ks * np.float32(2.0 ** -140)).astype(np.float32)
            Kc[rng.random((p, 128)) < 0.2] = 0x80
        vals = dequant(Kc, Ks)
        for i in range(1, p):
            old_min, old_max = orc.page_summary_q8(Kc[:i], Ks[:i], p)
            new_min, new_max = orc.page_summary_q8(Kc[:i + 1], Ks[:i + 1], p)
            dn = orc.bf16_round_outward(vals[i], True)
            up = orc.bf16_round_outward(vals[i], False)
            want_min = np.where(_order(dn) < _order(old_min[0]), dn, old_min[0])
            want_max = np.where(_order(up) > _order(old_max[0]), up, old_max[0])
            assert np.array_equal(new_min[0], want_min), (trial, i)
            assert np.array_equal(new_max[0], want_max), (trial, i)


def test_page_summary_q8_signed_zeros(orc):
    """-0 sorts below +0 whatever the position: a page of +0 keys then a -0 key
    has minimum -0 and maximum +0, and so does a page of -0 then +0; a key
    below the smallest bf16 subnormal rounds down to +0 (positive) or to the
    negative smallest subnormal."""
    X = np.zeros((4, 128), np.uint16)
    X[1, :] = 0x8000
    Kc, Ks = orc.quantize_rows(X)                 # zero rows: scale 0, codes +0
    Kc[1, :] = 0x80                               # -0 codes
    Ks[:] = 1.0
    for order in ([0, 1], [1, 0], [0, 0, 1, 0]):
        kmin, kmax = orc.page_summary_q8(Kc[order], Ks[order], 16)
        assert (kmin[0] == 0x8000).all() and (kmax[0] == 0x0000).all(), order
    kmin, kmax = orc.page_summary_q8(Kc[[0, 0]], Ks[[0, 0]], 16)
    assert (kmin[0] == 0x0000).all() and (kmax[0] == 0x0000).all()
    tiny = np.zeros((1, 128), np.uint8)
    tiny[0, :] = 0x01                              # smallest positive code, 2^-9
    kmin, kmax = orc.page_summary_q8(tiny, np.array([2.0 ** -140], np.float32), 16)
    assert (kmin[0] == 0x0000).all() and (kmax[0] == 0x0001).all()
    kmin, kmax = orc.page_summary_q8(tiny | 0x80, np.array([2.0 ** -140], np.float32), 16)
    assert (kmin[0] == 0x8001).all() and (kmax[0] == 0x8000).all()


# ------------------------------------------------------------ attention

def test_attend_q8_equals_sdpa(orc):
    rng = np.random.default_rng(17)
    L = 300
    Kc, Ks = orc.quantize_rows(rand_rows(rng, L))
    Vc, Vs = orc.quantize_rows(rand_rows(rng, L, outliers=False))
    q = bf16_bits(rng.standard_normal(128))
    mask = rng.random(L) < 0.4
    out, lse = orc.attend_q8(q, Kc, Ks, Vc, Vs, mask)
    ref = sdpa64(bf16_values(q)[None], dequant(Kc, Ks), dequant(Vc, Vs), mask)[0]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    x = (dequant(Kc, Ks)[mask] @ bf16_values(q)) / np.sqrt(128)
    assert abs(lse - (x.max() + np.log(np.exp(x - x.max()).sum()))) < 1e-12


@pytest.mark.parametrize("L", [1, 40, 333])
def test_decode_head_q8_full_budget_is_dense(orc, L):
    rng = np.random.default_rng(L)
    Kc, Ks = orc.quantize_rows(rand_rows(rng, L))
    Vc, Vs = orc.quantize_rows(rand_rows(rng, L, outliers=False))
    q = bf16_bits(rng.standard_normal((4, 128)))
    out, _, _ = orc.decode_head_q8(Kc, Ks, Vc, Vs, q, dynamic=True, sink=0, window=1, p=16,
                                   budget=L + 16, do_select=True)
    ref = sdpa64(bf16_values(q), dequant(Kc, Ks), dequant(Vc, Vs))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_decode_head_q8_streaming_is_masked_dense(orc):
    rng = np.random.default_rng(8)
    L, sink, window = 700, 64, 512
    Kc, Ks = orc.quantize_rows(rand_rows(rng, L))
    Vc, Vs = orc.quantize_rows(rand_rows(rng, L, outliers=False))
    q = bf16_bits(rng.standard_normal((4, 128)))
    out, _, _ = orc.decode_head_q8(Kc, Ks, Vc, Vs, q, dynamic=False, sink=sink, window=window,
                                   p=16, budget=0, do_select=False)
    mask = np.zeros(L, bool)
    mask[:sink] = True
    mask[L - window:] = True
    ref = sdpa64(bf16_values(q), dequant(Kc, Ks), dequant(Vc, Vs), mask)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_decode_head_q8_exact_values_equal_bf16_path(orc):
    """Selection under a budget below the context, then a reused selection: with
    power-of-two scales the fp8 path equals the bf16 path on the same values."""
    rng = np.random.default_rng(12)
    L, p, budget = 1000, 16, 256
    Kc, Ks, Kb = pow2_scaled(orc, rng, L)
    Vc, Vs, Vb = pow2_scaled(orc, rng, L)
    q = bf16_bits(rng.standard_normal((4, 128)))
    sa, sb = orc.HeadState(64), orc.HeadState(64)
    for step, do_select in enumerate([True, False]):
        n = L - 1 + step
        a = orc.decode_head_q8(Kc[:n], Ks[:n], Vc[:n], Vs[:n], q, dynamic=True, sink=0,
                               window=1, p=p, budget=budget, do_select=do_select, state=sa,
                               want_scores=True)
        b = orc.decode_head(Kb[:n], Vb[:n], q, dynamic=True, sink=0, window=1, p=p,
                            budget=budget, do_select=do_select, state=sb, want_scores=True)
        assert np.array_equal(sa.pages, sb.pages) and sa.pages.size == budget // p
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
        if do_select:
            np.testing.assert_array_equal(a[2], b[2])
