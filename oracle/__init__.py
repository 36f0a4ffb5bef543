"""CPU oracle for sparse paged decode attention -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package. The product (``sparse_paged_attention_amd``)
never does, and the two share no code.

This module is a thin ctypes layer over ``spa_oracle.c`` (plain C, fp64
attention, exact page scores, the E4M3 quantizer of fp8 pages) and
``prefill_oracle.c`` (prefill block-sparse attention: low-rank block scores,
block selection, exact attention on the selected blocks; fp64). Each wrapper takes and returns numpy arrays in
logical (position) order; bf16 values travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spa_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "prefill_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")

ORC_OK, ORC_ERR_ARG, ORC_ERR_NONFINITE, ORC_ERR_RANGE = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile spa_oracle.c with gcc (OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(os.path.getmtime(f) for f in _SRCS):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrcJob(ctypes.Structure):
    _fields_ = [
        ("K", ctypes.c_void_p), ("V", ctypes.c_void_p), ("q", ctypes.c_void_p),
        ("L", ctypes.c_int64),
        ("D", ctypes.c_int32), ("G", ctypes.c_int32), ("dynamic", ctypes.c_int32),
        ("sink", ctypes.c_int32), ("window", ctypes.c_int32), ("p", ctypes.c_int32),
        ("budget", ctypes.c_int64),
        ("do_select", ctypes.c_int32),
        ("sel", ctypes.c_void_p), ("sel_cap", ctypes.c_int64),
        ("nsel", ctypes.c_void_p), ("Ls", ctypes.c_void_p),
        ("scores", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("rc", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build()
        L = ctypes.CDLL(path)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_budget_tokens.argtypes = [i64]
        L.orc_budget_tokens.restype = i32
        L.orc_pages_to_select.argtypes = [i64, i64, i32]
        L.orc_pages_to_select.restype = i64
        L.orc_page_summary.argtypes = [vp, i64, i32, i32, vp, vp]
        L.orc_page_scores.argtypes = [vp, i32, i32, vp, vp, i64, vp]
        L.orc_topk.argtypes = [vp, i64, i64, vp]
        L.orc_attended_set.argtypes = [i32, i64, i32, i32, i32, vp, i64, i64, vp]
        L.orc_attended_set.restype = i64
        L.orc_attend.argtypes = [vp, vp, vp, i64, i32, vp, vp, vp]
        L.orc_decode_head.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i64,
                                      i32, vp, i64, vp, vp, vp, vp, vp]
        L.orc_decode_heads.argtypes = [i32, ctypes.POINTER(OrcJob)]
        L.orc_decode_heads.restype = i32
        L.orc_num_threads.restype = i32
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [vp, i64, vp]
        L.orc_quantize_rows.argtypes = [vp, i64, i32, vp, vp]
        L.orc_bf16_round_outward.argtypes = [vp, i64, i32, vp]
        L.orc_page_summary_q8.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        L.orc_attend_q8.argtypes = [vp, vp, vp, vp, vp, i64, i32, vp, vp, vp]
        L.orc_decode_head_q8.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32,
                                         i32, i64, i32, vp, i64, vp, vp, vp, vp, vp]
        L.orc_prefill_block_scores.argtypes = [vp, i32, vp, vp, vp, i64, i32, i32, i32, vp]
        L.orc_prefill_select.argtypes = [vp, i64, i64, vp, vp, i64]
        L.orc_prefill_attend.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp]
        L.orc_prefill_attend_rows.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, vp, vp, i64, vp, i64,
                                              vp, vp]
        for name in ("orc_prefill_block_scores", "orc_prefill_select", "orc_prefill_attend",
                     "orc_prefill_attend_rows"):
            getattr(L, name).restype = ctypes.c_int
        for name in ("orc_page_summary", "orc_page_scores", "orc_topk", "orc_attend",
                     "orc_decode_head", "orc_e4m3_encode", "orc_quantize_rows",
                     "orc_bf16_round_outward", "orc_page_summary_q8", "orc_attend_q8",
                     "orc_decode_head_q8"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != ORC_OK:
        raise OracleError(f"{what} failed with oracle status {rc}")


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 arrays travel as uint16 bit patterns")
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(bits)


def budget_tokens(L: int) -> int:
    return lib().orc_budget_tokens(L)


def pages_to_select(n: int, budget: int, p: int) -> int:
    return lib().orc_pages_to_select(n, budget, p)


def page_summary(K: np.ndarray, p: int):
    """K: uint16 [L][D] -> (kmin, kmax) uint16 [ceil(L/p)][D]."""
    K = _u16(K)
    L, D = K.shape
    n = -(-L // p)
    kmin = np.empty((n, D), np.uint16)
    kmax = np.empty((n, D), np.uint16)
    _check(lib().orc_page_summary(_ptr(K), L, D, p, _ptr(kmin), _ptr(kmax)), "page_summary")
    return kmin, kmax


def page_scores(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """q: uint16 [G][D]; kmin/kmax: uint16 [n][D] -> float32 [n]."""
    q, kmin, kmax = _u16(q), _u16(kmin), _u16(kmax)
    G, D = q.shape
    n = kmin.shape[0]
    s = np.empty(n, np.float32)
    _check(lib().orc_page_scores(_ptr(q), G, D, _ptr(kmin), _ptr(kmax), n, _ptr(s)), "page_scores")
    return s


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    s = np.ascontiguousarray(scores, dtype=np.float32)
    ids = np.empty(max(k, 1), np.int32)
    _check(lib().orc_topk(_ptr(s), s.size, k, _ptr(ids)), "topk")
    return ids[:k].copy()


def attended_set(dynamic: bool, L: int, sink: int, window: int, p: int,
                 sel=None, Ls: int | None = None) -> np.ndarray:
    sel = np.ascontiguousarray(sel if sel is not None else np.zeros(0), dtype=np.int32)
    mask = np.empty(max(L, 1), np.uint8)
    cnt = lib().orc_attended_set(int(dynamic), L, sink, window, p, _ptr(sel), sel.size,
                                 L if Ls is None else Ls, _ptr(mask))
    if cnt < 0:
        raise OracleError("attended_set failed")
    return mask[:L].astype(bool)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, mask) -> tuple[np.ndarray, float]:
    """q: uint16 [D]; K, V: uint16 [L][D]; mask: bool [L] -> (out fp64 [D], lse)."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    L, D = K.shape
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    out = np.empty(D, np.float64)
    lse = np.empty(1, np.float64)
    _check(lib().orc_attend(_ptr(q), _ptr(K), _ptr(V), L, D, _ptr(m), _ptr(out), _ptr(lse)), "attend")
    return out, float(lse[0])


class HeadState:
    """Selection carried between decode steps for one dynamic (sequence, KV head)."""

    def __init__(self, cap: int):
        self.sel = np.zeros(max(cap, 1), np.int32)
        self.nsel = np.zeros(1, np.int64)
        self.Ls = np.zeros(1, np.int64)

    @property
    def pages(self) -> np.ndarray:
        return self.sel[: int(self.nsel[0])].copy()


def decode_head(K, V, q, *, dynamic: bool, sink: int, window: int, p: int, budget: int,
                do_select: bool, state: HeadState | None = None, want_scores: bool = False):
    """One decode step for one (sequence, KV head); K, V [L][D], q [G][D] (uint16).

    Returns (out fp64 [G][D], lse fp64 [G], scores or None)."""
    K, V, q = _u16(K), _u16(V), _u16(q)
    L, D = K.shape
    G = q.shape[0]
    n = -(-L // p)
    if state is None:
        state = HeadState(n)
    scores = np.full(n, np.nan, np.float32) if (want_scores and dynamic and do_select) else None
    out = np.empty((G, D), np.float64)
    lse = np.empty(G, np.float64)
    rc = lib().orc_decode_head(_ptr(K), _ptr(V), _ptr(q), L, D, G, int(dynamic), sink, window, p,
                               budget, int(do_select), _ptr(state.sel), state.sel.size,
                               _ptr(state.nsel), _ptr(state.Ls),
                               _ptr(scores) if scores is not None else None,
                               _ptr(out), _ptr(lse))
    _check(rc, "decode_head")
    return out, lse, scores


def decode_heads(jobs: list[dict]) -> list[tuple]:
    """Runs many independent decode_head jobs in parallel (OpenMP).

    Each job dict holds K, V, q, dynamic, sink, window, p, budget, do_select,
    state (HeadState), and optionally want_scores. Returns [(out, lse)] in job
    order, or [(out, lse, scores)] for every job when any job asks for scores
    (scores None where the job does not select)."""
    arr = (OrcJob * len(jobs))()
    keep = []
    results = []
    any_scores = any(j.get("want_scores") for j in jobs)
    for i, j in enumerate(jobs):
        K, V, q = _u16(j["K"]), _u16(j["V"]), _u16(j["q"])
        L, D = K.shape
        G = q.shape[0]
        st = j["state"]
        out = np.empty((G, D), np.float64)
        lse = np.empty(G, np.float64)
        sc = None
        if j.get("want_scores") and j["dynamic"] and j["do_select"]:
            sc = np.full(-(-L // j["p"]), np.nan, np.float32)
            keep.append(sc)
        keep += [K, V, q, out, lse]
        results.append((out, lse, sc) if any_scores else (out, lse))
        arr[i] = OrcJob(_ptr(K), _ptr(V), _ptr(q), L, D, G, int(j["dynamic"]), j["sink"],
                        j["window"], j["p"], j["budget"], int(j["do_select"]), _ptr(st.sel),
                        st.sel.size, _ptr(st.nsel), _ptr(st.Ls), _ptr(sc) if sc is not None else None,
                        _ptr(out), _ptr(lse), 0)
    failed = lib().orc_decode_heads(len(jobs), arr)
    if failed:
        bad = [(i, arr[i].rc) for i in range(len(jobs)) if arr[i].rc]
        raise OracleError(f"{failed} oracle jobs failed: {bad[:4]}")
    return results


# ------------------------------------------------------------------ fp8 pages

def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code (NaN for 0x7F and 0xFF)."""
    return lib().orc_e4m3_value(code)


def e4m3_encode(x) -> np.ndarray:
    """float32 array -> uint8 E4M3 codes (nearest, ties to even, saturating at 448)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _check(lib().orc_e4m3_encode(_ptr(x), x.size, _ptr(out)), "e4m3_encode")
    return out


def quantize_rows(X: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """X: uint16 bf16 [L][D] -> (codes uint8 [L][D], scales float32 [L])."""
    X = _u16(X)
    L, D = X.shape
    codes = np.empty((L, D), np.uint8)
    scales = np.empty(max(L, 1), np.float32)
    _check(lib().orc_quantize_rows(_ptr(X), L, D, _ptr(codes), _ptr(scales)), "quantize_rows")
    return codes, scales[:L].copy()


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes uint8 [L][D], scales [L] -> fp64 [L][D] (code value x scale, exact)."""
    table = np.array([e4m3_value(c) for c in range(256)], np.float64)
    return table[np.asarray(codes)] * np.asarray(scales, np.float64)[:, None]


def bf16_round_outward(x, down: bool) -> np.ndarray:
    """fp64 array -> uint16 bf16 patterns, the largest bf16 <= x (down) or the smallest >= x."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _check(lib().orc_bf16_round_outward(_ptr(x), x.size, -1 if down else 1, _ptr(out)),
           "bf16_round_outward")
    return out


def page_summary_q8(Kc: np.ndarray, Ks: np.ndarray, p: int):
    """Kc uint8 [L][D], Ks float32 [L] -> (kmin, kmax) uint16 bf16 [ceil(L/p)][D]."""
    Kc = np.ascontiguousarray(Kc, dtype=np.uint8)
    Ks = np.ascontiguousarray(Ks, dtype=np.float32)
    L, D = Kc.shape
    n = -(-L // p)
    kmin = np.empty((n, D), np.uint16)
    kmax = np.empty((n, D), np.uint16)
    _check(lib().orc_page_summary_q8(_ptr(Kc), _ptr(Ks), L, D, p, _ptr(kmin), _ptr(kmax)),
           "page_summary_q8")
    return kmin, kmax


def attend_q8(q, Kc, Ks, Vc, Vs, mask) -> tuple[np.ndarray, float]:
    """attend() over fp8 rows: q uint16 [D]; Kc, Vc uint8 [L][D]; Ks, Vs float32 [L]."""
    q = _u16(q)
    Kc, Vc = (np.ascontiguousarray(a, dtype=np.uint8) for a in (Kc, Vc))
    Ks, Vs = (np.ascontiguousarray(a, dtype=np.float32) for a in (Ks, Vs))
    L, D = Kc.shape
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    out = np.empty(D, np.float64)
    lse = np.empty(1, np.float64)
    _check(lib().orc_attend_q8(_ptr(q), _ptr(Kc), _ptr(Ks), _ptr(Vc), _ptr(Vs), L, D, _ptr(m),
                               _ptr(out), _ptr(lse)), "attend_q8")
    return out, float(lse[0])


def decode_head_q8(Kc, Ks, Vc, Vs, q, *, dynamic: bool, sink: int, window: int, p: int,
                   budget: int, do_select: bool, state: HeadState | None = None,
                   want_scores: bool = False):
    """decode_head() over fp8 rows (codes uint8 [L][D], scales float32 [L])."""
    q = _u16(q)
    Kc, Vc = (np.ascontiguousarray(a, dtype=np.uint8) for a in (Kc, Vc))
    Ks, Vs = (np.ascontiguousarray(a, dtype=np.float32) for a in (Ks, Vs))
    L, D = Kc.shape
    G = q.shape[0]
    n = -(-L // p)
    if state is None:
        state = HeadState(n)
    scores = np.full(n, np.nan, np.float32) if (want_scores and dynamic and do_select) else None
    out = np.empty((G, D), np.float64)
    lse = np.empty(G, np.float64)
    rc = lib().orc_decode_head_q8(_ptr(Kc), _ptr(Ks), _ptr(Vc), _ptr(Vs), _ptr(q), L, D, G,
                                  int(dynamic), sink, window, p, budget, int(do_select),
                                  _ptr(state.sel), state.sel.size, _ptr(state.nsel),
                                  _ptr(state.Ls), _ptr(scores) if scores is not None else None,
                                  _ptr(out), _ptr(lse))
    _check(rc, "decode_head_q8")
    return out, lse, scores


def num_threads() -> int:
    return lib().orc_num_threads()


# ------------------------------------------------------- prefill (prefill_oracle.c)

PREFILL_STREAMING, PREFILL_DENSE, PREFILL_SPARSE = 0, 1, 2


def prefill_block_scores(Q, K, Wq, Wk, b: int) -> np.ndarray:
    """One KV head's block scores for its query group: Q uint16 [G][L][D] (or
    [L][D] for G = 1), K uint16 [L][D], Wq, Wk uint16 [D][R] -> float32
    [nb][nb], S[j][i] for i < j (NaN elsewhere)."""
    Q, K, Wq, Wk = _u16(Q), _u16(K), _u16(Wq), _u16(Wk)
    if Q.ndim == 2:
        Q = Q[None]
    G, L, D = Q.shape
    R = Wq.shape[1]
    nb = -(-L // b)
    S = np.empty((nb, nb), np.float32)
    _check(lib().orc_prefill_block_scores(_ptr(Q), G, _ptr(K), _ptr(Wq), _ptr(Wk), L, D, R, b, _ptr(S)),
           "prefill_block_scores")
    return S


def prefill_select(S: np.ndarray, kb: int):
    """Selected key blocks per query block: (sel int32 [nb][kb] ascending ids,
    cnt int32 [nb]); block j keeps itself and the min(j, kb - 1) best earlier
    blocks."""
    S = np.ascontiguousarray(S, dtype=np.float32)
    nb = S.shape[0]
    sel = np.full((nb, kb), -1, np.int32)
    cnt = np.zeros(nb, np.int32)
    _check(lib().orc_prefill_select(_ptr(S), nb, kb, _ptr(sel), _ptr(cnt), kb), "prefill_select")
    return sel, cnt


def prefill_attend(Q, K, V, b: int, mode: int, sink: int = 0, window: int = 1, sel=None, cnt=None,
                   rows=None):
    """One query head's prefill attention (mode PREFILL_STREAMING, _DENSE or
    _SPARSE with sel / cnt from prefill_select): (out fp64 [L][D], lse fp64
    [L]), or only the query positions `rows` when given."""
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    L, D = Q.shape
    cap = 1
    sp = cp = None
    if mode == PREFILL_SPARSE:
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        cnt = np.ascontiguousarray(cnt, dtype=np.int32)
        cap, sp, cp = sel.shape[1], _ptr(sel), _ptr(cnt)
    if rows is None:
        out = np.empty((L, D), np.float64)
        lse = np.empty(L, np.float64)
        _check(lib().orc_prefill_attend(_ptr(Q), _ptr(K), _ptr(V), L, D, b, mode, sink, window, sp, cp, cap,
                                        _ptr(out), _ptr(lse)), "prefill_attend")
        return out, lse
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, D), np.float64)
    lse = np.empty(max(rows.size, 1), np.float64)
    _check(lib().orc_prefill_attend_rows(_ptr(Q), _ptr(K), _ptr(V), L, D, b, mode, sink, window, sp, cp, cap,
                                         _ptr(rows), rows.size, _ptr(out), _ptr(lse)), "prefill_attend_rows")
    return out, lse[:rows.size]


def prefill_head(Q, K, V, Wq, Wk, *, b: int, dynamic: bool, dense: bool, budget: int, sink: int = 0,
                 window: int = 1, rows=None):
    """The whole prefill step for one KV head and its query group: Q uint16
    [G][L][D] (or [L][D]), K, V [L][D]. Returns (out fp64 [G][n][D], lse fp64
    [G][n], sel, cnt, S) with n = L or len(rows) (sel / cnt / S None unless
    the head selects)."""
    Q = _u16(Q)
    if Q.ndim == 2:
        Q = Q[None]
    sel = cnt = S = None
    if dynamic and not dense:
        S = prefill_block_scores(Q, K, Wq, Wk, b)
        sel, cnt = prefill_select(S, max(1, budget // b))
    outs, lses = [], []
    for g in range(Q.shape[0]):
        if not dynamic:
            o, l_ = prefill_attend(Q[g], K, V, b, PREFILL_STREAMING, sink, window, rows=rows)
        elif dense:
            o, l_ = prefill_attend(Q[g], K, V, b, PREFILL_DENSE, rows=rows)
        else:
            o, l_ = prefill_attend(Q[g], K, V, b, PREFILL_SPARSE, sel=sel, cnt=cnt, rows=rows)
        outs.append(o)
        lses.append(l_)
    return np.stack(outs), np.stack(lses), sel, cnt, S
