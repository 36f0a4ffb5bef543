"""Seeded synthetic inputs for sparse paged decode attention.

This module is shared by the GPU tests, the benchmark and the oracle checks.
It holds no part of the method's arithmetic: it only draws keys, values and
queries, plants structure into them, and lays out page tables. Both sides take
their inputs from here; neither side's results ever feed back into it.

Every tensor slice has its own random stream, keyed by (seed, tensor tag,
sequence, head or step), so any single (sequence, head) slice can be rebuilt
on the CPU without drawing the rest of the batch. Values are drawn as fp32
N(0, 1) and rounded to bf16 (round to nearest even).

Workloads (the shapes of the LServe write-up's Llama-3-8B / Llama-2-7B decode
measurements, bqwf.cn "3.2" latency table and "4.3"; head split from "2.1"):
  toy_4k     1 x (8 q / 2 kv), L 4096, p16/P64, kv0 streaming (64 + 512),
             kv1 dynamic budget 1024, 3 planted q-aligned pages
  llama3_32k 1 x (32 / 8), L 32768, p16/P64, kv0-3 streaming (64 + 1024),
             kv4-7 dynamic budget min(4096, L/32), massive-activation outliers
  llama3_128k 4 x (32 / 8), L 131072 + i for 16 steps, reuse C = 4,
             budget 4096, streaming window 2048, physical pages shuffled
  single_256k 1 x (32 / 8), L 262144, p32/P256, budget 4096, window 4096,
             32 planted pages correlated 0.5 with the query
  ragged_mha 16 x (32 / 32), L ~ U[16384, 131072], shared shuffled pool,
             kv0-15 streaming (64 + 1024), budget min(4096, L/32), C = 4
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream tags
_K, _V, _Q, _PLANT, _OUTLIER, _PERM, _LENS = 1, 2, 3, 4, 5, 6, 7
_PQ, _PK, _PV, _PW = 11, 12, 13, 14


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    hq: int
    hkv: int
    p: int
    P: int
    contexts: tuple          # L of each sequence at step 0 (includes that step's token)
    steps: int               # decode steps; step i appends one token, L = context + i
    reuse: int               # C: select at steps with step % C == 0
    kind: tuple              # per KV head: 0 streaming, 1 dynamic
    sink: int
    window: int
    budget: int | None       # fixed token budget; None = min(4096, L / 32)
    permute: bool            # shuffle physical pages across the pool
    planted: str | None = None   # "aligned3" or "rho05x32"
    outliers: bool = False
    quantized: bool = False  # keys, values and queries rounded to integers in [-2, 2] (many exact score ties)
    d: int = 128

    @property
    def G(self) -> int:
        return self.hq // self.hkv

    def final_len(self, b: int) -> int:
        """Tokens of sequence b after the last step."""
        return self.contexts[b] + self.steps - 1

    def seq_len(self, b: int, step: int) -> int:
        return self.contexts[b] + step

    def pages_per_seq(self, b: int) -> int:
        return -(-self.final_len(b) // self.P)

    @property
    def max_pages(self) -> int:
        return max(self.pages_per_seq(b) for b in range(self.batch))

    @property
    def num_phys_pages(self) -> int:
        return sum(self.pages_per_seq(b) for b in range(self.batch))

    def budget_at(self, L: int) -> int:
        return self.budget if self.budget is not None else min(4096, L // 32)

    @property
    def k_max(self) -> int:
        """Capacity of a selection row: the largest page count any step keeps."""
        best = 1
        for b in range(self.batch):
            for s in range(self.steps):
                L = self.seq_len(b, s)
                n = -(-L // self.p)
                best = max(best, min(n, max(1, self.budget_at(L) // self.p)))
        return best

    def selects_at(self, step: int) -> bool:
        return step % self.reuse == 0

    def scaled(self, **changes) -> "Workload":
        return dataclasses.replace(self, **changes)


def _ragged_lengths(seed: int, n: int, lo: int, hi: int) -> tuple:
    g = np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, _LENS])))
    return tuple(int(x) for x in g.integers(lo, hi + 1, size=n))


WORKLOADS = {
    "toy_4k": Workload("toy_4k", 1001, 1, 8, 2, 16, 64, (4096,), 1, 1, (0, 1), 64, 512,
                       1024, False, planted="aligned3"),
    "llama3_32k": Workload("llama3_32k", 1002, 1, 32, 8, 16, 64, (32768,), 1, 1,
                           (0, 0, 0, 0, 1, 1, 1, 1), 64, 1024, None, False, outliers=True),
    "llama3_128k": Workload("llama3_128k", 1003, 4, 32, 8, 16, 64, (131072,) * 4, 16, 4,
                            (0, 0, 0, 0, 1, 1, 1, 1), 64, 2048, 4096, True),
    "single_256k": Workload("single_256k", 1004, 1, 32, 8, 32, 256, (262144,), 1, 1,
                            (0, 0, 0, 0, 1, 1, 1, 1), 64, 4096, 4096, False,
                            planted="rho05x32"),
    "ragged_mha": Workload("ragged_mha", 1005, 16, 32, 32, 16, 64,
                           _ragged_lengths(1005, 16, 16384, 131072), 16, 4,
                           (0,) * 16 + (1,) * 16, 64, 1024, None, True),
}


def _gen(*key) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence(list(key))))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def query(wl: Workload, b: int, step: int) -> np.ndarray:
    """q of sequence b at decode step `step`: uint16 [H_q][D]."""
    g = _gen(wl.seed, _Q, b, step)
    x = g.standard_normal((wl.hq, wl.d), dtype=np.float32)
    if wl.quantized:
        x = np.clip(np.rint(x), -2, 2).astype(np.float32)
    return to_bf16_bits(x)


def planted_pages(wl: Workload, b: int, h: int) -> np.ndarray:
    """Logical pages of (b, h) whose keys are pulled toward the query."""
    if wl.planted is None or wl.kind[h] != 1:
        return np.zeros(0, np.int64)
    n = -(-wl.contexts[b] // wl.p)
    count = 3 if wl.planted == "aligned3" else 32
    g = _gen(wl.seed, _PLANT, b, h)
    # keep clear of the first page and of the page holding the newest tokens
    return np.sort(g.choice(np.arange(1, n - 1), size=count, replace=False))


def outlier_positions(wl: Workload, b: int) -> np.ndarray:
    """Positions carrying the massive activations: the start token and a
    seeded 'first newline' token in [8, 256)."""
    g = _gen(wl.seed, _OUTLIER, b)
    return np.array([0, int(g.integers(8, 256))], np.int64)


OUTLIER_CHANNELS = (1415 % 128, 2533 % 128)   # feature dims 1415 and 2533 folded into one head
OUTLIER_SCALE = 100.0


def kv_f32(wl: Workload, b: int, h: int, which: str, out: np.ndarray | None = None) -> np.ndarray:
    """Keys ('k') or values ('v') of (sequence b, KV head h) for all positions
    0 .. final_len-1, fp32 [L][D] before bf16 rounding."""
    L = wl.final_len(b)
    if out is None:
        out = np.empty((L, wl.d), np.float32)
    g = _gen(wl.seed, _K if which == "k" else _V, b, h)
    g.standard_normal(out=out, dtype=np.float32)
    if which == "k" and wl.planted is not None and wl.kind[h] == 1:
        q = bf16_to_f32(query(wl, b, 0))[h * wl.G:(h + 1) * wl.G]
        for j in planted_pages(wl, b, h):
            rows = out[j * wl.p:(j + 1) * wl.p]
            if wl.planted == "aligned3":
                s = q.sum(axis=0)
                rows += 3.0 * s / np.linalg.norm(s)
            else:
                qbar = q.sum(axis=0) / math.sqrt(wl.G)
                rows[:] = 0.5 * qbar + math.sqrt(0.75) * rows
    if wl.quantized:
        np.clip(np.rint(out, out=out), -2, 2, out=out)
    if wl.outliers:
        for t in outlier_positions(wl, b):
            if t < L:
                for c in OUTLIER_CHANNELS:
                    out[t, c] *= OUTLIER_SCALE
    return out


def kv(wl: Workload, b: int, h: int, which: str) -> np.ndarray:
    """bf16 bits [final_len][D] of keys or values for (b, h)."""
    return to_bf16_bits(kv_f32(wl, b, h, which))


def kv_all(wl: Workload, b: int, which: str, threads: int = 8) -> np.ndarray:
    """bf16 bits [H_kv][final_len][D] for sequence b, drawn in parallel."""
    L = wl.final_len(b)
    res = np.empty((wl.hkv, L, wl.d), np.uint16)

    def one(h):
        res[h] = kv(wl, b, h, which)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(wl.hkv)))
    return res


def physical_pages(wl: Workload) -> list:
    """Physical page ids of every sequence's page slots: a list of int32 arrays,
    one per sequence, together a permutation of 0 .. num_phys_pages-1
    (identity order unless the workload shuffles the pool)."""
    total = wl.num_phys_pages
    ids = np.arange(total, dtype=np.int32)
    if wl.permute:
        ids = _gen(wl.seed, _PERM).permutation(total).astype(np.int32)
    out, at = [], 0
    for b in range(wl.batch):
        n = wl.pages_per_seq(b)
        out.append(ids[at:at + n])
        at += n
    return out


def page_table(wl: Workload) -> np.ndarray:
    """int32 [B][max_pages]; unused slots hold -1."""
    pt = np.full((wl.batch, wl.max_pages), -1, np.int32)
    for b, ids in enumerate(physical_pages(wl)):
        pt[b, :ids.size] = ids
    return pt


# ---------------------------------------------------------------- prefill

@dataclasses.dataclass(frozen=True)
class Prefill:
    """A prompt's attention inputs for prefill: queries [H_q][L][D], keys and
    values [H_kv][L][D] in position order, and the low-rank projections W_q,
    W_k [D][D / 8] of the block-importance estimate. No trained projections
    exist here: W is a seeded random sketch with N(0, 1 / r) entries (r = D / 8,
    so E[W W^T] = I), and with `tied` the same W serves as W_q and W_k, which
    makes the low-rank score an unbiased estimate of the block pair's mean
    logit, the role the trained pair plays; untied, W_k has its own seed."""
    name: str
    seed: int
    L: int
    hq: int
    hkv: int
    kind: tuple
    sink: int
    window: int
    budget: int              # tokens of key blocks per query block (the diagonal block included)
    dense_below: int         # dense attention for dynamic heads when L < dense_below
    block: int = 64
    planted: int = 0         # key blocks per dynamic head pulled along the queries' shared direction
    tied: bool = True
    d: int = 128

    @property
    def rank(self) -> int:
        return self.d // 8

    @property
    def G(self) -> int:
        return self.hq // self.hkv

    @property
    def n_blocks(self) -> int:
        return -(-self.L // self.block)

    def scaled(self, **changes) -> "Prefill":
        return dataclasses.replace(self, **changes)


PREFILLS = {
    # the 128K prompt of the LServe write-up's prefill figure ("3.1": 17 s -> 9 s at
    # 128K) at Llama-3-8B attention shape, heads split as in the decode workloads
    "prefill_128k": Prefill("prefill_128k", 1101, 131072, 32, 8, (0, 0, 0, 0, 1, 1, 1, 1), 64, 2048, 4096,
                            32768, planted=16),
    # below the write-up's 32K threshold: dense attention for the dynamic heads
    "prefill_16k": Prefill("prefill_16k", 1102, 16384, 32, 8, (0, 0, 0, 0, 1, 1, 1, 1), 64, 1024, 4096, 32768),
}

QUERY_BIAS = 0.5          # queries: + 0.5 u, a shared direction (unit vector u)
PLANT_GAIN = 2.0          # planted key blocks: + 2 u


def _shared_direction(pf: Prefill) -> np.ndarray:
    u = _gen(pf.seed, _PLANT, 999).standard_normal(pf.d).astype(np.float64)
    return (u / np.linalg.norm(u)).astype(np.float32)


def prefill_planted_blocks(pf: Prefill, h: int) -> np.ndarray:
    """Key blocks of KV head h carrying the shared direction (dynamic heads)."""
    nb = pf.n_blocks
    if not pf.planted or pf.kind[h] != 1 or nb < 2:
        return np.zeros(0, np.int64)
    g = _gen(pf.seed, _PLANT, h)
    return np.sort(g.choice(np.arange(nb - 1), size=min(pf.planted, nb - 1), replace=False))


def prefill_rows(pf: Prefill, which: str, h: int) -> np.ndarray:
    """bf16 bits [L][D] of the queries ('q', query head h) or keys / values
    ('k' / 'v', KV head h) of a prefill input, N(0, 1) draws; with planted
    blocks, every query also carries QUERY_BIAS along a shared direction and
    the planted key blocks PLANT_GAIN along it."""
    tag = {"q": _PQ, "k": _PK, "v": _PV}[which]
    x = _gen(pf.seed, tag, h).standard_normal((pf.L, pf.d), dtype=np.float32)
    if pf.planted:
        u = _shared_direction(pf)
        if which == "q":
            x += np.float32(QUERY_BIAS) * u
        elif which == "k":
            for i in prefill_planted_blocks(pf, h):
                x[i * pf.block:(i + 1) * pf.block] += np.float32(PLANT_GAIN) * u
    return to_bf16_bits(x)


def prefill_projection(pf: Prefill, which: str) -> np.ndarray:
    """bf16 bits [D][D / 8] of W_q ('q') or W_k ('k')."""
    g = _gen(pf.seed, _PW, 1 if (which == "q" or pf.tied) else 2)
    x = g.standard_normal((pf.d, pf.rank), dtype=np.float32) / np.float32(math.sqrt(pf.rank))
    return to_bf16_bits(x)
