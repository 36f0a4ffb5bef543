"""Python binding of libspa.so, the sparse paged decode-attention library for
MI355X (gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch provides device memory and the current HIP stream. The C ABI
is documented in include/spa.h; the functions here take the same arguments as
its entry points, with torch tensors in place of device pointers.

The library must be built (``python __graft_entry__.py`` or
``sparse_paged_attention_amd._build.build_library()``); importing this module
fails loudly when it is not.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPA_LIB_PATH may name another build of the same C ABI (the tests load a
# host-only AddressSanitizer build of the argument checks that way)
LIB_PATH = os.environ.get("SPA_LIB_PATH") or os.path.join(_HERE, "libspa.so")

SPA_OK, SPA_ERR_INVALID, SPA_ERR_UNSUPPORTED, SPA_ERR_POOL_EXHAUSTED, SPA_ERR_WORKSPACE, SPA_ERR_HIP = range(6)

HEAD_DIM = 128


class SpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status
        self.message = message


class PoolExhausted(SpaError):
    pass


class c_pool(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("logical_page", ctypes.c_int32), ("physical_page", ctypes.c_int32),
                ("num_phys_pages", ctypes.c_int32), ("k_pool", ctypes.c_void_p),
                ("v_pool", ctypes.c_void_p), ("summary", ctypes.c_void_p),
                ("head_slots", ctypes.c_int32), ("kv_format", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


SPA_KV_BF16, SPA_KV_FP8 = 0, 1


class c_heads(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("sink", ctypes.c_int32),
                ("window", ctypes.c_int32), ("kind", ctypes.POINTER(ctypes.c_uint8))]


class c_prefill(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("dense_below", ctypes.c_int32)]


class c_batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("stream_pages", ctypes.c_void_p)]


EXPORTS = ("spa_kv_pool_append", "spa_kv_pool_write", "spa_page_summary_update",
           "spa_select_pages", "spa_append_select_pages", "spa_sparse_decode_attn", "spa_append_decode_attn",
           "spa_workspace_bytes",
           "spa_default_budget", "spa_stream_ring_pages", "spa_alloc_create", "spa_alloc_pages", "spa_alloc_free",
           "spa_alloc_num_free", "spa_alloc_destroy", "spa_status_string", "spa_last_error",
           "spa_set_attn_blocks_per_item", "spa_probe_read_chunks",
           "spa_sparse_decode_attn_noalloc", "spa_prefill_attn", "spa_prefill_workspace_bytes")

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libspa.so; raises if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P, H, B = ctypes.POINTER(c_pool), ctypes.POINTER(c_heads), ctypes.POINTER(c_batch)
        sig = {
            "spa_kv_pool_append": ([P, H, B, vp, vp, vp], ctypes.c_int),
            "spa_kv_pool_write": ([P, H, vp, i32, i32, i64, i64, vp, vp, vp], ctypes.c_int),
            "spa_page_summary_update": ([P, H, B, vp, i32, vp], ctypes.c_int),
            "spa_select_pages": ([P, H, B, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spa_append_select_pages": ([P, H, B, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp],
                                        ctypes.c_int),
            "spa_sparse_decode_attn": ([P, H, B, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp], ctypes.c_int),
            "spa_append_decode_attn": ([P, H, B, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp],
                                       ctypes.c_int),
            "spa_workspace_bytes": ([P, H, i32, i32, i32], sz),
            "spa_default_budget": ([i64], i32),
            "spa_stream_ring_pages": ([P, H], i32),
            "spa_set_attn_blocks_per_item": ([i32], ctypes.c_int),
            "spa_alloc_create": ([i32, ctypes.POINTER(vp)], ctypes.c_int),
            "spa_alloc_pages": ([vp, i32, vp], ctypes.c_int),
            "spa_alloc_free": ([vp, i32, vp], ctypes.c_int),
            "spa_alloc_num_free": ([vp], i32),
            "spa_alloc_destroy": ([vp], None),
            "spa_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "spa_last_error": ([], ctypes.c_char_p),
            "spa_probe_read_chunks": ([vp, sz, vp, i32, i32, vp, vp], ctypes.c_int),
            "spa_sparse_decode_attn_noalloc": ([P, H, B, vp, vp, vp, vp, vp, i32, vp, vp, vp], ctypes.c_int),
            "spa_prefill_attn": ([H, i32, ctypes.POINTER(c_prefill), i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, sz, vp], ctypes.c_int),
            "spa_prefill_workspace_bytes": ([H, i32, ctypes.POINTER(c_prefill), i64], sz),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != SPA_OK:
        msg = lib().spa_last_error().decode()
        cls = PoolExhausted if status == SPA_ERR_POOL_EXHAUSTED else SpaError
        raise cls(status, msg)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


_DT = {"bf16": "torch.bfloat16", "f32": "torch.float32", "i32": "torch.int32", "u8": "torch.uint8"}


def _need(t, shape, dtype: str, name: str, optional: bool = False) -> None:
    """Checks a device tensor argument: shape (None = any extent), dtype,
    contiguity. The C ABI cannot see buffer extents, so they are checked here."""
    if t is None:
        if optional:
            return
        raise SpaError(SPA_ERR_INVALID, f"{name} is None")
    if str(t.dtype) != _DT[dtype]:
        raise SpaError(SPA_ERR_INVALID, f"{name}: dtype {t.dtype}, expected {_DT[dtype]}")
    if not t.is_contiguous():
        raise SpaError(SPA_ERR_INVALID, f"{name} must be contiguous")
    if not t.is_cuda:
        raise SpaError(SPA_ERR_INVALID, f"{name} must be a device tensor")
    if len(t.shape) != len(shape) or any(e is not None and e != a for e, a in zip(shape, t.shape)):
        raise SpaError(SPA_ERR_INVALID, f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _heads_for(heads, pool):
    if len(heads.kind) != pool.num_kv_heads:
        raise SpaError(SPA_ERR_INVALID, f"heads.kind has {len(heads.kind)} entries, pool has "
                                        f"{pool.num_kv_heads} KV heads")
    return heads.c()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ------------------------------------------------------------------ objects

@dataclass
class Pool:
    """A physical-page pool of one attention layer (device tensors).

    k: bf16 [N][S][P][D]; v: bf16 [N][S][P/p][D][p];
    summary: bf16 [N][S][P/p][2][D] or None; S = head_slots or H_kv.
    kv_format "fp8": k and v hold E4M3 codes (uint8, same shapes) and
    k_scale / v_scale the fp32 row scales [N][S][P]."""
    num_kv_heads: int
    logical_page: int
    physical_page: int
    num_phys_pages: int
    k: object
    v: object
    summary: object = None
    head_dim: int = HEAD_DIM
    head_slots: int = 0
    kv_format: str = "bf16"
    k_scale: object = None
    v_scale: object = None

    @classmethod
    def empty(cls, num_kv_heads: int, logical_page: int, physical_page: int, num_phys_pages: int,
              with_summary: bool = True, device="cuda", zero: bool = True, head_slots: int = 0,
              kv_format: str = "bf16") -> "Pool":
        import torch
        if kv_format not in ("bf16", "fp8"):
            raise SpaError(SPA_ERR_INVALID, f"kv_format {kv_format!r}: 'bf16' or 'fp8'")
        mk = torch.zeros if zero else torch.empty
        r = physical_page // logical_page
        S = head_slots or num_kv_heads
        el = torch.bfloat16 if kv_format == "bf16" else torch.uint8
        k = mk((num_phys_pages, S, physical_page, HEAD_DIM), dtype=el, device=device)
        v = mk((num_phys_pages, S, r, HEAD_DIM, logical_page), dtype=el, device=device)
        s = mk((num_phys_pages, S, r, 2, HEAD_DIM), dtype=torch.bfloat16, device=device) \
            if with_summary else None
        ks = vs = None
        if kv_format == "fp8":
            ks = mk((num_phys_pages, S, physical_page), dtype=torch.float32, device=device)
            vs = mk((num_phys_pages, S, physical_page), dtype=torch.float32, device=device)
        return cls(num_kv_heads, logical_page, physical_page, num_phys_pages, k, v, s, head_slots=head_slots,
                   kv_format=kv_format, k_scale=ks, v_scale=vs)

    def check(self) -> None:
        r = self.physical_page // max(self.logical_page, 1)
        N, S, P, p = self.num_phys_pages, self.head_slots or self.num_kv_heads, self.physical_page, self.logical_page
        el = "bf16" if self.kv_format == "bf16" else "u8"
        _need(self.k, (N, S, P, HEAD_DIM), el, "pool.k")
        _need(self.v, (N, S, r, HEAD_DIM, p), el, "pool.v")
        _need(self.summary, (N, S, r, 2, HEAD_DIM), "bf16", "pool.summary", optional=True)
        if self.kv_format == "fp8":
            _need(self.k_scale, (N, S, P), "f32", "pool.k_scale")
            _need(self.v_scale, (N, S, P), "f32", "pool.v_scale")

    def c(self) -> c_pool:
        self.check()
        fmt = SPA_KV_FP8 if self.kv_format == "fp8" else SPA_KV_BF16
        return c_pool(self.num_kv_heads, self.head_dim, self.logical_page, self.physical_page,
                      self.num_phys_pages, _ptr(self.k), _ptr(self.v), _ptr(self.summary), self.head_slots,
                      fmt, _ptr(self.k_scale), _ptr(self.v_scale))


@dataclass
class Heads:
    """Head kinds (0 streaming, 1 dynamic per KV head) and the streaming pattern."""
    num_q_heads: int
    kind: tuple
    sink: int
    window: int

    def c(self) -> c_heads:
        if len(self.kind) < 1:
            raise SpaError(SPA_ERR_INVALID, "heads.kind is empty")
        arr = (ctypes.c_uint8 * len(self.kind))(*[int(k) for k in self.kind])
        h = c_heads(self.num_q_heads, self.sink, self.window,
                    ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8)))
        h._keep = arr
        return h


@dataclass
class Batch:
    """page_table: int32 [B][max_pages] (device); seq_lens: int32 [B] (device);
    stream_pages: None or int32 [B] (device), the first page of each sequence's
    ring for window-only storage of the streaming heads."""
    page_table: object
    seq_lens: object
    stream_pages: object = None

    def c(self) -> c_batch:
        _need(self.page_table, (None, None), "i32", "page_table")
        B, mp = self.page_table.shape
        _need(self.seq_lens, (B,), "i32", "seq_lens")
        _need(self.stream_pages, (B,), "i32", "stream_pages", optional=True)
        return c_batch(B, mp, _ptr(self.page_table), _ptr(self.seq_lens), _ptr(self.stream_pages))


# ------------------------------------------------------------ entry points

def kv_pool_append(pool: Pool, batch: Batch, k_new, v_new, heads: "Heads | None" = None,
                   stream=None) -> None:
    """spa_kv_pool_append: k_new, v_new bf16 [B][H_kv][D]; with `heads`, the
    summaries of the dynamic heads' receiving pages are rebuilt in the same launch."""
    p, b = pool.c(), batch.c()
    h = _heads_for(heads, pool) if heads is not None else None
    shape = (b.batch, pool.num_kv_heads, HEAD_DIM)
    _need(k_new, shape, "bf16", "k_new")
    _need(v_new, shape, "bf16", "v_new")
    _check(lib().spa_kv_pool_append(ctypes.byref(p), ctypes.byref(h) if h is not None else None,
                                    ctypes.byref(b), _ptr(k_new), _ptr(v_new), _stream(stream)))


def kv_pool_write(pool: Pool, page_table_row, start: int, k, v, heads=None, stream_base: int = -1,
                  stream=None) -> None:
    """spa_kv_pool_write: k, v bf16 [H_kv][count][D] for positions [start, start+count);
    with `heads`, the dynamic heads' summaries of the written pages are built in the same pass;
    stream_base >= 0: the streaming heads go to the sequence's ring starting at that page."""
    p = pool.c()
    h = _heads_for(heads, pool) if heads is not None else None
    _need(page_table_row, (None,), "i32", "page_table_row")
    _need(k, (pool.num_kv_heads, None, HEAD_DIM), "bf16", "k")
    count = k.shape[1]
    _need(v, (pool.num_kv_heads, count, HEAD_DIM), "bf16", "v")
    _check(lib().spa_kv_pool_write(ctypes.byref(p), ctypes.byref(h) if h is not None else None,
                                   _ptr(page_table_row), page_table_row.shape[0], int(stream_base),
                                   start, count, _ptr(k), _ptr(v), _stream(stream)))


def stream_ring_pages(pool: Pool, heads: "Heads") -> int:
    """spa_stream_ring_pages: pages of one sequence's ring for window-only storage."""
    p, h = pool.c(), _heads_for(heads, pool)
    n = lib().spa_stream_ring_pages(ctypes.byref(p), ctypes.byref(h))
    if n <= 0:
        raise SpaError(SPA_ERR_INVALID, "stream_ring_pages: invalid shapes")
    return n


def page_summary_update(pool: Pool, heads: Heads, batch: Batch, first_pos=None, max_tokens: int = 1,
                        stream=None) -> None:
    """spa_page_summary_update (first_pos None: the page of the newest token)."""
    p, h, b = pool.c(), _heads_for(heads, pool), batch.c()
    _need(first_pos, (b.batch,), "i32", "first_pos", optional=True)
    _check(lib().spa_page_summary_update(ctypes.byref(p), ctypes.byref(h), ctypes.byref(b),
                                         _ptr(first_pos), max_tokens, _stream(stream)))


def workspace_bytes(pool: Pool, heads: Heads, batch: int, max_pages: int, k_max: int) -> int:
    p, h = pool.c(), _heads_for(heads, pool)
    n = lib().spa_workspace_bytes(ctypes.byref(p), ctypes.byref(h), batch, max_pages, k_max)
    if n == 0:
        raise SpaError(SPA_ERR_INVALID, "workspace_bytes: invalid shapes")
    return n


def select_pages(pool: Pool, heads: Heads, batch: Batch, q, budget_tokens, k_max: int,
                 sel_pages, sel_count, sel_len, scores=None, workspace=None, stream=None,
                 sel_phys=None, k_new=None, v_new=None) -> None:
    """spa_select_pages: q bf16 [B][H_q][D]; budget_tokens int32 [B];
    writes sel_pages int32 [B][H_kv][k_max], sel_count int32 [B][H_kv], sel_len int32 [B],
    and, when given, sel_phys int32 [B][H_kv][k_max] (physical page of each selected page).
    With k_new / v_new (bf16 [B][H_kv][D]): spa_append_select_pages, which also appends the
    step's token in the same launches."""
    p, h, b = pool.c(), _heads_for(heads, pool), batch.c()
    B, H = b.batch, pool.num_kv_heads
    _need(q, (B, heads.num_q_heads, HEAD_DIM), "bf16", "q")
    _need(budget_tokens, (B,), "i32", "budget_tokens")
    _need(sel_pages, (B, H, k_max), "i32", "sel_pages")
    _need(sel_count, (B, H), "i32", "sel_count")
    _need(sel_len, (B,), "i32", "sel_len")
    _need(sel_phys, (B, H, k_max), "i32", "sel_phys", optional=True)
    n_max = b.max_pages * (pool.physical_page // pool.logical_page)
    _need(scores, (B, H, n_max), "f32", "scores", optional=True)
    _need(workspace, (None,), "u8", "workspace", optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if k_new is None and v_new is None:
        _check(lib().spa_select_pages(ctypes.byref(p), ctypes.byref(h), ctypes.byref(b), _ptr(q),
                                      _ptr(budget_tokens), k_max, _ptr(sel_pages), _ptr(sel_count),
                                      _ptr(sel_len), _ptr(sel_phys), _ptr(scores), _ptr(workspace), ws_bytes,
                                      _stream(stream)))
        return
    _need(k_new, (B, H, HEAD_DIM), "bf16", "k_new")
    _need(v_new, (B, H, HEAD_DIM), "bf16", "v_new")
    _check(lib().spa_append_select_pages(ctypes.byref(p), ctypes.byref(h), ctypes.byref(b), _ptr(k_new),
                                         _ptr(v_new), _ptr(q), _ptr(budget_tokens), k_max, _ptr(sel_pages),
                                         _ptr(sel_count), _ptr(sel_len), _ptr(sel_phys), _ptr(scores),
                                         _ptr(workspace), ws_bytes, _stream(stream)))


def sparse_decode_attn(pool: Pool, heads: Heads, batch: Batch, q, sel_pages, sel_count, sel_len,
                       k_max: int, out, lse=None, workspace=None, stream=None, sel_phys=None,
                       k_new=None, v_new=None) -> None:
    """spa_sparse_decode_attn: out fp32 [B][H_q][D], lse fp32 [B][H_q] or None; sel_phys as
    written by the selection that produced sel_pages, or None to use the page table.
    With k_new / v_new (bf16 [B][H_kv][D]): spa_append_decode_attn, which also appends the
    step's token in the same launch."""
    p, h, b = pool.c(), _heads_for(heads, pool), batch.c()
    B, H, HQ = b.batch, pool.num_kv_heads, heads.num_q_heads
    _need(q, (B, HQ, HEAD_DIM), "bf16", "q")
    dyn = any(heads.kind)
    _need(sel_pages, (B, H, k_max), "i32", "sel_pages", optional=not dyn)
    _need(sel_count, (B, H), "i32", "sel_count", optional=not dyn)
    _need(sel_len, (B,), "i32", "sel_len", optional=not dyn)
    _need(sel_phys, (B, H, k_max), "i32", "sel_phys", optional=True)
    _need(out, (B, HQ, HEAD_DIM), "f32", "out")
    _need(lse, (B, HQ), "f32", "lse", optional=True)
    _need(workspace, (None,), "u8", "workspace", optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if k_new is None and v_new is None:
        _check(lib().spa_sparse_decode_attn(ctypes.byref(p), ctypes.byref(h), ctypes.byref(b), _ptr(q),
                                            _ptr(sel_pages), _ptr(sel_count), _ptr(sel_len), _ptr(sel_phys),
                                            k_max, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                            _stream(stream)))
        return
    _need(k_new, (B, H, HEAD_DIM), "bf16", "k_new")
    _need(v_new, (B, H, HEAD_DIM), "bf16", "v_new")
    _check(lib().spa_append_decode_attn(ctypes.byref(p), ctypes.byref(h), ctypes.byref(b), _ptr(k_new),
                                        _ptr(v_new), _ptr(q), _ptr(sel_pages), _ptr(sel_count), _ptr(sel_len),
                                        _ptr(sel_phys), k_max, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                        _stream(stream)))


def probe_read_chunks(base, chunk_ids, chunks_per_wave: int, sink, stream=None) -> None:
    """spa_probe_read_chunks (include/spa_probe.h): reads the 4 KiB chunks
    chunk_ids (int32, device) of the device tensor `base` once each; a
    measurement aid for the benchmark's read ceiling."""
    _need(chunk_ids, (None,), "i32", "chunk_ids")
    n = chunk_ids.numel()
    nbytes = base.numel() * base.element_size()
    _need(sink, (None,), "i32", "sink")
    if sink.numel() < -(-n // chunks_per_wave):
        raise SpaError(SPA_ERR_INVALID, "sink holds fewer words than waves")
    rc = lib().spa_probe_read_chunks(_ptr(base), nbytes, _ptr(chunk_ids), n, chunks_per_wave, _ptr(sink),
                                     _stream(stream))
    if rc != SPA_OK:
        raise SpaError(rc, "probe_read_chunks failed")


def sparse_decode_attn_noalloc(pool: Pool, heads: Heads, batch: Batch, q, sel_pages, sel_count, sel_len,
                               k_max: int, out, lse=None, stream=None, sel_phys=None) -> None:
    """spa_sparse_decode_attn_noalloc: spa_sparse_decode_attn without a
    workspace (the library's static per-GPU scratch holds the split partials;
    calls overlapping on one GPU race). Allocates nothing."""
    p, h, b = pool.c(), _heads_for(heads, pool), batch.c()
    B, H, HQ = b.batch, pool.num_kv_heads, heads.num_q_heads
    _need(q, (B, HQ, HEAD_DIM), "bf16", "q")
    dyn = any(heads.kind)
    _need(sel_pages, (B, H, k_max), "i32", "sel_pages", optional=not dyn)
    _need(sel_count, (B, H), "i32", "sel_count", optional=not dyn)
    _need(sel_len, (B,), "i32", "sel_len", optional=not dyn)
    _need(sel_phys, (B, H, k_max), "i32", "sel_phys", optional=True)
    _need(out, (B, HQ, HEAD_DIM), "f32", "out")
    _need(lse, (B, HQ), "f32", "lse", optional=True)
    _check(lib().spa_sparse_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(h), ctypes.byref(b), _ptr(q),
                                                _ptr(sel_pages), _ptr(sel_count), _ptr(sel_len), _ptr(sel_phys),
                                                k_max, _ptr(out), _ptr(lse), _stream(stream)))


@dataclass
class Prefill:
    """Configuration of spa_prefill_attn: blocks of 64 tokens, `budget` tokens
    of key blocks per query block (its own block included), dense attention
    for the dynamic heads below `dense_below` tokens."""
    budget: int = 4096
    dense_below: int = 32768
    block: int = 64
    head_dim: int = HEAD_DIM

    def c(self) -> c_prefill:
        return c_prefill(self.head_dim, self.block, self.budget, self.dense_below)


def prefill_workspace_bytes(heads: Heads, num_kv_heads: int, cfg: Prefill, seq_len: int) -> int:
    h = heads.c()
    n = lib().spa_prefill_workspace_bytes(ctypes.byref(h), num_kv_heads, ctypes.byref(cfg.c()), seq_len)
    if n == 0:
        raise SpaError(SPA_ERR_INVALID, "prefill_workspace_bytes: invalid shapes")
    return n


def prefill_attn(heads: Heads, cfg: Prefill, q, k, v, w_q, w_k, out, lse=None, sel_blocks=None, sel_count=None,
                 block_scores=None, workspace=None, stream=None) -> None:
    """spa_prefill_attn: q bf16 [H_q][L][D], k, v bf16 [H_kv][L][D], w_q, w_k bf16
    [D][D / 8]; out fp32 [H_q][L][D], lse fp32 [H_q][L] or None; optional
    sel_blocks int32 [H_kv][nb][kb], sel_count int32 [H_kv][nb], block_scores
    fp32 [H_kv][nb][nb] (nb = ceil(L / 64), kb = max(1, budget / 64) capped at nb)."""
    hkv = len(heads.kind)
    _need(q, (heads.num_q_heads, None, HEAD_DIM), "bf16", "q")
    L = q.shape[1]
    _need(k, (hkv, L, HEAD_DIM), "bf16", "k")
    _need(v, (hkv, L, HEAD_DIM), "bf16", "v")
    _need(w_q, (HEAD_DIM, HEAD_DIM // 8), "bf16", "w_q", optional=True)
    _need(w_k, (HEAD_DIM, HEAD_DIM // 8), "bf16", "w_k", optional=True)
    _need(out, (heads.num_q_heads, L, HEAD_DIM), "f32", "out")
    _need(lse, (heads.num_q_heads, L), "f32", "lse", optional=True)
    nb = -(-L // 64)
    kb = min(max(1, cfg.budget // 64), max(nb, 1))
    _need(sel_blocks, (hkv, nb, kb), "i32", "sel_blocks", optional=True)
    _need(sel_count, (hkv, nb), "i32", "sel_count", optional=True)
    _need(block_scores, (hkv, nb, nb), "f32", "block_scores", optional=True)
    _need(workspace, (None,), "u8", "workspace", optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    h = heads.c()
    _check(lib().spa_prefill_attn(ctypes.byref(h), hkv, ctypes.byref(cfg.c()), L, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(w_q), _ptr(w_k), _ptr(out), _ptr(lse), _ptr(sel_blocks), _ptr(sel_count),
                                  _ptr(block_scores), _ptr(workspace), ws_bytes, _stream(stream)))


def set_attn_blocks_per_item(blocks: int) -> None:
    """Fix the attention work-item size (16-token blocks per item), or 0 for
    the per-call automatic choice (spa_set_attn_blocks_per_item)."""
    _check(lib().spa_set_attn_blocks_per_item(blocks))


def default_budget(context_len: int) -> int:
    """min(4096, L // 32): the write-up's dynamic budget rule."""
    return lib().spa_default_budget(context_len)


class Allocator:
    """Host free list of physical page ids (spa_alloc_*)."""

    def __init__(self, num_pages: int):
        h = ctypes.c_void_p()
        _check(lib().spa_alloc_create(num_pages, ctypes.byref(h)))
        self._h = h

    def alloc(self, count: int) -> list:
        ids = (ctypes.c_int32 * max(count, 1))()
        _check(lib().spa_alloc_pages(self._h, count, ids))
        return list(ids[:count])

    def free(self, ids) -> None:
        arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        _check(lib().spa_alloc_free(self._h, len(ids), arr))

    @property
    def num_free(self) -> int:
        return lib().spa_alloc_num_free(self._h)

    def close(self) -> None:
        if self._h:
            lib().spa_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
