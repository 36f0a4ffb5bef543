"""A decode-step driver for one attention layer, built on the C ABI.

DecodeLayer owns the device buffers of one layer (pool, page table, sequence
lengths, selection state, workspace, outputs) and runs the method's step:

    append the new token -> refresh the page summary it landed in
    -> [every C steps] select pages for the dynamic heads
    -> sparse decode attention for all heads

(LServe write-up, bqwf.cn: "2.1" hybrid static/dynamic sparsity, "2.2"
hierarchical pages, "3.2" reusable page selector.) All arithmetic happens in
the library's kernels; this class only allocates tensors and calls the entry
points on the current stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (Batch, Heads, Pool, kv_pool_append, kv_pool_write, page_summary_update,
               select_pages, sparse_decode_attn, stream_ring_pages, workspace_bytes)


class DecodeLayer:
    def __init__(self, *, hq: int, hkv: int, p: int, P: int, kind, sink: int, window: int,
                 page_table: np.ndarray, num_phys_pages: int, k_max: int, device="cuda",
                 resolve_at_selection: bool = True, window_only: bool = False, compact: bool = False,
                 kv_format: str = "bf16"):
        self.hq, self.hkv, self.p, self.P = hq, hkv, p, P
        self.k_max = int(k_max)
        self.device = device
        self.heads = Heads(hq, tuple(int(k) for k in kind), sink, window)
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        self.B, self.max_pages = pt.shape
        # window-only storage: each sequence's streaming heads live in a ring of
        # R pages placed after the page table's pages
        self.ring_pages = 0
        n_pages = num_phys_pages
        if window_only:
            probe = Pool.empty(hkv, p, P, 1, with_summary=any(kind), device=device)   # sizes only
            self.ring_pages = stream_ring_pages(probe, self.heads)
            n_pages += self.B * self.ring_pages
        # compact: the page table's pages hold the dynamic heads only, the rings the
        # streaming heads only (as many slots per page as the larger kind)
        n_dyn = sum(1 for x in kind if x)
        slots = max(n_dyn, hkv - n_dyn) if compact else 0
        if compact and not window_only:
            raise ValueError("the compact layout keeps streaming heads in rings: needs window_only")
        self.pool = Pool.empty(hkv, p, P, n_pages, with_summary=any(kind), device=device, head_slots=slots,
                               kv_format=kv_format)
        self.stream_pages = None
        if window_only:
            self.stream_pages = torch.arange(self.B, dtype=torch.int32, device=device) * self.ring_pages \
                + num_phys_pages
        self.page_table = torch.from_numpy(pt).to(device)
        self.lens_host = np.zeros(self.B, np.int32)
        self.seq_lens = torch.zeros(self.B, dtype=torch.int32, device=device)
        self.batch = Batch(self.page_table, self.seq_lens, self.stream_pages)
        self.sel_pages = torch.zeros((self.B, hkv, self.k_max), dtype=torch.int32, device=device)
        self.sel_count = torch.zeros((self.B, hkv), dtype=torch.int32, device=device)
        self.sel_len = torch.zeros(self.B, dtype=torch.int32, device=device)
        # physical pages of the selection, resolved once by the selection call
        # (None: attention looks the selected pages up in the page table)
        self.sel_phys = torch.zeros((self.B, hkv, self.k_max), dtype=torch.int32, device=device) \
            if resolve_at_selection else None
        self.budget = torch.zeros(self.B, dtype=torch.int32, device=device)
        nbytes = workspace_bytes(self.pool, self.heads, self.B, self.max_pages, self.k_max)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.out = torch.empty((self.B, hq, 128), dtype=torch.float32, device=device)
        self.lse = torch.empty((self.B, hq), dtype=torch.float32, device=device)

    # ----------------------------------------------------------- set-up
    def write_tokens(self, b: int, start: int, K: torch.Tensor, V: torch.Tensor, summaries: bool = True) -> None:
        """Positions [start, start + K.shape[1]) of sequence b; K, V bf16 [H_kv][n][D] on device.
        With `summaries`, the dynamic heads' page summaries are built in the same pass."""
        base = -1 if self.stream_pages is None else int(self.stream_pages[b])
        kv_pool_write(self.pool, self.page_table[b], start, K.contiguous(), V.contiguous(),
                      heads=self.heads if (summaries or base >= 0) else None, stream_base=base)

    def set_lengths(self, lens) -> None:
        self.lens_host = np.asarray(lens, np.int32).copy()
        self.seq_lens.copy_(torch.from_numpy(self.lens_host))

    def rebuild_summaries(self) -> None:
        """Summaries of every page of every sequence (bulk mode)."""
        first = torch.zeros(self.B, dtype=torch.int32, device=self.device)
        page_summary_update(self.pool, self.heads, self.batch, first, int(self.lens_host.max()))

    # ------------------------------------------------------------- step
    def set_budget(self, budget) -> None:
        self.budget.copy_(torch.as_tensor(np.asarray(budget, np.int32)))

    def use_lengths(self, seq_lens: torch.Tensor) -> None:
        """Points the batch at a device int32 [B] tensor of lengths prepared by the caller."""
        self.seq_lens = seq_lens
        self.batch = Batch(self.page_table, seq_lens, self.stream_pages)

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        """Appends one token to every sequence: k_new, v_new bf16 [B][H_kv][D].
        seq_lens must already count the new token (see use_lengths / set_lengths)."""
        kv_pool_append(self.pool, self.batch, k_new, v_new, heads=self.heads)

    def select(self, q: torch.Tensor, scores=None) -> None:
        select_pages(self.pool, self.heads, self.batch, q, self.budget, self.k_max, self.sel_pages,
                     self.sel_count, self.sel_len, scores=scores, workspace=self.workspace,
                     sel_phys=self.sel_phys)

    def attend(self, q: torch.Tensor) -> None:
        sparse_decode_attn(self.pool, self.heads, self.batch, q, self.sel_pages, self.sel_count,
                           self.sel_len, self.k_max, self.out, self.lse, workspace=self.workspace,
                           sel_phys=self.sel_phys)

    def append_select(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, scores=None) -> None:
        """append + select, the append inside the selection's scoring launch."""
        select_pages(self.pool, self.heads, self.batch, q, self.budget, self.k_max, self.sel_pages,
                     self.sel_count, self.sel_len, scores=scores, workspace=self.workspace,
                     sel_phys=self.sel_phys, k_new=k_new, v_new=v_new)

    def append_attend(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        """append + attend in one launch (steps that reuse an earlier selection)."""
        sparse_decode_attn(self.pool, self.heads, self.batch, q, self.sel_pages, self.sel_count,
                           self.sel_len, self.k_max, self.out, self.lse, workspace=self.workspace,
                           sel_phys=self.sel_phys, k_new=k_new, v_new=v_new)

    def step(self, q, k_new, v_new, do_select: bool) -> None:
        """One decode step; seq_lens must already hold the lengths after the append.
        The append runs inside the selection's scoring launch on selecting steps and
        inside the attention launch on the others."""
        if do_select:
            self.append_select(q, k_new, v_new)
            self.attend(q)
        else:
            self.append_attend(q, k_new, v_new)
