"""The algorithmic byte counts the benchmark divides by its times, against the
closed form of the 128K workload (4 sequences, 32 query / 8 KV heads, d 128,
logical pages of 16 in physical pages of 64, 4 streaming heads with sink 64 +
window 2048, 4 dynamic heads keeping 256 pages of 16 tokens), written out here
term by term."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402

ROW = 128 * 2            # one bf16 key or value row


def test_attention_bytes_at_128k():
    wl = W.WORKLOADS["llama3_128k"]
    L = 131072 + 15                                    # the last decode step's length
    kv = 4 * (4 * (64 + 2048) + 4 * 256 * 16) * 2 * ROW  # streaming and dynamic tokens, K and V rows
    q = 4 * 32 * ROW
    out = 4 * 32 * (128 * 4 + 4)                       # fp32 output rows and lse
    sel = 4 * 4 * 256 * 4                              # selected page ids
    pt = 4 * (L // 64 + 1) * 4                         # page-table entries
    assert bench.algorithmic_bytes(wl, L, False)["attn"] == kv + q + out + sel + pt == 51003920


def test_selection_and_write_bytes_at_128k():
    wl = W.WORKLOADS["llama3_128k"]
    L = 131072
    n = L // 16                                        # logical pages (L is a multiple of 16 here)
    summaries = 4 * 4 * n * 2 * ROW                    # min and max rows of every page of each dynamic head
    scores = 4 * 4 * n * 4 * 2                         # fp32 scores written and read back
    sel = bench.algorithmic_bytes(wl, L, True)["select"]
    assert sel == summaries + 4 * 32 * ROW + scores + 4 * 4 * 256 * 4
    count = 131071                                     # one prompt
    rows = 2 * 2 * 8 * count * ROW                     # K and V rows of 8 heads, read and written
    summaries_written = 4 * 8192 * 2 * ROW             # 8192 logical pages of each dynamic head
    page_table = 2048 * 4                              # physical pages of the prompt
    assert bench.bulk_write_bytes(wl, count) == rows + summaries_written + page_table == 1090519040


def test_fp8_bytes_at_128k():
    """fp8 pages: a stored row is 128 one-byte codes and its 4-byte fp32 scale;
    the query, output, selection and page-table terms are those of bf16."""
    wl = W.WORKLOADS["llama3_128k"]
    L = 131072 + 15
    ROW8 = 128 + 4
    kv = 4 * (4 * (64 + 2048) + 4 * 256 * 16) * 2 * ROW8
    rest = 4 * 32 * ROW + 4 * 32 * (128 * 4 + 4) + 4 * 4 * 256 * 4 + 4 * (L // 64 + 1) * 4
    assert bench.algorithmic_bytes(wl, L, False, ROW8)["attn"] == kv + rest == 26370576
    count = 131071
    written = 2 * 8 * count * (ROW + ROW8)              # bf16 rows read, fp8 rows written, K and V
    assert bench.bulk_write_bytes(wl, count, ROW8) == written + 4 * 8192 * 2 * ROW + 2048 * 4


def test_timed_steps_are_whole_reuse_cycles():
    """Whatever --steps / --warmup say, the timed region is whole reuse cycles
    of every layer replica (one selecting step in C), at least 20 of them, so
    the headline is the C-weighted step."""
    for steps, warmup in ((20, 5), (64, 16), (1, 0), (640, 64), (33, 100)):
        for R, C in ((8, 4), (12, 1), (2, 4)):
            replays, warm = bench.timing_plan(steps, warmup, R, C)
            assert replays >= bench.MIN_REPLAYS and replays * R * C >= steps
            assert warm >= 1 and (warm + 1) * R * C >= warmup
            timed_select = replays * R                    # the first step of each cycle selects
            assert timed_select * C == replays * R * C
    # 20 / 5 and 64 / 16 time the same work at the benchmark shape
    assert bench.timing_plan(20, 5, 8, 4)[0] == bench.timing_plan(64, 16, 8, 4)[0] == 20


def test_ring_write_bytes_at_128k():
    """Ring storage: a streaming head's prompt write keeps the sink's page
    (tokens 0-63) and the last ceil(2048 / 64) + 1 = 33 physical pages of the
    131071-token prompt (pages 2015-2047: tokens 128960-131070); the dynamic
    heads write every token."""
    wl = W.WORKLOADS["llama3_128k"]
    count = 131071
    kept = 64 + (count - 2015 * 64)
    assert kept == 2175
    rows = 2 * (4 * count + 4 * kept) * 2 * ROW
    assert bench.bulk_write_bytes(wl, count, ring=True) == rows + 4 * 8192 * 2 * ROW + 2048 * 4
    # a prompt shorter than sink + window is kept whole
    assert bench.bulk_write_bytes(wl, 2000, ring=True) == bench.bulk_write_bytes(wl, 2000)
    assert bench.bulk_write_bytes(wl, 0, ring=True) == 0
