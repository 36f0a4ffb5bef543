"""Summaries of rocprofv3 result databases for this library's kernels.

    python -m sparse_paged_attention_amd.profiling stats <results.db>
        per-kernel count / average / median / min / max duration (us) from a
        --kernel-trace (--stats) run;
    python -m sparse_paged_attention_amd.profiling pmc <results.db>
        per-kernel average of every collected counter, summed over the
        counter's hardware instances for each dispatch;
    python -m sparse_paged_attention_amd.profiling traffic <fetch.db> <write.db> <kernels> <copy_bytes>
        HBM bytes per launch of the |-separated <kernels> (name parts, each
        matching one kernel; together one call of the
        entry point that launches them, summed) from a FETCH_SIZE run and a
        WRITE_SIZE run, each scaled by what the same counter reads for the
        plain copy kernel of <copy_bytes> bytes (the largest copy dispatch) in
        that run; the JSON carries the hash of the sources of those kernels
        it was taken on.

rocprofv3 writes SQLite databases; only the standard `kernels` and
`pmc_events` views are read.
"""
from __future__ import annotations

import collections
import hashlib
import json
import os
import sqlite3
import statistics
import sys


_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").split("(")[0].strip()


def kernel_stats(db_path: str) -> list:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, duration from kernels order by start").fetchall()
    agg = collections.OrderedDict()
    for name, dur in rows:
        agg.setdefault(_short(name), []).append(dur / 1e3)
    out = []
    for k, ds in agg.items():
        out.append(dict(kernel=k, n=len(ds), avg_us=sum(ds) / len(ds), med_us=statistics.median(ds),
                        min_us=min(ds), max_us=max(ds)))
    return out


def pmc_per_dispatch(db_path: str) -> dict:
    """{kernel: {counter: [value per dispatch]}} (instances summed)."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall()
    per = collections.defaultdict(float)
    names = {}
    for name, disp, ctr, val in rows:
        per[(disp, ctr)] += val
        names[disp] = _short(name)
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (disp, ctr), v in per.items():
        out[names[disp]][ctr].append(v)
    return out


# Sources each kernel is built from (name part -> files).
_KERNEL_SOURCES = (
    (("attn_kernel", "combine_kernel"), ("attn.hip", "pool_rows.h", "psplit.h", "spa_internal.h")),
    (("write_kernel", "summary_kernel", "append_kernel"), ("pool.hip", "pool_rows.h", "spa_internal.h")),
    (("score_kernel", "topk_kernel"), ("select.hip", "pool_rows.h", "spa_internal.h")),
)


def source_hash(kernels: str) -> str:
    """Hash of the sources the |-separated kernels are built from; a stored
    traffic figure is only valid for the kernels it was measured on."""
    files = []
    for part in kernels.split("|"):
        for names, srcs in _KERNEL_SOURCES:
            if any(n in part for n in names):
                files.extend(f for f in srcs if f not in files)
                break
        else:
            raise ValueError(f"no sources known for kernel '{part}'")
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(fetch_db: str, write_db: str, kernels: str, copy_bytes: float) -> dict:
    f = pmc_per_dispatch(fetch_db)
    w = pmc_per_dispatch(write_db)
    copy = [k for k in f if "copy" in k.lower() and "FETCH_SIZE" in f[k]]
    if not copy:
        raise SystemExit("no copy kernel in the FETCH_SIZE run")
    ck = max(copy, key=lambda k: max(f[k]["FETCH_SIZE"]))
    f_copy = max(f[ck]["FETCH_SIZE"]) * 1024.0
    w_copy = max(w[ck]["WRITE_SIZE"]) * 1024.0
    f_scale = copy_bytes / f_copy
    w_scale = copy_bytes / w_copy
    per = {}
    for part in kernels.split("|"):
        match = [k for k in f if part in k]
        if len(match) != 1:
            raise SystemExit(f"'{part}' names {len(match)} kernels in the FETCH_SIZE run: {match}")
        kernel = match[0]
        fk = [v * 1024.0 * f_scale for v in f[kernel]["FETCH_SIZE"]]
        wk = [v * 1024.0 * w_scale for v in w[kernel]["WRITE_SIZE"]]
        per[kernel] = dict(launches=len(fk), fetch_bytes=sum(fk) / len(fk), write_bytes=sum(wk) / len(wk))
    fetch = sum(v["fetch_bytes"] for v in per.values())
    write = sum(v["write_bytes"] for v in per.values())
    return dict(kernels=per, fetch_bytes_per_launch=fetch, write_bytes_per_launch=write,
                bytes_per_launch=fetch + write, fetch_scale=f_scale, write_scale=w_scale,
                copy_kernel=ck, copy_bytes=copy_bytes, kernel_source_hash=source_hash(kernels))


def _print_stats(db: str) -> None:
    print(f"{'kernel':70s} {'n':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for r in kernel_stats(db):
        print(f"{r['kernel'][-70:]:70s} {r['n']:6d} {r['avg_us']:9.2f} {r['med_us']:9.2f} "
              f"{r['min_us']:9.2f} {r['max_us']:9.2f}")


def main(argv) -> int:
    if len(argv) >= 2 and argv[0] == "stats":
        _print_stats(argv[1])
    elif len(argv) >= 2 and argv[0] == "pmc":
        for k, cs in pmc_per_dispatch(argv[1]).items():
            print(k)
            for c, vs in sorted(cs.items()):
                print(f"    {c:28s} avg {sum(vs) / len(vs):16.1f}  dispatches={len(vs)}")
    elif len(argv) >= 5 and argv[0] == "traffic":
        print(json.dumps(traffic(argv[1], argv[2], argv[3], float(argv[4])), indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
