#!/usr/bin/env python3
"""Summarise a rocprofv3 --kernel-trace database: per kernel, grid and LDS
size, the dispatch count and the average / median / minimum duration.

Usage (R = the repository root, after `cd /tmp && export TMPDIR=/tmp`):
  rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 $R/bench.py ARGS
  python3 $R/profile_trace.py <dir>/run_results.db "ARGS" > OUT.md

Dispatches are kept apart by grid and LDS size as well as by name, so that
the calls of the bench that run one kernel template with different shapes
(the MFMA GEMV of gate+up and of down, say) get rows of their own.

A second table follows the calls the bench makes: a one-column GEMV call
(an MFMA GEMV dispatch and the finisher dispatch after it) and a b = 64 GEMM
call (input transform, GEMM, output transform), with the average span from
the first dispatch's start to the last one's end beside the sum of the
dispatches' durations.  Under the tracer the dispatches of a call leave gaps
between them, so the span exceeds the sum; both exceed the same call timed
by HIP events without the tracer.
"""
import re
import sqlite3
import statistics
import sys


def short(name):
    return re.sub(r"^void ", "", name).split("(")[0]


def call_spans(db):
    """Average span of the bench's calls, keyed by their first dispatch."""
    try:
        rows = db.execute("select name, grid_x, workgroup_x, lds_size, start, end from kernels "
                          "order by start").fetchall()
    except sqlite3.OperationalError:
        return {}
    spans = {}
    i = 0
    while i < len(rows):
        nm = short(rows[i][0])
        key = (nm, rows[i][1] // max(rows[i][2], 1), rows[i][3])
        if nm.startswith("qdec::gemv_mma") and i + 1 < len(rows) and \
                short(rows[i + 1][0]).startswith("qdec::gemv_finish"):
            last, n = i + 1, 2
        elif nm.startswith("qdec::rht_split_kernel") and i + 2 < len(rows) and \
                short(rows[i + 1][0]).startswith("qdec::gemm_kernel") and \
                short(rows[i + 2][0]).startswith("qdec::rht_"):
            last, n = i + 2, 3
        else:
            i += 1
            continue
        span = (rows[last][5] - rows[i][4]) / 1000.0
        durs = sum((rows[j][5] - rows[j][4]) for j in range(i, last + 1)) / 1000.0
        spans.setdefault(key, (n, []))[1].append((span, durs))
        i = last + 1
    return spans


def main():
    db = sqlite3.connect(sys.argv[1])
    args = sys.argv[2] if len(sys.argv) > 2 else ""
    rows = db.execute("select name, grid_x, workgroup_x, lds_size, duration from kernels").fetchall()
    groups = {}
    for name, gx, wx, lds, du in rows:
        key = (re.sub(r"^void ", "", name).split("(")[0], gx // max(wx, 1), wx, lds)
        groups.setdefault(key, []).append(du / 1000.0)
    print("# Kernel durations: `bench.py %s`" % args)
    print()
    print("Command: `rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 $R/bench.py %s`, summarised by "
          "`python3 profile_trace.py <dir>/run_results.db \"%s\"`.  Durations in us, per dispatch; rows by kernel, "
          "grid (workgroups), workgroup size and LDS bytes; kernels of the library first, by total time." % (args, args))
    print()
    print("| kernel | workgroups | threads | LDS bytes | dispatches | avg us | median us | min us |")
    print("|---|---|---|---|---|---|---|---|")
    order = sorted(groups.items(), key=lambda kv: (not kv[0][0].startswith("qdec::"), -sum(kv[1])))
    for (nm, wgs, wx, lds), d in order:
        if not nm.startswith("qdec::") and len(d) < 8:
            continue                                   # set-up kernels of the bench (torch fills, copies)
        print("| `%s` | %d | %d | %d | %d | %.2f | %.2f | %.2f |" % (
            nm[:90], wgs, wx, lds, len(d), sum(d) / len(d), statistics.median(d), min(d)))
    spans = call_spans(db)
    if spans:
        print()
        print("Calls (consecutive dispatches from the first one's start to the last one's end; the first "
              "dispatch's kernel, workgroups and LDS bytes name the call):")
        print()
        print("| first kernel | workgroups | LDS bytes | dispatches per call | calls | avg span us | "
              "avg sum of durations us |")
        print("|---|---|---|---|---|---|---|")
        for (nm, wgs, lds), (n, v) in sorted(spans.items(), key=lambda kv: -len(kv[1][1])):
            print("| `%s` | %d | %d | %d | %d | %.2f | %.2f |" % (
                nm[:90], wgs, lds, n, len(v), sum(a for a, b in v) / len(v), sum(b for a, b in v) / len(v)))


if __name__ == "__main__":
    main()
