#!/usr/bin/env python3
"""Summarise a rocprofv3 --kernel-trace database: per kernel, grid and LDS
size, the dispatch count and the average / median / minimum duration.

Usage (R = the repository root, after `cd /tmp && export TMPDIR=/tmp`):
  rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 $R/bench.py ARGS
  python3 $R/profile_trace.py <dir>/run_results.db "ARGS" > OUT.md

Dispatches are kept apart by grid and LDS size as well as by name, so that
the calls of the bench that run one kernel template with different shapes
(the MFMA GEMV of gate+up and of down, say) get rows of their own.
"""
import re
import sqlite3
import statistics
import sys


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


if __name__ == "__main__":
    main()
