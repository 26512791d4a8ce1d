#!/usr/bin/env python3
"""Summarise two rocprofv3 --pmc runs (SQ counters, eight per run) of the
bench, or of one layer of it, into a markdown table under profiles/.

Usage (from the repository root R, after `cd /tmp && export TMPDIR=/tmp`):
  rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU \\
      SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_VALU_MFMA_BUSY_CYCLES -d <dir1> -o run -- python3 $R/bench.py ARGS
  rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS \\
      SQ_ACTIVE_INST_ANY SQ_INSTS_SALU SQ_LDS_ADDR_CONFLICT -d <dir2> -o run -- python3 $R/bench.py ARGS
  rocprofv3 --pmc MfmaUtil -d <dir3> -o run -- python3 $R/bench.py ARGS      (optional third pass)
  python3 profile_counters.py <dir1>/run_results.db <dir2>/run_results.db OUT.md "ARGS" [WEIGHTS [<dir3>/run_results.db]]

ARGS is the bench's argument string (it goes into the summary's command
line): `--steps 20 --warmup 5 --no-cpu-baseline` for the bench, or
`--layer CODE:M:N:K:B` for one layer.  With WEIGHTS (the layer's m x n) the
table gives VALU and LDS lane-instructions per weight for the layer's
decode kernel (the gemv_kernel, gemv_mma_kernel, gemv_mma1_kernel, gemv_mma1r_kernel, gemv_mma2_kernel,
gemv_mma3_kernel or gemm_kernel dispatches).
Rows are kept apart by kernel, grid and LDS size; every qdec kernel gets a
row.

Counters are per dispatch, summed over the chip; instruction counts are per
wave (64 lanes).  With the third pass the table adds MfmaUtil, rocprofv3's
derived MFMA utilisation: MFMA-busy cycles summed over the SIMDs over
(GPU-active cycles x SIMD count), in percent.
"""
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE = ("qdec::gemv_kernel<", "qdec::gemv_mma_kernel<", "qdec::gemv_mma1_kernel<", "qdec::gemv_mma1r_kernel<",
          "qdec::gemv_mma2_kernel<", "qdec::gemv_mma3_kernel<", "qdec::gemm_kernel<")


def load(db):
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, grid_size, lds_block_size, counter_name, avg(value), count(*) "
                     "from counters_collection group by kernel_name, grid_size, lds_block_size, "
                     "counter_name").fetchall()
    out = {}
    for kn, gs, lds, cn, v, n in rows:
        k = (kn.split("(")[0].replace("void ", ""), gs, lds)
        out.setdefault(k, {})[cn] = (v, n)
    return out


def main():
    a, b = load(sys.argv[1]), load(sys.argv[2])
    out = sys.argv[3]
    bench_args = sys.argv[4]
    weights = int(sys.argv[5]) if len(sys.argv) > 5 else 0
    c = load(sys.argv[6]) if len(sys.argv) > 6 else None
    keys = [k for k in a if k in b and k[0].startswith("qdec::")]
    keys.sort(key=lambda k: -a[k].get("SQ_WAVE_CYCLES", (0, 0))[0] * a[k].get("SQ_WAVE_CYCLES", (0, 1))[1])
    title = "the bench's kernels" if not weights else "one layer (`%s`)" % bench_args
    lines = ["# SQ counters of %s" % title, "",
             "Commands: %s `rocprofv3 --pmc` runs of `python3 $R/bench.py %s`, eight SQ counters in each "
             "of the first two%s (the lists are in `profile_counters.py`), summarised by `python3 "
             "profile_counters.py <pass 1 db> <pass 2 db> %s \"%s\"%s%s`." % (
                 "three" if c else "two", bench_args, ", MfmaUtil in the third" if c else "",
                 os.path.relpath(out, ROOT), bench_args, (" %d" % weights) if weights else "",
                 " <pass 3 db>" if c else ""), "",
             "Per dispatch, averaged over dispatches.  wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave time "
             "waiting on a dependency); LDS wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; bank = "
             "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (conflict cycles per LDS issue cycle).", "",
             "| kernel | grid | LDS bytes | dispatches | VALU inst | LDS inst | MFMA inst | wait | LDS wait | bank | "
             "VALU/weight | LDS/weight |%s" % (" MfmaUtil % |" if c else ""),
             "|---|---|---|---|---|---|---|---|---|---|---|---|%s" % ("---|" if c else "")]
    for k in keys:
        d = dict(a[k])
        d.update(b[k])
        g = lambda c: d.get(c, (0.0, 0))[0]
        wc = g("SQ_WAVE_CYCLES") or 1.0
        wts = weights if weights and k[0].startswith(DECODE) else None
        vpw = "%.3f" % (g("SQ_INSTS_VALU") * 64 / wts) if wts else ""
        lpw = "%.3f" % (g("SQ_INSTS_LDS") * 64 / wts) if wts else ""
        util = ""
        if c:
            util = " %.1f |" % c[k]["MfmaUtil"][0] if k in c and "MfmaUtil" in c[k] else " |"
        lines.append("| `%s` | %d | %d | %d | %.0f | %.0f | %.0f | %.2f | %.2f | %.2f | %s | %s |%s" % (
            k[0], k[1], k[2], d.get("SQ_INSTS_VALU", (0, 0))[1], g("SQ_INSTS_VALU"), g("SQ_INSTS_LDS"),
            g("SQ_INSTS_MFMA"), g("SQ_WAIT_INST_ANY") / wc, g("SQ_WAIT_INST_LDS") / wc,
            g("SQ_LDS_BANK_CONFLICT") / (g("SQ_ACTIVE_INST_LDS") or 1.0), vpw, lpw, util))
    lines += ["", "VALU/weight and LDS/weight are lane-instructions per weight (wave instructions x 64 / "
              "weights) of the decode kernels: gemv_kernel counts the decode and the dot products (v_dot2, "
              "one per two weights); gemv_mma_kernel and gemm_kernel count the decode only (the products "
              "are MFMA instructions).  The decode kernels also carry their start-up work (the input "
              "Hadamard transform and the table fill)."]
    if c:
        lines += ["", "MfmaUtil is rocprofv3's derived counter: the MFMA-busy cycles of all SIMDs over the "
                  "GPU-active cycles of the dispatch times the SIMD count (1024), in percent."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
