#!/usr/bin/env python3
"""Turn two rocprofv3 counter runs of the bench into HBM-traffic summaries.

Usage (R = the repository root, P = a scratch folder for the raw counter
databases, after `cd /tmp && export TMPDIR=/tmp`):
  rocprofv3 --pmc FETCH_SIZE -d $P/FETCH_SIZE -o run -- \\
      python3 $R/bench.py --steps 20 --warmup 5 --no-detail --no-cpu-baseline --copy-calibration-mib 256
  rocprofv3 --pmc WRITE_SIZE -d $P/WRITE_SIZE -o run -- (same command)
  python3 $R/profile_traffic.py $P/FETCH_SIZE/run_results.db $P/WRITE_SIZE/run_results.db

Each counter (KiB per dispatch) is scaled by what it reads for the bench's
plain device-to-device copy of 256 MiB (bytes read and written are known), so
the figures are HBM bytes.  Writes profiles/gemv_hbm_traffic.md and
profiles/gemv_hbm_traffic.json; the JSON carries a hash of the kernel sources
(comments and blank lines left out) so the bench reports the traffic only
while the kernels are unchanged.
"""
import json
import os
import re
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
from bench import kernel_source_hash  # noqa: E402  (one definition of the hash)
CSRC = os.path.join(ROOT, "dequant_matmul_packed_amd", "csrc")
COPY_MIB = 256
CODES = {1: "HYB", 2: "1MAD", 3: "3INST", 4: "NUQ", 5: "VQ"}


def per_kernel(db_path):
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, grid_size, count(*), avg(value) from counters_collection "
                      "group by kernel_name, grid_size").fetchall()
    return {(r[0].split("(")[0].replace("void ", ""), r[1]): (r[2], r[3]) for r in rows}


def main():
    fetch = per_kernel(sys.argv[1])
    write = per_kernel(sys.argv[2])
    copy_bytes = COPY_MIB << 20
    # the copy kernel: the dispatch whose WRITE_SIZE is the copy size
    ck = max(write, key=lambda k: write[k][1])
    f_scale = copy_bytes / (fetch[ck][1] * 1024)
    w_scale = copy_bytes / (write[ck][1] * 1024)
    finish = [k for k in fetch if k[0].startswith("qdec::gemv_finish_kernel")]
    fin_f = sum(fetch[k][1] for k in finish) / max(len(finish), 1) * 1024 * f_scale
    fin_w = sum(write[k][1] for k in finish) / max(len(finish), 1) * 1024 * w_scale
    out = {"kernel_source_hash": kernel_source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
           "calibration": "device-to-device copy of %d MiB (%s)" % (COPY_MIB, ck[0]), "variants": {}}
    lines = ["# HBM traffic of the fused GEMV (bench workload, 4096x4096, b=1)", "",
             "Counters: `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch), one rocprofv3 --pmc run each, of",
             "`python3 $R/bench.py --steps 20 --warmup 5 --no-detail --no-cpu-baseline --copy-calibration-mib 256`,",
             "summarised by `python3 profile_traffic.py <FETCH db> <WRITE db>`.", "",
             "Calibration: the plain %d MiB copy reads FETCH %.0f KiB and WRITE %.0f KiB per dispatch, so the" % (
                 COPY_MIB, fetch[ck][1], write[ck][1]),
             "counters are scaled by %.3f (reads) and %.3f (writes) to give HBM bytes." % (f_scale, w_scale), "",
             "| variant | codes MiB | decode kernel read MiB | decode kernel write KiB | finish kernel read+write KiB | total / algorithmic |",
             "|---|---|---|---|---|---|"]
    for k in sorted(fetch):
        if not k[0].startswith("qdec::gemv_kernel<"):
            continue
        # template arguments: code, k, batch columns, code-ring depth, small loads
        code, kk, nb = (int(v) for v in k[0][len("qdec::gemv_kernel<"):-1].split(",")[:3])
        fb = fetch[k][1] * 1024 * f_scale
        wb = write.get(k, (0, 0.0))[1] * 1024 * w_scale
        m = n = 4096
        codes = m * n * kk // 8
        algo = codes + 2 * (m + n) + (m + n) // 8
        total = fb + wb + fin_f + fin_w
        name = "%s_k%d" % (CODES[code], kk)
        out["variants"][name] = {"bytes_per_call": total, "decode_read": fb, "decode_write": wb,
                                 "finish_read": fin_f, "finish_write": fin_w, "algorithmic": algo}
        lines.append("| %s | %.2f | %.3f | %.1f | %.1f | %.3f |" % (
            name, codes / 2 ** 20, fb / 2 ** 20, wb / 1024, (fin_f + fin_w) / 1024, total / algo))
    lines += ["", "The decode kernel's writes are its split-K fp32 atomic adds (each reaches HBM as its own",
              "4-byte write); the reads are the packed codes plus x, signs and the tables.",
              "Kernel source hash (comments and blank lines left out): `%s`." % out["kernel_source_hash"]]
    with open(os.path.join(ROOT, "profiles", "gemv_hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", "gemv_hbm_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
