#!/usr/bin/env python3
"""Turn rocprofv3 counter runs of the headline's calls into HBM-traffic
summaries.

Usage (R = the repository root, P = a scratch folder for the raw counter
databases, after `cd /tmp && export TMPDIR=/tmp`), for each call C of
qkv, o, gate_up, down (the calls of one Llama-3-8B-shaped layer at b = 1) and
gemm (the 28672x8192 b = 64 product):
  rocprofv3 --pmc FETCH_SIZE -d $P/fetch_C -o run -- \\
      python3 $R/bench.py --call C --copy-calibration-mib 256
  rocprofv3 --pmc WRITE_SIZE -d $P/write_C -o run -- (same command)
then
  python3 $R/profile_traffic.py $P

Each run holds 8 calls and 5 plain device-to-device copies of 256 MiB.  Each
counter (KiB per dispatch) is scaled by what it reads for that copy (bytes
read and written are known), so the figures are HBM bytes; a call's bytes
are the sums over its kernels (one dispatch each per call).  Writes
profiles/traffic.md and profiles/traffic.json; the JSON carries a hash of
the kernel sources (comments and blank lines left out) so the bench reports
the traffic only while the kernels are unchanged.
"""
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
from bench import kernel_source_hash  # noqa: E402  (one definition of the hash)

COPY_MIB = 256
CALLS = ["qkv", "o", "gate_up", "down", "gemm"]
WHAT = {"qkv": "q, k, v (4096x4096, 1024x4096, 1024x4096), grouped, b=1",
        "o": "o (4096x4096), b=1",
        "gate_up": "gate, up (14336x4096 each), grouped, b=1",
        "down": "down (4096x14336), b=1",
        "gemm": "28672x8192 k=3, b=64"}


def per_kernel(db_path):
    """(kernel, grid, LDS) -> (dispatches, average counter value)."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, grid_size, lds_block_size, count(*), avg(value) "
                      "from counters_collection group by kernel_name, grid_size, lds_block_size").fetchall()
    return {(r[0].split("(")[0].replace("void ", ""), r[1], r[2]): (r[3], r[4]) for r in rows}


def main():
    P = sys.argv[1]
    out = {"kernel_source_hash": kernel_source_hash(), "calibration": "device-to-device copy of %d MiB" % COPY_MIB,
           "calls": {}}
    lines = ["# HBM traffic of the headline's calls", "",
             "Counters: `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch), one rocprofv3 `--pmc` run each per call,",
             "of `python3 $R/bench.py --call C --copy-calibration-mib 256` (8 calls, then 5 copies of 256 MiB),",
             "summarised by `python3 profile_traffic.py <folder of the runs>`.  Each counter is scaled by what it",
             "reads for the plain copy (bytes known), so the figures are HBM bytes per call.", "",
             "| call | kernels (dispatches per call) | read MB | written MB | scale read / write |",
             "|---|---|---|---|---|"]
    for c in CALLS:
        fp, wp = (os.path.join(P, "%s_%s" % (k, c), "run_results.db") for k in ("fetch", "write"))
        if not (os.path.exists(fp) and os.path.exists(wp)):
            continue
        fetch, write = per_kernel(fp), per_kernel(wp)
        # the copy: the blit kernel, else the kernel whose writes come
        # closest to its size (the largest write can be the code pool's
        # random fill, which writes 1 GiB and reads nothing)
        copies = [k for k in write if "copyBuffer" in k[0]]
        ck = (max(copies, key=lambda k: write[k][1]) if copies
              else min(write, key=lambda k: abs(write[k][1] - (COPY_MIB << 10))))
        f_scale = (COPY_MIB << 20) / (fetch[ck][1] * 1024)
        w_scale = (COPY_MIB << 20) / (write[ck][1] * 1024)
        ks = [k for k in fetch if k[0].startswith("qdec::") and k in write]
        rd = sum(fetch[k][1] * fetch[k][0] / 8 for k in ks) * 1024 * f_scale
        wr = sum(write[k][1] * write[k][0] / 8 for k in ks) * 1024 * w_scale
        out["calls"][c] = {"what": WHAT[c], "read_bytes": rd, "write_bytes": wr, "bytes_per_call": rd + wr,
                           "kernels": {"%s grid %d lds %d" % k: {"dispatches_per_call": fetch[k][0] / 8,
                                                                 "read_bytes": fetch[k][1] * 1024 * f_scale,
                                                                 "write_bytes": write[k][1] * 1024 * w_scale}
                                       for k in ks}}
        lines.append("| %s: %s | %s | %.3f | %.3f | %.3f / %.3f |" % (
            c, WHAT[c], ", ".join("`%s` (%g)" % (k[0], fetch[k][0] / 8) for k in sorted(ks)),
            rd / 1e6, wr / 1e6, f_scale, w_scale))
    lines += ["", "bench.py divides these bytes by the call's algorithmic bytes (codes, x and y in fp16, the",
              "sign vectors and the table) in the roofline entries' `traffic_detail`.",
              "Kernel source hash (comments and blank lines left out): `%s`." % out["kernel_source_hash"]]
    with open(os.path.join(ROOT, "profiles", "traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
