"""Summaries of rocprofv3 output (rocpd SQLite databases) for the profiles/
folder: kernel-trace statistics and HBM traffic from the FETCH_SIZE /
WRITE_SIZE counters, scaled by what the same counters read for a plain copy
of known size.

    python -m mla_latent_kv_15_amd.profsum trace DB
    python -m mla_latent_kv_15_amd.profsum counters --kernel attn_v2_kernel DB [DB ...]
    python -m mla_latent_kv_15_amd.profsum traffic --kernel attn_v2_kernel \\
        --fetch DB --write DB --copy-fetch DB --copy-write DB --copy-bytes N

The traffic summary records the SHA-256 of the kernel sources it was taken
on; bench.py reports the figure only while those sources are unchanged.
"""
from __future__ import annotations

import argparse
import hashlib
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
# sources whose change invalidates a traffic measurement of the attention path
TRAFFIC_SOURCES = ("csrc/k_attn_v2.hip", "csrc/k_plan.hip", "csrc/plan_device.h")


def sources_digest() -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)", "anon")
    return re.sub(r"\(.*", "", name)


def kernel_rows(db: str):
    """(name, wgs, calls, avg_us, min_us, max_us, total_us) grouped by kernel and grid."""
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute(
        "select name, grid_x / workgroup_x, grid_y, grid_z, count(*), avg(duration), "
        "min(duration), max(duration), sum(duration) from kernels "
        "group by name, grid_x, grid_y, grid_z order by sum(duration) desc").fetchall()
    return [(_short(r[0]), (r[1], r[2], r[3]), r[4], r[5] / 1e3, r[6] / 1e3, r[7] / 1e3,
             r[8] / 1e3) for r in rows]


def trace_table(db: str) -> str:
    rows = kernel_rows(db)
    tot = sum(r[6] for r in rows) or 1.0
    out = [f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6} {'wgs(x,y,z)':>16}  kernel"]
    for name, wgs, n, avg, mn, mx, s in rows:
        out.append(f"{n:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} {100 * s / tot:6.1f} {str(wgs):>16}  {name[:90]}")
    return "\n".join(out)


def counter_mean(db: str, counter: str, kernel: str) -> tuple[float, int]:
    """Mean per dispatch of a counter (summed over its instances) for kernels
    whose name contains `kernel`; and the number of dispatches."""
    cur = sqlite3.connect(db).cursor()
    cols = [d[0] for d in cur.execute("select * from counters_collection limit 1").description]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    disp_col = "dispatch_id" if "dispatch_id" in cols else None
    q = f"select {name_col}, value" + (f", {disp_col}" if disp_col else "") + \
        " from counters_collection where counter_name = ?"
    per = {}
    for r in cur.execute(q, (counter,)).fetchall():
        if kernel not in r[0]:
            continue
        key = r[2] if disp_col else len(per)
        per[key] = per.get(key, 0.0) + r[1]
    if not per:
        raise SystemExit(f"no {counter} rows for a kernel matching {kernel!r} in {db}")
    return sum(per.values()) / len(per), len(per)


def counter_names(db: str) -> list:
    cur = sqlite3.connect(db).cursor()
    return sorted(r[0] for r in cur.execute(
        "select distinct counter_name from counters_collection").fetchall())


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    k = sub.add_parser("counters")
    k.add_argument("--kernel", required=True)
    k.add_argument("dbs", nargs="+")
    f = sub.add_parser("traffic")
    f.add_argument("--kernel", required=True)
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--copy-fetch", required=True)
    f.add_argument("--copy-write", required=True)
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--copy-kernel", default="copyBuffer")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_table(a.db))
        return
    if a.cmd == "counters":
        print(f"kernel: {a.kernel} (mean per dispatch, summed over counter instances)")
        for db in a.dbs:
            for c in counter_names(db):
                v, n = counter_mean(db, c, a.kernel)
                print(f"{c:32s} {v:18.1f}   ({n} dispatches)")
        return
    # FETCH_SIZE / WRITE_SIZE are in KiB per dispatch
    fk, nf = counter_mean(a.fetch, "FETCH_SIZE", a.kernel)
    wk, nw = counter_mean(a.write, "WRITE_SIZE", a.kernel)
    cfk, _ = counter_mean(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cwk, _ = counter_mean(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_scale = a.copy_bytes / (cfk * 1024.0)
    w_scale = a.copy_bytes / (cwk * 1024.0)
    fetch_b = fk * 1024.0 * f_scale
    write_b = wk * 1024.0 * w_scale
    print(f"kernel: {a.kernel}")
    print(f"dispatches: fetch pass {nf}, write pass {nw}")
    print(f"FETCH_SIZE_KiB_per_dispatch: {fk:.1f}")
    print(f"WRITE_SIZE_KiB_per_dispatch: {wk:.1f}")
    print(f"copy_bytes: {a.copy_bytes}")
    print(f"copy_FETCH_SIZE_KiB: {cfk:.1f}")
    print(f"copy_WRITE_SIZE_KiB: {cwk:.1f}")
    print(f"fetch_scale: {f_scale:.4f}")
    print(f"write_scale: {w_scale:.4f}")
    print(f"fetch_bytes_per_launch: {fetch_b:.0f}")
    print(f"write_bytes_per_launch: {write_b:.0f}")
    print(f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}")
    print(f"sources_sha256: {sources_digest()}")


if __name__ == "__main__":
    main(sys.argv[1:])
