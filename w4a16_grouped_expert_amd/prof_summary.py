"""Summaries of rocprofv3 result databases (the SQLite files rocprofv3 writes).

    python -m w4a16_grouped_expert_amd.prof_summary stats <results.db> [name-filter]
        per kernel: dispatches, average / min / max duration in microseconds
    python -m w4a16_grouped_expert_amd.prof_summary pmc <results.db> [name-filter]
        per kernel: dispatches and the average value of each counter per dispatch

    python -m w4a16_grouped_expert_amd.prof_summary traffic <fetch.db> <write.db> <copy_fetch.db> \
            <copy_write.db> <kernel-filter> <source> [<source> ...]
        HBM bytes per dispatch of the kernel matching the filter: FETCH_SIZE and
        WRITE_SIZE (KiB per dispatch) each scaled by what the same counter reads
        for a plain device copy of known size (the bench's --copy-calibration run,
        1 GiB), plus the sha256 of the listed kernel sources (the bench uses the
        figure only while that hash matches).

The filter is a substring of the kernel name.  Output is plain text, one kernel
per line, longest total time first.
"""
import hashlib
import os
import sqlite3
import sys
from collections import defaultdict


def _views(c):
    return {r[0] for r in c.execute("select name from sqlite_master where type in ('view', 'table')")}


def stats(db, filt=""):
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                     "from kernels group by name order by sum(duration) desc").fetchall()
    out = []
    for name, n, avg, mn, mx, tot in rows:
        if filt and filt not in name:
            continue
        out.append(f"{name[:100]:100s} dispatches {n:6d} avg_us {avg / 1e3:10.3f} min_us {mn / 1e3:10.3f} "
                   f"max_us {mx / 1e3:10.3f} total_ms {tot / 1e6:10.3f}")
    return "\n".join(out)


def pmc(db, filt=""):
    c = sqlite3.connect(db)
    cols = [r[1] for r in c.execute("pragma table_info(counters_collection)")]
    ix = {n: i for i, n in enumerate(cols)}
    name_col = "kernel_name" if "kernel_name" in ix else "name"
    agg = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    for r in c.execute("select * from counters_collection"):
        name = r[ix[name_col]]
        if filt and filt not in name:
            continue
        agg[name][r[ix["counter_name"]]] += r[ix["value"]]
        disp[name].add(r[ix["dispatch_id"]] if "dispatch_id" in ix else 0)
    out = []
    for name in sorted(agg, key=lambda k: -len(disp[k])):
        n = len(disp[name])
        vals = " ".join(f"{k}={v / n:.1f}" for k, v in sorted(agg[name].items()))
        out.append(f"{name[:100]:100s} dispatches {n:6d} per_dispatch {vals}")
    return "\n".join(out)


def _counter_per_dispatch(db, counter, filt):
    """(kernel name, average value per dispatch) of the kernel matching filt."""
    c = sqlite3.connect(db)
    cols = [r[1] for r in c.execute("pragma table_info(counters_collection)")]
    ix = {n: i for i, n in enumerate(cols)}
    name_col = "kernel_name" if "kernel_name" in ix else "name"
    tot, disp, names = 0.0, set(), set()
    for r in c.execute("select * from counters_collection"):
        name = r[ix[name_col]]
        if filt not in name or r[ix["counter_name"]] != counter:
            continue
        tot += r[ix["value"]]
        disp.add(r[ix["dispatch_id"]] if "dispatch_id" in ix else 0)
        names.add(name)
    if len(names) != 1 or not disp:
        raise SystemExit(f"filter {filt!r} matches {sorted(names)} in {db}")
    return names.pop(), tot / len(disp)


COPY_BYTES = 1 << 30  # bench.py --copy-calibration copies this many bytes per launch


def traffic(fetch_db, write_db, cfetch_db, cwrite_db, filt, sources):
    name, fetch = _counter_per_dispatch(fetch_db, "FETCH_SIZE", filt)
    _, write = _counter_per_dispatch(write_db, "WRITE_SIZE", filt)
    _, cfetch = _counter_per_dispatch(cfetch_db, "FETCH_SIZE", "copyBuffer")
    _, cwrite = _counter_per_dispatch(cwrite_db, "WRITE_SIZE", "copyBuffer")
    fs, wsc = COPY_BYTES / 1024.0 / cfetch, COPY_BYTES / 1024.0 / cwrite
    h = hashlib.sha256()
    for f in sources:
        h.update(open(f, "rb").read())
    return "\n".join([
        f"# kernel sources hashed (sha256 over, in order): {' '.join(sources)}",
        f"source_sha256 = {h.hexdigest()}",
        f"kernel = {name}",
        f"fetch_kib_per_dispatch = {fetch:.1f}",
        f"write_kib_per_dispatch = {write:.1f}",
        f"copy_bytes = {COPY_BYTES}",
        f"copy_fetch_kib = {cfetch:.1f}",
        f"copy_write_kib = {cwrite:.1f}",
        f"fetch_scale = {fs:.4f}",
        f"write_scale = {wsc:.4f}",
        f"traffic_bytes_per_launch = {int(round((fetch * fs + write * wsc) * 1024))}",
    ])


def main(argv):
    if len(argv) >= 8 and argv[1] == "traffic":
        print(traffic(argv[2], argv[3], argv[4], argv[5], argv[6], argv[7:]))
        return 0
    if len(argv) < 3 or argv[1] not in ("stats", "pmc"):
        print(__doc__)
        return 2
    filt = argv[3] if len(argv) > 3 else ""
    print(stats(argv[2], filt) if argv[1] == "stats" else pmc(argv[2], filt))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
