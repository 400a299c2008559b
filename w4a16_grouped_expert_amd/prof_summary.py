"""Summaries of rocprofv3 result databases (the SQLite files rocprofv3 writes).

    python -m w4a16_grouped_expert_amd.prof_summary stats <results.db> [name-filter]
        per kernel: dispatches, average / min / max duration in microseconds
    python -m w4a16_grouped_expert_amd.prof_summary pmc <results.db> [name-filter]
        per kernel: dispatches and the average value of each counter per dispatch

The filter is a substring of the kernel name.  Output is plain text, one kernel
per line, longest total time first.
"""
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


def main(argv):
    if len(argv) < 3 or argv[1] not in ("stats", "pmc"):
        print(__doc__)
        return 2
    filt = argv[3] if len(argv) > 3 else ""
    print(stats(argv[2], filt) if argv[1] == "stats" else pmc(argv[2], filt))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
