"""Summaries of rocprofv3 result databases (the SQLite "rocpd" output).

    python -m routed_mixture_experts_amd.rocprof_summary trace <results.db> [N]
    python -m routed_mixture_experts_amd.rocprof_summary counters <results.db> [name-filter]
    python -m routed_mixture_experts_amd.rocprof_summary dispatches <results.db> [name-filter]

``trace`` prints per-kernel call counts and total/average durations of a
``--kernel-trace`` run; ``counters`` prints per-dispatch averages of every
counter of a ``--pmc`` run (summed over the counter's hardware instances);
``dispatches`` prints every dispatch's counter values in dispatch order (to
tell apart launches of one kernel with different sizes, such as copies).
"""
from __future__ import annotations

import collections
import sqlite3
import sys


def kernel_stats(db_path: str):
    """[(name, calls, total_ns, avg_ns)] sorted by total time."""
    db = sqlite3.connect(db_path)
    agg = collections.defaultdict(list)
    for name, dur in db.execute("select name, duration from kernels"):
        agg[name].append(dur)
    rows = [(n, len(v), sum(v), sum(v) / len(v)) for n, v in agg.items()]
    return sorted(rows, key=lambda r: -r[2])


def counter_means(db_path: str, name_filter: str = ""):
    """{kernel: {counter: mean per dispatch}} (instances summed per dispatch)."""
    db = sqlite3.connect(db_path)
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(lambda: collections.defaultdict(set))
    for n, c, v, d in db.execute(
            "select name, counter_name, counter_value, dispatch_id from pmc_events"):
        if name_filter and name_filter not in n:
            continue
        tot[n][c] += v
        disp[n][c].add(d)
    return {n: {c: tot[n][c] / len(disp[n][c]) for c in tot[n]} for n in tot}


def counter_dispatches(db_path: str, name_filter: str = ""):
    """[(dispatch_id, kernel, {counter: value})] in dispatch order (instances
    summed per dispatch)."""
    db = sqlite3.connect(db_path)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for n, c, v, d in db.execute(
            "select name, counter_name, counter_value, dispatch_id from pmc_events"):
        if name_filter and name_filter not in n:
            continue
        per[d][c] += v
        names[d] = n
    return [(d, names[d], dict(per[d])) for d in sorted(per)]


def main(argv):
    if len(argv) < 3 or argv[1] not in ("trace", "counters", "dispatches"):
        print(__doc__)
        return 2
    if argv[1] == "trace":
        top = int(argv[3]) if len(argv) > 3 else 20
        print(f"{'calls':>6} {'total_ms':>10} {'avg_us':>11}  kernel")
        for n, c, t, a in kernel_stats(argv[2])[:top]:
            print(f"{c:6d} {t / 1e6:10.3f} {a / 1e3:11.2f}  {n[:110]}")
    elif argv[1] == "dispatches":
        flt = argv[3] if len(argv) > 3 else ""
        for d, n, cs in counter_dispatches(argv[2], flt):
            vals = " ".join(f"{c}={v:.1f}" for c, v in sorted(cs.items()))
            print(f"{d:6d} {vals}  {n[:90]}")
    else:
        flt = argv[3] if len(argv) > 3 else ""
        for n, cs in counter_means(argv[2], flt).items():
            print(n[:110])
            for c, v in sorted(cs.items()):
                print(f"    {c:34s} {v:18.1f}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
