"""Summaries of rocprofv3 result databases for the step's kernels.

``python -m block_drafting_sd_amd.profiling trace <run_results.db>`` prints
the per-kernel dispatch count and average / total duration;
``python -m block_drafting_sd_amd.profiling pmc <run_results.db>`` prints the
average value per dispatch of every collected counter, per kernel;
``python -m block_drafting_sd_amd.profiling pmcgrid <run_results.db>`` the
same per (kernel, grid size), which separates dispatches of one kernel with
different sizes (e.g. a calibration copy of known size from other copies).

rocprofv3 writes its results as a SQLite database (``--output-format`` rocpd,
the default); the views ``kernels`` and ``counters_collection`` hold one row
per dispatch and per (dispatch, counter instance).
"""
from __future__ import annotations

import collections
import re
import sqlite3
import sys


def short_name(name: str) -> str:
    """Kernel name without namespaces noise and argument list."""
    n = name.replace("(anonymous namespace)::", "")
    n = re.sub(r"\(.*$", "", n)
    return n[-80:]


def kernel_times(db: str):
    """{kernel: [durations in ns]} from a --kernel-trace database."""
    con = sqlite3.connect(db)
    out = collections.defaultdict(list)
    for name, dur in con.execute("select name, duration from kernels"):
        out[short_name(name)].append(dur)
    return out


def counters(db: str):
    """{kernel: {counter: [value per dispatch]}} from a --pmc database
    (instances of a counter summed per dispatch)."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, counter_name, sum(value) "
                       "from counters_collection group by dispatch_id, counter_name")
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for kn, _, cn, v in rows:
        out[short_name(kn)][cn].append(v)
    return out


def counters_by_grid(db: str):
    """{(kernel, grid size): {counter: [value per dispatch]}}."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, grid_size, dispatch_id, counter_name, sum(value) "
                       "from counters_collection group by dispatch_id, counter_name")
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for kn, grid, _, cn, v in rows:
        out[(short_name(kn), int(grid))][cn].append(v)
    return out


def pmc_grid_table(db: str) -> str:
    c = counters_by_grid(db)
    lines = ["| kernel | grid size | counter | dispatches | avg per dispatch |", "|---|---|---|---|---|"]
    for (k, grid), cs in sorted(c.items()):
        for cn, vals in sorted(cs.items()):
            lines.append(f"| `{k}` | {grid} | {cn} | {len(vals)} | {sum(vals) / len(vals):.6g} |")
    return "\n".join(lines)


def trace_table(db: str) -> str:
    t = kernel_times(db)
    total = sum(sum(v) for v in t.values()) or 1
    lines = ["| kernel | calls | avg us | total us | share % |", "|---|---|---|---|---|"]
    for k, v in sorted(t.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v) / 1e3:.1f} | {sum(v) / 1e3:.1f} | "
                     f"{100 * sum(v) / total:.2f} |")
    return "\n".join(lines)


def pmc_table(db: str) -> str:
    c = counters(db)
    lines = ["| kernel | counter | dispatches | avg per dispatch |", "|---|---|---|---|"]
    for k, cs in sorted(c.items()):
        for cn, vals in sorted(cs.items()):
            lines.append(f"| `{k}` | {cn} | {len(vals)} | {sum(vals) / len(vals):.6g} |")
    return "\n".join(lines)


def main(argv):
    tables = {"trace": trace_table, "pmc": pmc_table, "pmcgrid": pmc_grid_table}
    if len(argv) != 3 or argv[1] not in tables:
        print(__doc__)
        return 2
    print(tables[argv[1]](argv[2]))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
