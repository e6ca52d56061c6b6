"""Summaries of rocprofv3 result databases (SQLite, as written with ``-d <dir> -o <name>``).

Used to produce the text summaries and the HBM traffic record that are kept with the sources:

  python profiling.py summary <results.db> [--title T] [--command C]
      per-kernel dispatch count and average / median / min duration, as Markdown
  python profiling.py traffic --fetch <db> --write <db>
          --copy-fetch <db> --copy-write <db> --kernels k1,k2 --source <file> --out <json>
      FETCH_SIZE / WRITE_SIZE per dispatch of the named kernels, scaled by what the same
      counters read for a plain copy of known size (bench.py --copy-calibration)
"""
import argparse
import collections
import hashlib
import json
import sqlite3
import statistics
import sys


def _rows(db, table):
    con = sqlite3.connect(db)
    cols = [d[1] for d in con.execute(f"pragma table_info({table})")]
    if not cols:
        raise ValueError(f"{db}: no table {table}")
    return cols, con.execute(f"select * from {table}").fetchall()


def kernel_durations(db):
    """{kernel name: [duration ns, ...]} in dispatch order."""
    cols, rows = _rows(db, "kernels")
    ci = {c: i for i, c in enumerate(cols)}
    out = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: r[ci["start"]]):
        out.setdefault(r[ci["name"]], []).append(r[ci["end"]] - r[ci["start"]])
    return out


def counter_values(db, counter):
    """{kernel name: [value per dispatch, ...]} for one collected counter."""
    cols, rows = _rows(db, "counters_collection")
    ci = {c: i for i, c in enumerate(cols)}
    per = collections.OrderedDict()
    for r in rows:
        if r[ci["counter_name"]] != counter:
            continue
        per.setdefault(r[ci["kernel_name"]], {}).setdefault(r[ci["dispatch_id"]], 0.0)
        per[r[ci["kernel_name"]]][r[ci["dispatch_id"]]] += r[ci["value"]]
    return collections.OrderedDict((k, [v[d] for d in sorted(v)]) for k, v in per.items())


def _short(name, n=90):
    return name if len(name) <= n else name[:n - 3] + "..."


def summary(db, title="", command=""):
    lines = []
    if title:
        lines.append(f"# {title}\n")
    if command:
        lines.append(f"Command: `{command}`\n")
    lines.append("| kernel | dispatches | avg µs | median µs | min µs | total µs |")
    lines.append("|---|---:|---:|---:|---:|---:|")
    d = kernel_durations(db)
    for name, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{_short(name)}` | {len(v)} | {statistics.mean(v) / 1e3:.2f} | "
                     f"{statistics.median(v) / 1e3:.2f} | {min(v) / 1e3:.2f} | {sum(v) / 1e3:.1f} |")
    return "\n".join(lines) + "\n"


def _match(values, pattern):
    hits = [k for k in values if pattern in k]
    if len(hits) != 1:
        raise ValueError(f"kernel pattern {pattern!r} matches {hits}")
    return values[hits[0]]


def traffic(fetch_db, write_db, copy_fetch_db, copy_write_db, kernels, source, copy_bytes,
            algorithmic_bytes=None, commands=()):
    """HBM traffic record for one launch of the named kernels (their per-dispatch medians)."""
    cf = counter_values(copy_fetch_db, "FETCH_SIZE")
    cw = counter_values(copy_write_db, "WRITE_SIZE")
    # the copy kernel is the dispatch kind that reads the most (the source fill reads nothing)
    copy_name = max(cf, key=lambda k: statistics.median(cf[k]))
    if copy_name not in cw:
        raise ValueError(f"copy kernel {copy_name!r} has no WRITE_SIZE record")
    fetch_scale = copy_bytes / (statistics.median(cf[copy_name]) * 1024.0)
    write_scale = copy_bytes / (statistics.median(cw[copy_name]) * 1024.0)
    f = counter_values(fetch_db, "FETCH_SIZE")
    w = counter_values(write_db, "WRITE_SIZE")
    raw_f = {k: _match(f, k) for k in kernels}
    raw_w = {k: _match(w, k) for k in kernels}
    fetch_b = sum(statistics.median(v) for v in raw_f.values()) * 1024.0 * fetch_scale
    write_b = sum(statistics.median(v) for v in raw_w.values()) * 1024.0 * write_scale
    rec = {
        "kernels": list(kernels),
        "source_sha256": hashlib.sha256(open(source, "rb").read()).hexdigest(),
        "fetch_kib_per_dispatch_raw": raw_f,
        "write_kib_per_dispatch_raw": raw_w,
        "copy_kernel": copy_name,
        "copy_bytes": copy_bytes,
        "fetch_scale": round(fetch_scale, 4),
        "write_scale": round(write_scale, 4),
        "fetch_bytes_per_launch": int(fetch_b),
        "write_bytes_per_launch": int(write_b),
        "bytes_per_launch": int(fetch_b + write_b),
        "commands": list(commands),
    }
    if algorithmic_bytes is not None:
        rec["algorithmic_bytes_per_launch"] = int(algorithmic_bytes)
    return rec


def counters_table(db, kernels, cus=256, xcds=8, title="", command=""):
    """Markdown: per-dispatch median of every counter in `db` for each kernel pattern."""
    cols, rows = _rows(db, "counters_collection")
    ci = {c: i for i, c in enumerate(cols)}
    names = sorted({r[ci["counter_name"]] for r in rows})
    vals = {n: counter_values(db, n) for n in names}
    lines = []
    if title:
        lines.append(f"# {title}\n")
    if command:
        lines.append(f"Command: `{command}`\n")
    has_busy = "SQ_VALU_MFMA_BUSY_CYCLES" in names and "GRBM_GUI_ACTIVE" in names
    extra = " matrix-core busy |" if has_busy else ""
    lines.append("| kernel | dispatches | " + " | ".join(names) + " |" + extra)
    lines.append("|---|---:|" + "---:|" * (len(names) + has_busy))
    for pat in kernels:
        med = {}
        n = 0
        for c in names:
            v = _match(vals[c], pat)
            n = len(v)
            med[c] = statistics.median(v)
        busy = ""
        if has_busy and med["GRBM_GUI_ACTIVE"]:
            busy = f" {med['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * cus * med['GRBM_GUI_ACTIVE'] / xcds):.3f} |"
        elif has_busy:
            busy = "  |"
        lines.append(f"| `{pat}` | {n} | " + " | ".join(f"{med[c]:.4g}" for c in names) + " |" + busy)
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summary")
    s.add_argument("db")
    s.add_argument("--title", default="")
    s.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernels", "--source", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, default=64 << 20)
    t.add_argument("--algorithmic-bytes", type=int)
    t.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("db")
    c.add_argument("--kernels", required=True, help="kernel name patterns, separated by ',' (or by ';' "
                                                    "when a pattern holds a comma)")
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--title", default="")
    c.add_argument("--command", default="")
    a = ap.parse_args(argv)
    if a.cmd == "summary":
        sys.stdout.write(summary(a.db, a.title, a.command))
    elif a.cmd == "counters":
        pats = a.kernels.split(";" if ";" in a.kernels else ",")
        sys.stdout.write(counters_table(a.db, pats, a.cus, a.xcds, a.title, a.command))
    else:
        rec = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.kernels.split(","), a.source,
                      a.copy_bytes, a.algorithmic_bytes, a.command)
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps({k: rec[k] for k in ("fetch_scale", "write_scale", "bytes_per_launch")}))


if __name__ == "__main__":
    main()
