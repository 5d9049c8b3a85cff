"""Summaries of rocprofv3 results (the SQLite ``*_results.db`` it writes) for the
credit-assignment kernels.

  python profiling.py stats DB [--command CMD] [--step SUBSTR[xK] ...]
         [--call NAME=SUBSTR ...] [--out FILE]
      per-kernel dispatch count and average / min / max duration (us), from a
      ``rocprofv3 --kernel-trace --stats`` run; --step names the kernels of one
      benchmark step (K launches of that kernel per step) and records the sum
      of their averages as step_avg_us, --call records one call's kernel
      average as call_avg_us.NAME.  bench.py reads those two back.

  python profiling.py traffic --fetch DB --write DB
         --kernel SUBSTR --copy-bytes N --algorithmic-bytes B --out FILE [...]
      HBM bytes per launch of one kernel (or per step of several, --kernel
      repeated) from a ``--pmc FETCH_SIZE`` run and a
      ``--pmc WRITE_SIZE`` run of the same command.  Both counters are scaled
      by what they read for a plain device copy of N bytes (N read + N
      written) captured in the same runs: on gfx950 FETCH_SIZE reads about
      half of the bytes a copy really fetches, WRITE_SIZE reads them exactly.

  python profiling.py counters DB [DB ...]
         --kernel SUBSTR [--command CMD ...]
      median per dispatch of every counter in ``--pmc`` runs, for the kernels
      whose name contains SUBSTR, and per wave where the runs hold SQ_WAVES.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def _kernel_sources():
    csrc = sorted(glob.glob(os.path.join(ROOT, "linear_recurrence_scan_row_amd", "csrc", "*")))
    return [os.path.relpath(p, ROOT) for p in csrc] + ["include/rlca.h"]


def source_digest() -> str:
    """Digest of the kernel sources; stored with a counter summary so that a
    summary taken on other code is not reported for this code."""
    h = hashlib.sha256()
    for rel in _kernel_sources():
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Template arguments of the library's kernels in Itanium mangling, for names
# the trace leaves mangled (rocprofv3 and c++filt do not demangle __bf16).
_TYPE_CODES = {"float": "f", "double": "d", "unsigned int": "j", "__bf16": "DF16b",
               "_Float16": "DF16_", "int": "i"}
_CODE_TYPES = {v: k for k, v in _TYPE_CODES.items()}


def mangled_spec(spec: str) -> str:
    """'backward_scan<0, true, float>' -> 'backward_scanILi0ELb1EfE' (the part
    of the mangled name that identifies the instantiation)."""
    if not spec.endswith(">") or "<" not in spec:
        return spec
    name, args = spec[:-1].split("<", 1)
    codes = []
    for a in (x.strip() for x in args.split(",")):
        if a in ("true", "false"):
            codes.append(f"Lb{int(a == 'true')}E")
        elif a.lstrip("-").isdigit():
            codes.append(f"Li{a}E")
        else:
            codes.append(_TYPE_CODES[a])
    return f"{name}I{''.join(codes)}E"


def readable(name: str) -> str:
    """The mangled names of rlca:: kernel instantiations, demangled enough to
    read (name and template arguments); other names unchanged."""
    import re

    m = re.match(r"_ZN4rlca(\d+)", name)
    if not m:
        return name
    n = int(m.group(1))
    base = name[m.end():m.end() + n]
    rest = name[m.end() + n:]
    if not rest.startswith("I"):
        return name
    rest = rest[1:]
    args = []
    while not rest.startswith("E"):
        t = re.match(r"L([bi])(-?\d+)E", rest)
        if t:
            args.append(("true" if t.group(2) == "1" else "false") if t.group(1) == "b"
                        else t.group(2))
            rest = rest[t.end():]
            continue
        for code, typ in sorted(_CODE_TYPES.items(), key=lambda kv: -len(kv[0])):
            if rest.startswith(code):
                args.append(typ)
                rest = rest[len(code):]
                break
        else:
            return name
    return f"rlca::{base}<{', '.join(args)}>"


def kernel_stats(db: str, match: str = ""):
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, count(*), avg(duration), min(duration), max(duration) from kernels "
        "where name like ? group by name order by sum(duration) desc", (f"%{match}%",)).fetchall()
    return [(n, c, a / 1e3, lo / 1e3, hi / 1e3) for n, c, a, lo, hi in rows]


def counter_values(db: str, counter: str):
    con = sqlite3.connect(db)
    return con.execute(
        "select dispatch_id, kernel_name, value from counters_collection where counter_name = ? "
        "order by dispatch_id", (counter,)).fetchall()


def counter_medians(dbs, kernel):
    """{kernel name: {counter: (dispatches, median value per dispatch)}}."""
    per = {}
    for db in dbs:
        con = sqlite3.connect(db)
        for name, counter, value in con.execute(
                "select kernel_name, counter_name, value from counters_collection"):
            if kernel in name:
                per.setdefault(name.split("(")[0], {}).setdefault(counter, []).append(value)
    out = {}
    for name, counters in per.items():
        out[name] = {}
        for counter, values in counters.items():
            values.sort()
            out[name][counter] = (len(values), values[len(values) // 2])
    return out


def traffic(fetch_db, write_db, kernel, copy_bytes):
    fetch = counter_values(fetch_db, "FETCH_SIZE")
    write = counter_values(write_db, "WRITE_SIZE")
    # calibration: copy dispatches whose writes equal the known copy size
    copy_ids = {d for d, name, v in write
                if "copyBuffer" in name and abs(v * 1024 - copy_bytes) <= 0.01 * copy_bytes}
    if not copy_ids:
        raise SystemExit("no calibration copy found in the WRITE_SIZE run")
    cf = [v for d, name, v in fetch if d in copy_ids]
    cw = [v for d, name, v in write if d in copy_ids]
    fetch_factor = copy_bytes / (1024 * sum(cf) / len(cf))
    write_factor = copy_bytes / (1024 * sum(cw) / len(cw))
    # one step may launch several kernels: the step's traffic is the sum of
    # their average traffic per dispatch
    kernels = [kernel] if isinstance(kernel, str) else list(kernel)
    f_kib = w_kib = 0.0
    counts = []
    for k in kernels:
        alt = mangled_spec(k)
        kf = [v for d, name, v in fetch if k in name or alt in name]
        kw = [v for d, name, v in write if k in name or alt in name]
        if not kf or not kw:
            raise SystemExit(f"kernel {k!r} not found in the counter runs")
        f_kib += sum(kf) / len(kf)
        w_kib += sum(kw) / len(kw)
        counts.append(str(len(kf)))
    return dict(dispatches=counts[0] if len(counts) == 1 else " + ".join(counts),
                fetch_kib_raw=f_kib, write_kib_raw=w_kib,
                calibration_copy_bytes=copy_bytes, calibration_dispatches=len(copy_ids),
                fetch_factor=fetch_factor, write_factor=write_factor,
                traffic_bytes_per_launch=f_kib * 1024 * fetch_factor + w_kib * 1024 * write_factor)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    s.add_argument("--match", default="")
    s.add_argument("--command", default="")
    s.add_argument("--step", action="append", default=[])
    s.add_argument("--call", action="append", default=[])
    s.add_argument("--out", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, action="append",
                   help="kernel name substring; repeat for a step of several launches")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, required=True)
    t.add_argument("--fetch-command", default="")
    t.add_argument("--write-command", default="")
    t.add_argument("--out", default="")
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        lines = [f"command: {cmd}" for cmd in a.command]
        lines.append(f"source_digest: {source_digest()}")
        for name, counters in sorted(counter_medians(a.dbs, a.kernel).items()):
            waves = counters.get("SQ_WAVES", (0, 0.0))[1]
            lines += ["", f"kernel: {name}", "",
                      "| counter | dispatches | median per dispatch | per wave |", "|---|---|---|---|"]
            for counter, (n, v) in sorted(counters.items()):
                # counters summed over waves (instructions, wave-cycles); the
                # others (SQ_BUSY_CYCLES and the like) count per engine
                summed = counter.startswith(("SQ_INSTS", "SQ_ACTIVE", "SQ_WAIT", "SQ_WAVE"))
                pw = f"{v / waves:.2f}" if waves and summed else ""
                lines.append(f"| {counter} | {n} | {v:.6g} | {pw} |")
        print("\n".join(lines))
        return
    if a.cmd == "stats":
        lines = []
        if a.command:
            lines.append(f"command: {a.command}")
        lines.append(f"source_digest: {source_digest()}")
        lines.append("")
        rows = kernel_stats(a.db, a.match)
        every = kernel_stats(a.db)

        def avg_of(sub):
            alt = mangled_spec(sub)
            hits = [r for r in every if sub in r[0] or alt in r[0]]
            if len(hits) != 1:
                raise SystemExit(f"{sub!r} matches {len(hits)} kernels")
            return hits[0][2]

        if a.step:
            total, names = 0.0, []
            for spec in a.step:
                sub, _, times = spec.rpartition("x") if spec[-1].isdigit() and "x" in spec[-3:] \
                    else (spec, "", "1")
                total += int(times) * avg_of(sub)
                names.append(spec)
            lines.append(f"step_kernels: {' + '.join(names)}")
            lines.append(f"step_avg_us: {total:.3f}")
        for spec in a.call:
            name, sub = spec.split("=", 1)
            lines.append(f"call_avg_us.{name}: {avg_of(sub):.3f}")
        lines.append("")
        lines.append("| kernel | dispatches | avg us | min us | max us |")
        lines.append("|---|---|---|---|---|")
        for n, c, avg, lo, hi in rows:
            lines.append(f"| {readable(n)} | {c} | {avg:.3f} | {lo:.3f} | {hi:.3f} |")
        text = "\n".join(lines) + "\n"
        if a.out:
            with open(a.out, "w") as f:
                f.write(text)
        sys.stdout.write(text)
        return
    r = traffic(a.fetch, a.write, a.kernel, a.copy_bytes)
    out = [f"kernel: {' + '.join(a.kernel)}",
           f"fetch_command: {a.fetch_command}",
           f"write_command: {a.write_command}"]
    out += [f"{k}: {v:.6g}" if isinstance(v, float) else f"{k}: {v}" for k, v in r.items()]
    out.append(f"algorithmic_bytes_per_launch: {a.algorithmic_bytes}")
    out.append(f"traffic_over_algorithmic: {r['traffic_bytes_per_launch'] / a.algorithmic_bytes:.4f}")
    out.append(f"source_digest: {source_digest()}")
    text = "\n".join(out) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
