"""Text summaries of rocprofv3 result databases for the kernels of this package.

    python -m fp8_quantized_skinny_amd.profile_summary trace DB [--match SUBSTR]
    python -m fp8_quantized_skinny_amd.profile_summary counters DB [--match SUBSTR]
    python -m fp8_quantized_skinny_amd.profile_summary traffic FETCH_DB WRITE_DB COPY_FETCH_DB COPY_WRITE_DB
            --match SUBSTR --copy-bytes BYTES
    python -m fp8_quantized_skinny_amd.profile_summary sources

`trace` prints, per kernel, the dispatch count and the mean / median / p10 /
p90 duration in microseconds from a `rocprofv3 --kernel-trace` run.
`counters` prints, per kernel and counter, the median value per dispatch from a
`rocprofv3 --pmc` run (FETCH_SIZE and WRITE_SIZE are in KiB).  `traffic`
turns one FETCH_SIZE run and one WRITE_SIZE run of a kernel into HBM bytes per
dispatch, each counter scaled by what it reads for a device-to-device copy of
known size (runs of `bench.py --copy-calibration`): bytes = count * copy_bytes
/ copy_count.  `sources`
prints the SHA-256 of the kernel sources, which ties a counter measurement to
the code it was taken on.
"""

import argparse
import collections
import hashlib
import os
import sqlite3
import sys

import numpy as np

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
KERNEL_SOURCES = ("common.cuh", "internal.h", "xsplit.cuh", "nvfp4_gemm.hip", "fp8_gemm.hip", "reduce.hip")


def _code_only(text):
    """C++ source without its comments and with each line's whitespace collapsed:
    what the compiler sees, so that editing a comment keeps a measurement valid.
    (String literals in these sources hold no comment markers.)"""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = (" ".join(line.split()) for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def sources_sha256():
    """SHA-256 over the code of the kernel source files (comments and blank
    space left out), in a fixed order."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def _demangle(name):
    """Readable name of a mangled kernel symbol of this package (name and template
    arguments only; the system demangler may not know the _Float16 mangling)."""
    import re
    m = re.match(r"_ZN6skinny12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    rest = name[m.end():]
    ident, rest = rest[:int(m.group(1))], rest[int(m.group(1)):]
    args = []
    if rest.startswith("I"):
        for kind, val in re.findall(r"L([bi])(\d+)E", rest[:rest.index("EE") + 1] if "EE" in rest else rest):
            args.append(("true" if val == "1" else "false") if kind == "b" else val)
    return f"skinny::{ident}" + (f"<{', '.join(args)}>" if args else "") + "()"


def _short(name):
    name = _demangle(name).replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0][:48]


def trace_rows(db, match=""):
    cur = sqlite3.connect(db).cursor()
    durs = collections.defaultdict(list)
    for name, d in cur.execute("select name, duration from kernels"):
        if match in name:
            durs[_short(name)].append(d / 1e3)
    return {k: np.array(v) for k, v in durs.items()}


def counter_rows(db, match=""):
    cur = sqlite3.connect(db).cursor()
    vals = collections.defaultdict(list)
    for name, counter, value in cur.execute("select kernel_name, counter_name, value from counters_collection"):
        if match in name:
            vals[(_short(name), counter)].append(value)
    return {k: np.array(v) for k, v in vals.items()}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=("trace", "counters", "traffic", "sources"))
    ap.add_argument("db", nargs="*")
    ap.add_argument("--match", default="")
    ap.add_argument("--copy-bytes", type=float, default=512e6)
    a = ap.parse_args(argv)
    if a.mode == "traffic":
        fetch_db, write_db, copy_fetch_db, copy_write_db = a.db
        def one(db, counter, match):
            rows = {k: v for k, v in counter_rows(db, match).items() if k[1] == counter}
            if len(rows) != 1:
                raise SystemExit(f"{db}: expected one kernel matching {match!r} with {counter}, got {list(rows)}")
            return float(np.median(next(iter(rows.values()))))
        f, w = one(fetch_db, "FETCH_SIZE", a.match), one(write_db, "WRITE_SIZE", a.match)
        cf = one(copy_fetch_db, "FETCH_SIZE", "copyBuffer")
        cw = one(copy_write_db, "WRITE_SIZE", "copyBuffer")
        kf, kw = a.copy_bytes / cf, a.copy_bytes / cw
        print(f"copy of {a.copy_bytes:.0f} bytes: FETCH_SIZE {cf:.4f}, WRITE_SIZE {cw:.4f} per dispatch "
              f"-> {kf:.4f} and {kw:.4f} bytes per count")
        print(f"kernel: FETCH_SIZE {f:.4f}, WRITE_SIZE {w:.4f} per dispatch")
        print(f"hbm_read_bytes_per_launch: {f * kf:.0f}")
        print(f"hbm_write_bytes_per_launch: {w * kw:.0f}")
        print(f"traffic_bytes_per_launch: {f * kf + w * kw:.0f}")
        return
    a.db = a.db[0] if len(a.db) == 1 else a.db
    if a.mode == "sources":
        print(f"kernel_sources_sha256: {sources_sha256()}")
        return
    if a.mode == "trace":
        print(f"{'kernel':48s} {'calls':>6s} {'mean_us':>9s} {'median_us':>9s} {'p10_us':>8s} {'p90_us':>8s}")
        for k, v in sorted(trace_rows(a.db, a.match).items(), key=lambda kv: -kv[1].sum()):
            print(f"{k:48s} {len(v):6d} {v.mean():9.3f} {np.median(v):9.3f} "
                  f"{np.percentile(v, 10):8.3f} {np.percentile(v, 90):8.3f}")
    else:
        print(f"{'kernel':48s} {'counter':18s} {'dispatches':>10s} {'median_per_dispatch':>20s}")
        for (k, c), v in sorted(counter_rows(a.db, a.match).items()):
            print(f"{k:48s} {c:18s} {len(v):10d} {np.median(v):20.4f}")


if __name__ == "__main__":
    sys.exit(main())
