"""HBM traffic per kernel launch from rocprofv3 counter passes.

Two `rocprofv3 --pmc` runs of the same command (one with FETCH_SIZE, one with
WRITE_SIZE; the counters are KiB per dispatch) are reduced to mean KiB per launch of a
kernel, then scaled by what the same counters read for a plain copy of known size in
the same runs (bench.py --copy-calibration runs one): factor = known KiB / counted KiB.
The result is written as JSON (read by bench.py for the roofline "traffic" field) plus
a short text summary, both stamped with a digest of the kernel's sources so that a
stale measurement is not reported after the kernel changes.

    python -m cohere2_block_mrope_amd.pmc_traffic --fetch DIR --write DIR \\
        --kernel 'gemm_bf16_kernel<256, 256, 0, 1>' --copy-bytes N --name NAME \\
        --sources gemm_bf16.hip gemm_common.h common.h launch.h --command '...'
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL = "copyBuffer"


def source_digest(files) -> str:
    """sha256 over the named csrc files, in the given order."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _rows(d: str):
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def mean_kib(d: str, counter: str, kernel: str, min_kib: float = 0.0, grid: int = 0):
    """(mean value, dispatch count) of `counter` over dispatches whose name contains `kernel`
    (and, when grid > 0, whose grid holds exactly `grid` work-items)."""
    vals = [float(r["Counter_Value"]) for r in _rows(d)
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]
            and (grid <= 0 or int(r.get("Grid_Size", -1)) == grid)]
    vals = [v for v in vals if v >= min_kib]
    if not vals:
        raise SystemExit(f"no {counter} dispatches of '{kernel}' under {d}")
    return sum(vals) / len(vals), len(vals)


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--fetch", required=True, help="output dir of the FETCH_SIZE pass")
    p.add_argument("--write", required=True, help="output dir of the WRITE_SIZE pass")
    p.add_argument("--kernel", required=True, help="substring of the kernel name")
    p.add_argument("--copy-bytes", type=int, required=True, help="bytes read (= written) by one calibration copy")
    p.add_argument("--name", required=True, help="record name: profiles/<name>_traffic.{json,md}")
    p.add_argument("--sources", nargs="+", required=True, help="csrc files the kernel is built from")
    p.add_argument("--algorithmic-bytes", type=float, default=None)
    p.add_argument("--grid", type=int, default=0, help="only dispatches of this many work-items")
    p.add_argument("--command", default="", help="the command line of the counter passes, for the summary")
    a = p.parse_args(argv)

    known_kib = a.copy_bytes / 1024.0
    # Only the large calibration copies (the runtime also issues small copy kernels).
    big = 0.25 * known_kib
    cf, ncf = mean_kib(a.fetch, "FETCH_SIZE", COPY_KERNEL, big)
    cw, ncw = mean_kib(a.write, "WRITE_SIZE", COPY_KERNEL, big)
    kf, nkf = mean_kib(a.fetch, "FETCH_SIZE", a.kernel, grid=a.grid)
    kw, nkw = mean_kib(a.write, "WRITE_SIZE", a.kernel, grid=a.grid)
    f_fetch, f_write = known_kib / cf, known_kib / cw
    read_b, write_b = kf * 1024 * f_fetch, kw * 1024 * f_write
    rec = {
        "kernel": a.kernel,
        "grid_work_items": a.grid or None,
        "source_files": a.sources,
        "source_sha256": source_digest(a.sources),
        "hbm_bytes_per_launch": read_b + write_b,
        "hbm_read_bytes_per_launch": read_b,
        "hbm_write_bytes_per_launch": write_b,
        "algorithmic_bytes_per_launch": a.algorithmic_bytes,
        "counters_kib_per_launch": {"FETCH_SIZE": kf, "WRITE_SIZE": kw},
        "launches": {"fetch_pass": nkf, "write_pass": nkw},
        "calibration": {"copy_bytes": a.copy_bytes, "FETCH_SIZE_kib": cf, "WRITE_SIZE_kib": cw,
                        "fetch_factor": f_fetch, "write_factor": f_write, "copies": [ncf, ncw]},
        "command": a.command,
    }
    out = os.path.join(ROOT, "profiles", f"{a.name}_traffic")
    with open(out + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    alg = f"{a.algorithmic_bytes / 1e6:.1f} MB" if a.algorithmic_bytes else "n/a"
    lines = [
        f"# HBM traffic of `{a.kernel}` ({a.name})" + (f", dispatches of {a.grid:,} work-items" if a.grid else ""),
        "",
        f"Counter passes (each its own run): `{a.command}`",
        "",
        "| quantity | per launch |",
        "|---|---|",
        f"| FETCH_SIZE (counter) | {kf:,.0f} KiB over {nkf} launches |",
        f"| WRITE_SIZE (counter) | {kw:,.0f} KiB over {nkw} launches |",
        f"| calibration copy of {a.copy_bytes / 2**20:.0f} MiB | FETCH {cf:,.0f} KiB, WRITE {cw:,.0f} KiB "
        f"-> factors {f_fetch:.4f} / {f_write:.4f} |",
        f"| HBM read (scaled) | {read_b / 1e6:,.1f} MB |",
        f"| HBM write (scaled) | {write_b / 1e6:,.1f} MB |",
        f"| algorithmic bytes | {alg} |",
        "",
        f"Sources digest (sha256 of {', '.join(a.sources)}): `{rec['source_sha256']}`",
        "",
    ]
    with open(out + ".md", "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
