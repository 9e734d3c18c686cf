"""HBM traffic per kernel launch from two rocprofv3 counter runs.

    python -m bit_nf4_quantized_double_amd.pmc FETCH_CSV WRITE_CSV \\
        --copy-bytes B [--out profiles/pmc_traffic.json]

FETCH_CSV / WRITE_CSV are the ``*_counter_collection.csv`` files of
``rocprofv3 --pmc FETCH_SIZE`` and ``rocprofv3 --pmc WRITE_SIZE`` runs of
``bench.py --pmc-pass`` (the same workload as the timed benchmark, plus an
elementwise copy, torch.neg, that reads and writes B bytes once).  FETCH_SIZE and WRITE_SIZE are in KiB per
dispatch; each is scaled by the ratio of the copy's known size to what the
same counter reads for the copy, so the figure is in bytes of the kernel's
own HBM traffic.  The result is keyed by a hash of the kernel's source files;
bench.py reports it only while the sources are unchanged.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel key -> (kernel-name match, source files that define the kernel)
KERNELS = {
    "gemm_fwd_7b": ("k_gemm_nf4<false, qlora::Bf16>", ["gemm.hip", "gemm_args.h", "nf4_lut.h", "common.h",
                                                      "dropout.h"]),
    "gemm_dx_7b": ("k_gemm_nf4<true, qlora::Bf16>", ["gemm.hip", "gemm_args.h", "nf4_lut.h", "common.h",
                                                    "dropout.h"]),
    # the adapter passes of the same layer steps
    "rowpass_x_7b": ("k_rowpass<true, 1, qlora::Bf16, false>", ["adapter.hip", "gemm_args.h", "nf4_lut.h", "common.h",
                                                         "dropout.h"]),
    "rowpass_dy_7b": ("k_rowpass<false, 1, qlora::Bf16, false>", ["adapter.hip", "gemm_args.h", "nf4_lut.h", "common.h",
                                                           "dropout.h"]),
    "colpass_7b": ("k_colpass<1, qlora::Bf16, false>", ["adapter.hip", "gemm_args.h", "nf4_lut.h", "common.h",
                                                 "dropout.h"]),
}
COPY_KERNEL = "neg_kernel"  # torch.neg over PMC_COPY_BYTES of fp32 (bench.py --pmc-pass)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for name in sorted(files):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def per_kernel_kib(path: str, counter: str) -> dict:
    """Average counter value (KiB) per dispatch, by kernel name."""
    acc = defaultdict(lambda: [0.0, 0])
    per_dispatch = defaultdict(float)
    names = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            did = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per_dispatch[did] += float(row["Counter_Value"])
            names[did] = row["Kernel_Name"]
    for did, v in per_dispatch.items():
        a = acc[names[did]]
        a[0] += v
        a[1] += 1
    return {k: (v[0] / v[1], v[1]) for k, v in acc.items()}


def pick(table: dict, needle: str):
    hits = [(k, v) for k, v in table.items() if needle in k]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel matching {needle!r}")
    tot = sum(v[0] * v[1] for _, v in hits)
    n = sum(v[1] for _, v in hits)
    return tot / n, n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--out", default=os.path.join(os.path.dirname(HERE), "profiles", "pmc_traffic.json"))
    args = ap.parse_args()
    fetch = per_kernel_kib(args.fetch_csv, "FETCH_SIZE")
    write = per_kernel_kib(args.write_csv, "WRITE_SIZE")
    cf, _ = pick(fetch, COPY_KERNEL)
    cw, _ = pick(write, COPY_KERNEL)
    f_fetch = args.copy_bytes / (cf * 1024.0)
    f_write = args.copy_bytes / (cw * 1024.0)
    out = {"_calibration": {"copy_bytes": args.copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
                            "fetch_factor": f_fetch, "write_factor": f_write}}
    for key, (needle, files) in KERNELS.items():
        fk, n = pick(fetch, needle)
        wk, _ = pick(write, needle)
        fb = fk * 1024.0 * f_fetch
        wb = wk * 1024.0 * f_write
        out[key] = {"kernel": needle, "dispatches": n, "source_hash": source_hash(files),
                    "fetch_bytes": round(fb), "write_bytes": round(wb),
                    "bytes_per_launch": round(fb + wb)}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
