"""Turn two rocprofv3 counter runs of bench.py into HBM bytes per launch of a kernel.

Run from the repository root on one MI355X (each pass its own process):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d prof/fetch -o p -- \\
      python bench.py --steps 2 --warmup 1 --skip-cpu-baseline --skip-decode --traffic-copy-mib 512 --traffic-dma-check
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d prof/write -o p -- \\
      python bench.py --steps 2 --warmup 1 --skip-cpu-baseline --skip-decode --traffic-copy-mib 512 --traffic-dma-check
  python bench_traffic.py --fetch prof/fetch --write prof/write --copy-mib 512 --dma-check

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what each reads for the
plain copy of known size that bench.py runs first (the copy2d dispatch with the
largest grid): factor = counter bytes / true bytes. With --dma-check the runs also hold one
LDS-DMA GEMM whose weights are each read exactly once; its scaled bytes against its
algorithmic bytes check that a factor taken on 16-byte register loads holds for the
buffer_load ... lds traffic of the GEMM kernels. The result is written to
profiles/<name>_traffic.json, with the sha256 of the kernel's source so that
bench.py reports null once the kernel has changed.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.abspath(__file__))

KERNELS = {
    # name -> (substring of the mangled kernel name, source file)
    "gemm_gateup_swiglu_llama70b_tp8_m4096": (
        "gemm_dtl_kernelILi128ELi256ELi4ELi4ELi1ELb1ELb0EDF16b",
        "tensor_transformer_linear_col_amd/csrc/k_gemm.hip"),
}


def load(d):
    f = glob.glob(os.path.join(d, "*counter_collection.csv"))
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = collections.defaultdict(float)
    meta = {}
    for r in csv.DictReader(open(f[0])):
        key = int(r["Dispatch_Id"])
        per[key] += float(r["Counter_Value"])
        meta[key] = (r["Kernel_Name"], int(r["Grid_Size"]))
    return per, meta


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--dma-check", action="store_true",
                    help="the runs include bench.py --traffic-dma-check: report its scaled bytes")
    args = ap.parse_args()
    true_bytes = args.copy_mib * (1 << 20)
    out = {}
    for counter, d in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        per, meta = load(d)
        copies = [k for k, (n, g) in meta.items() if "copy2d_kernel" in n]
        cal = max(copies, key=lambda k: meta[k][1])
        factor = per[cal] * 1024 / true_bytes
        out[counter] = {"factor": factor, "per": per, "meta": meta}
        print(f"{counter}: calibration copy dispatch {cal} reads {per[cal]:.0f} KiB for {true_bytes} B "
              f"-> factor {factor:.4f}")
    dma_check = None
    if args.dma_check:
        # The LDS-DMA GEMM of 256 tokens x 65536 features x 1024: one 256 x 256 tile per CU
        # (grid 256 x 512 threads); its weights (128 MiB) are read once, the 512 KiB token panel
        # once per XCD at most, the 32 MiB output written once.
        sub = "gemm_dtl_kernelILi256ELi256ELi2ELi4ELi0ELb0ELb0EDF16b"
        dma_check = {}
        for counter, true in (("FETCH_SIZE", (128 << 20) + (256 * 1024 * 2)), ("WRITE_SIZE", 32 << 20)):
            o = out[counter]
            ks = [k for k, (n, g) in o["meta"].items() if sub in n and g == 256 * 512]
            if not ks:
                raise SystemExit(f"DMA check dispatch not found in the {counter} run")
            got = o["per"][ks[0]] * 1024 / o["factor"]
            dma_check[counter] = {"scaled_bytes": round(got), "algorithmic_bytes": true, "ratio": round(got / true, 4)}
            print(f"DMA check {counter}: {got / 2**20:.1f} MiB scaled vs {true / 2**20:.1f} MiB algorithmic "
                  f"(ratio {got / true:.3f})")
    for name, (sub, src) in KERNELS.items():
        vals = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            o = out[counter]
            ks = [k for k, (n, g) in o["meta"].items() if sub in n]
            if not ks:
                raise SystemExit(f"kernel {sub} not found in the {counter} run")
            vals[counter] = sum(o["per"][k] for k in ks) / len(ks) * 1024 / o["factor"]
        total = vals["FETCH_SIZE"] + vals["WRITE_SIZE"]
        sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
        rec = {"kernel": sub, "source": src, "kernel_source_sha256": sha,
               "fetch_bytes_per_launch": round(vals["FETCH_SIZE"]),
               "write_bytes_per_launch": round(vals["WRITE_SIZE"]),
               "bytes_per_launch": round(total),
               "copy_calibration_mib": args.copy_mib,
               "fetch_factor": round(out["FETCH_SIZE"]["factor"], 4),
               "write_factor": round(out["WRITE_SIZE"]["factor"], 4),
               "dma_calibration_check": dma_check}
        path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"{name}: fetch {vals['FETCH_SIZE']/1e6:.1f} MB, write {vals['WRITE_SIZE']/1e6:.1f} MB per launch "
              f"-> {path}")


if __name__ == "__main__":
    main()
