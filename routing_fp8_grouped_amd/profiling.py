"""Summaries of rocprofv3 output for the layer's kernels.

    python -m routing_fp8_grouped_amd.profiling stats DIR --command CMD
    python -m routing_fp8_grouped_amd.profiling traffic FETCH_DIR WRITE_DIR \\
        --workload NAME --command-fetch CMD --command-write CMD
    python -m routing_fp8_grouped_amd.profiling counters DIR [DIR ...] \\
        --kernel FRAGMENT [--kernel ...] --command CMD [--command ...]

``stats`` condenses ``rocprofv3 --kernel-trace --stats --output-format csv``
(the ``*kernel_stats.csv`` file) into a short table of per-kernel call
counts and durations.

``counters`` averages every counter of one or more ``rocprofv3 --pmc`` runs
per dispatch of the kernels whose names contain the given fragments.

``traffic`` turns two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``
runs of ``bench.py`` into HBM bytes per launch of the first expert GEMM (the
tiled kernel, or with ``--kernel`` the weight-streaming one of small batches).  Both
counters are in KiB per dispatch but count L2-to-memory requests, so each is
scaled by what it reads for the 1 GiB elementwise copy ``bench.py`` runs
before its timed region (1 GiB read and 1 GiB written): factor = 1 GiB /
counter(copy).  The copy is taken as the elementwise dispatch with the largest
counter value.  The summary records a hash of the GEMM's source so that
``bench.py`` reports the figure only while the kernel is the one measured.
"""

import argparse
import collections
import csv
import glob
import hashlib
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TILED = "grouped_gemm_kernel<true, false>"
STREAMING = "grouped_gemm_small_kernel<true, false>"
# sources whose hash identifies the kernel a traffic summary was taken on
KERNEL_SOURCES = {
    TILED: ["routing_fp8_grouped_amd/csrc/gemm.hip", "routing_fp8_grouped_amd/csrc/common.h"],
    STREAMING: ["routing_fp8_grouped_amd/csrc/gemm_small.hip", "routing_fp8_grouped_amd/csrc/common.h"],
}
GEMM_SOURCES = KERNEL_SOURCES[TILED]
KERNELS = {
    "grouped_gemm_kernel<true, false>": "grouped_gemm_fp8_up",
    "grouped_gemm_kernel<false, false>": "grouped_gemm_fp8_down",
    "grouped_gemm_kernel<true, true>": "grouped_gemm_fp8_up_e8m0",
    "grouped_gemm_kernel<false, true>": "grouped_gemm_fp8_down_e8m0",
    "grouped_gemm_small_kernel<true, false>": "grouped_gemm_fp8_up (few rows)",
    "grouped_gemm_small_kernel<true, true>": "grouped_gemm_fp8_up_e8m0 (few rows)",
    "grouped_gemm_small_kernel<false, false>": "grouped_gemm_fp8_down (few rows)",
    "route_kernel": "moe_route",
    "route_logits_kernel": "moe_route_ws (logits)",
    "route_select_kernel": "moe_route_ws (select)",
    "quant_1x128_kernel<false>": "fp8_quant_1x128",
    "quant_128x128_kernel<false>": "fp8_quant_128x128",
    "quant_1x128_kernel<true>": "fp8_quant_1x128_pow2",
    "quant_128x128_kernel<true>": "fp8_quant_128x128_pow2",
    "permute_count": "moe_permute (count)",
    "permute_scan": "moe_permute (scan)",
    "permute_scatter": "moe_permute (scatter)",
    "permute_gather": "moe_permute (gather)",
    "combine_kernel": "moe_combine",
    "bias_update_kernel": "moe_bias_update",
    "roof_mfma_kernel": "moe_roof_fp8_mfma",
    "roof_read_kernel": "moe_roof_hbm_read",
    "roof_dma_kernel": "moe_roof_dma_read",
    "roof_chase_kernel": "moe_roof_hbm_latency",
}
GIB_KIB = float(1 << 20)


def gemm_source_hash(kernel=TILED):
    """First 16 hex digits of the SHA-256 of the first expert GEMM's sources
    (the tiled kernel, or the weight-streaming kernel of small batches)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name):
    for frag, label in KERNELS.items():
        if frag in name:
            return label
    return None


def _find(d, suffix):
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return files


def stats_table(d):
    rows = []
    for path in _find(d, "kernel_stats.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append(r)
    out = []
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        label = _short(r["Name"]) or r["Name"][:60]
        out.append(f"{label:<40} calls {int(r['Calls']):>6}  avg {float(r['AverageNs']) / 1e3:>10.1f} us  "
                   f"min {float(r['MinNs']) / 1e3:>10.1f}  max {float(r['MaxNs']) / 1e3:>10.1f}  "
                   f"share {100 * float(r['TotalDurationNs']) / total:5.1f}%")
    return out


def per_dispatch(d, counter):
    """{dispatch id: (kernel name, value)} summed over the counter's
    instances (one row per dispatch after rocprofv3's own reduction)."""
    vals = collections.defaultdict(float)
    names = {}
    for path in _find(d, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (path, r["Dispatch_Id"])
                vals[key] += float(r["Counter_Value"])
                names[key] = r["Kernel_Name"]
    return {k: (names[k], v) for k, v in vals.items()}


def counters(dirs, fragments):
    """{kernel label: {counter: (mean per dispatch, dispatches)}} over the
    --pmc runs in ``dirs``, for kernels whose names contain a fragment."""
    per = collections.defaultdict(float)
    names = {}
    for d in dirs:
        for path in _find(d, "counter_collection.csv"):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if not any(fr in r["Kernel_Name"] for fr in fragments):
                        continue
                    per[(path, r["Dispatch_Id"], r["Counter_Name"])] += float(r["Counter_Value"])
                    names[(path, r["Dispatch_Id"])] = r["Kernel_Name"]
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for (path, disp, counter), v in per.items():
        name = names[(path, disp)]
        agg[_short(name) or name[:60]][counter].append(v)
    return {k: {c: (sum(v) / len(v), len(v)) for c, v in cs.items()} for k, cs in agg.items()}


def traffic(fetch_dir, write_dir, kernel_frag=TILED):
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = per_dispatch(d, counter)
        gemm = [v for n, v in disp.values() if kernel_frag in n]
        copy = [v for n, v in disp.values() if _short(n) is None and "moe" not in n]
        if not gemm or not copy:
            raise SystemExit(f"{counter}: kernel or calibration copy missing in {d}")
        res[counter] = {"kib_per_launch": sum(gemm) / len(gemm), "launches": len(gemm),
                        "copy_kib": max(copy)}
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--workload", required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--kernel", default=TILED, choices=sorted(KERNEL_SOURCES))
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--command", action="append", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(f"rocprofv3 kernel statistics\ncommand: {a.command}\n")
        print("\n".join(stats_table(a.dir)))
        return
    if a.cmd == "counters":
        print("rocprofv3 hardware counters, mean per dispatch")
        for cmd in a.command:
            print(f"command: {cmd}")
        for k, cs in sorted(counters(a.dirs, a.kernel).items()):
            print(f"\n{k}")
            for cname, (v, n) in sorted(cs.items()):
                print(f"    {cname:<32} {v:12.5g}   ({n} dispatches)")
        return
    r = traffic(a.fetch_dir, a.write_dir, a.kernel)
    f, w = r["FETCH_SIZE"], r["WRITE_SIZE"]
    kf, kw = GIB_KIB / f["copy_kib"], GIB_KIB / w["copy_kib"]
    hbm = (f["kib_per_launch"] * kf + w["kib_per_launch"] * kw) * 1024
    print(f"grouped_gemm_fp8_up HBM traffic, workload {a.workload}")
    print(f"command_fetch: {a.command_fetch}")
    print(f"command_write: {a.command_write}")
    print(f"kernel: {a.kernel}")
    print(f"kernel_source_sha256_16: {gemm_source_hash(a.kernel)}")
    print(f"launches: {f['launches']}")
    print(f"fetch_kib_per_launch: {f['kib_per_launch']:.1f}")
    print(f"write_kib_per_launch: {w['kib_per_launch']:.1f}")
    print(f"copy_fetch_kib (1 GiB copy): {f['copy_kib']:.1f}")
    print(f"copy_write_kib (1 GiB copy): {w['copy_kib']:.1f}")
    print(f"fetch_factor: {kf:.4f}")
    print(f"write_factor: {kw:.4f}")
    print(f"hbm_bytes_per_launch: {hbm:.6g}")


if __name__ == "__main__":
    sys.exit(main())
