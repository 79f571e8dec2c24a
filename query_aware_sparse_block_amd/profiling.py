"""Profiling helpers: rocprofv3 summaries, counter-based HBM traffic, and the
plain-copy reference the counters are scaled by.

  python -m query_aware_sparse_block_amd.profiling copy-probe
      One device-to-device copy of exactly 1 GiB (after a warm-up copy): the
      known-size reference for FETCH_SIZE / WRITE_SIZE scaling.
  python -m query_aware_sparse_block_amd.profiling stats STATS_CSV OUT_TXT "COMMAND"
      Text summary of a `rocprofv3 --kernel-trace --stats` kernel_stats.csv.
  python -m query_aware_sparse_block_amd.profiling traffic KERNEL WORKLOAD FETCH_CSV WRITE_CSV \
          COPY_FETCH_CSV COPY_WRITE_CSV "COMMANDS"
      Per-launch HBM bytes of KERNEL (attend, score or dkv_attend) from two
      --pmc runs, scaled by the copy reference, stamped with the digest of the
      kernel's sources; written to profiles/traffic_KERNEL_WORKLOAD.txt.
  python -m query_aware_sparse_block_amd.profiling counters KERNEL WORKLOAD "COMMANDS" CSV [CSV ...]
      The median per launch of every counter the --pmc runs' CSVs hold for
      KERNEL (rocprofv3's derived metrics: VALUBusy, OccupancyPercent, ...),
      stamped with the sources' digest; written to
      profiles/counters_KERNEL_WORKLOAD.txt.
"""

from __future__ import annotations

import csv
import hashlib
import os
import statistics
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_PKG)
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SOURCES = ["csrc/kvsp_attend.h", "csrc/kvsp_decode.hip", "csrc/kvsp_device.h",
                  "csrc/kvsp_api.hip", "csrc/kvsp_internal.h"]
SELECT_SOURCES = ["csrc/kvsp_select.hip", "csrc/kvsp_device.h", "csrc/kvsp_api.hip",
                  "csrc/kvsp_internal.h"]
DKV_SOURCES = ["csrc/kvsp_dkv.hip", "csrc/kvsp_device.h", "csrc/kvsp_api.hip",
               "csrc/kvsp_internal.h"]
SUMMARY_SOURCES = ["csrc/kvsp_summaries.hip", "csrc/kvsp_device.h", "csrc/kvsp_api.hip",
                   "csrc/kvsp_internal.h"]
COPY_BYTES = 1 << 30
# kernel key -> (name prefixes as rocprofv3 prints them, sources, title). The
# DKV kernel's name also contains "attend_kernel", so the main one is matched
# with its namespace.
KERNELS = {
    "attend": (["kvsp::attend_kernel<"], DECODE_SOURCES, "the decode kernel (attend_kernel)"),
    "score": (["kvsp::score_select_kernel<", "kvsp::score_kernel<"], SELECT_SOURCES,
              "the scoring kernel (score_select_kernel / score_kernel)"),
    "dkv_attend": (["dkv_attend_kernel<"], DKV_SOURCES, "the DKV decode kernel (dkv_attend_kernel)"),
    "dkv_compress": (["dkv_compress_kernel<"], DKV_SOURCES, "the DKV codec kernel (dkv_compress_kernel)"),
    "summaries": (["build_summaries_kernel<"], SUMMARY_SOURCES,
                  "the summary build kernel (build_summaries_kernel)"),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{kernel}_{workload.replace('/', '_')}.txt")


def source_digest(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(_PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy_probe():
    import torch
    n = COPY_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)  # warm-up
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes twice", flush=True)


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(path, kernel_prefixes, counter):
    if isinstance(kernel_prefixes, str):
        kernel_prefixes = [kernel_prefixes]
    return [float(r["Counter_Value"]) for r in _rows(path)
            if any(k in r["Kernel_Name"] for k in kernel_prefixes) and r["Counter_Name"] == counter]


def copy_scale(copy_csv, counter):
    """Bytes per counter unit, from the largest copy dispatch (the 1 GiB one)."""
    vals = counter_per_dispatch(copy_csv, COPY_KERNEL, counter)
    if not vals:
        raise RuntimeError(f"no {COPY_KERNEL} dispatch with {counter} in {copy_csv}")
    return COPY_BYTES / max(vals)


def write_traffic(kernel, workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                  commands):
    prefixes, sources, title = KERNELS[kernel]
    fetch = counter_per_dispatch(fetch_csv, prefixes, "FETCH_SIZE")
    write = counter_per_dispatch(write_csv, prefixes, "WRITE_SIZE")
    if not fetch or not write:
        raise RuntimeError(f"no {prefixes} dispatch in {fetch_csv} / {write_csv}")
    fs = copy_scale(copy_fetch_csv, "FETCH_SIZE")
    ws = copy_scale(copy_write_csv, "WRITE_SIZE")
    f_med = statistics.median(fetch)
    w_med = statistics.median(write)
    traffic = f_med * fs + w_med * ws
    lines = [
        f"# HBM traffic of {title}, per launch",
        f"kernel = {kernel}",
        f"workload = {workload}",
        f"source_digest = {source_digest(sources)}",
        f"fetch_size_median_kib = {f_med:.1f}",
        f"write_size_median_kib = {w_med:.1f}",
        f"dispatches = {len(fetch)} / {len(write)}",
        f"fetch_scale_bytes_per_unit = {fs:.4f}",
        f"write_scale_bytes_per_unit = {ws:.4f}",
        f"bytes_read = {f_med * fs:.0f}",
        f"bytes_written = {w_med * ws:.0f}",
        f"traffic_bytes = {traffic:.0f}",
        f"commands = {commands}",
    ]
    out_txt = traffic_path(kernel, workload)
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def recorded_traffic(workload, kernel="attend"):
    """Traffic bytes recorded for `kernel` on `workload`, or None when absent
    or when the kernel's sources changed since the counters were taken."""
    path = traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    sources = KERNELS[kernel][1]
    if kv.get("workload") != workload or kv.get("source_digest") != source_digest(sources):
        return None
    return float(kv["traffic_bytes"])


def write_counters(kernel, workload, commands, *csvs):
    prefixes, sources, title = KERNELS[kernel]
    values = {}
    for path in csvs:
        for r in _rows(path):
            if any(k in r["Kernel_Name"] for k in prefixes):
                values.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not values:
        raise RuntimeError(f"no {prefixes} dispatch in {csvs}")
    lines = [f"# rocprofv3 counters of {title}, median per launch",
             f"kernel = {kernel}",
             f"workload = {workload}",
             f"source_digest = {source_digest(sources)}"]
    for name in sorted(values):
        v = values[name]
        lines.append(f"{name} = {statistics.median(v):.2f}  (dispatches {len(v)}, "
                     f"min {min(v):.2f}, max {max(v):.2f})")
    lines.append(f"commands = {commands}")
    out_txt = os.path.join(PROFILES, f"counters_{kernel}_{workload.replace('/', '_')}.txt")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_stats(stats_csv, out_txt, command, top=12):
    rows = _rows(stats_csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 --kernel-trace --stats: {command}", "",
             f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows[:top]:
        name = r["Name"]
        if len(name) > 72:
            name = name[:69] + "..."
        lines.append(f"{name:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                     f"{float(r['Percentage']):>6.2f}")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv):
    if not argv:
        print(__doc__)
        return 2
    cmd = argv[0]
    if cmd == "copy-probe":
        copy_probe()
    elif cmd == "stats":
        write_stats(argv[1], argv[2], argv[3])
    elif cmd == "traffic":
        write_traffic(*argv[1:8])
    elif cmd == "counters":
        write_counters(*argv[1:])
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
