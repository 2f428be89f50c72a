"""Turn two ``rocprofv3 --pmc`` runs of ``traffic_probe.py`` (one with
FETCH_SIZE, one with WRITE_SIZE) into HBM bytes per launch.

Both counters are reported in KiB per dispatch. The probe's plain 1 GiB
device copy (``__amd_rocclr_copyBuffer``) reads and writes a known number of
bytes, so its readings give the counter-to-bytes factors applied to every
kernel of the layer. Writes ``profiles/traffic.json`` entries keyed
``"<kernel>/<workload>"`` (with the hash of the kernel's source file, so
stale entries are recognisable) and prints a markdown table.

Usage: python -m sparse_mixture_experts_20_amd.traffic_summary WORKLOAD \\
           FETCH_DIR WRITE_DIR PROBE_JSON [--json profiles/traffic.json]
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_20_amd", "csrc")
COPY = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def source_sha(path):
    """Hash of a kernel source with its comments and spacing removed (the
    same definition bench.py checks against)."""
    with open(path) as f:
        t = f.read()
    t = re.sub(r"//[^\n]*", "", t)
    t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)
    t = re.sub(r"\s+", " ", t).strip()
    return hashlib.sha256(t.encode()).hexdigest()[:16]


def short(name):
    n = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].strip()


def per_dispatch(run_dir, counter):
    """Average counter value per dispatch, by kernel; for the calibration
    copy, the largest dispatch (small copies of other data may share its
    kernel name)."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    vals = collections.defaultdict(list)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    vals[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (max(v) if k == COPY else sum(v) / len(v)) for k, v in vals.items()}


def algorithmic(kernel, p):
    """Bytes a launch must move at least, from the probe's sizes and counts."""
    N, d, E, k, dff, kept = p["N"], p["d"], p["E"], p["k"], p["d_ff"], p["kept"]
    sx = 2 if p["dtype"] == "bf16" else 4
    noise = N * E * 4 if p["noise"] else 0
    m = re.search(r"expert_gemm_kernel<[^>]*, (\d)>", kernel)
    if m and m.group(1) == "0":       # x (whole), W_up, H rows written
        return N * d * sx + E * dff * d * sx + kept * dff * sx, "x + W_up + H"
    if m and m.group(1) == "1":       # H rows read, W_down, Y rows written
        return kept * dff * sx + E * d * dff * sx + kept * d * sx, "H + W_down + Y"
    if kernel.startswith("router"):
        return N * d * sx + E * d * 4 + noise + N * k * 8, "x + W_g + noise + ids/gates"
    if kernel.startswith("combine"):
        return kept * d * sx + N * k * 8 + N * d * sx, "Y + ids/gates + out"
    return None, ""


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("probe_json")
    ap.add_argument("--json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a = ap.parse_args()
    with open(a.probe_json) as f:
        probe = json.load(f)
    fetch = per_dispatch(a.fetch_dir, "FETCH_SIZE")
    write = per_dispatch(a.write_dir, "WRITE_SIZE")
    ff = COPY_BYTES / (fetch[COPY] * 1024.0)
    wf = COPY_BYTES / (write[COPY] * 1024.0)
    try:
        with open(a.json) as f:
            out = json.load(f)
    except (OSError, ValueError):
        out = {}
    out["_calibration"] = {
        "copy_bytes": COPY_BYTES, "fetch_size_kib": fetch[COPY], "write_size_kib": write[COPY],
        "fetch_factor": ff, "write_factor": wf,
        "note": "bytes = counter_KiB * 1024 * factor, factors from a 1 GiB device copy"}
    print(f"| kernel | fetch MB | write MB | total MB | algorithmic MB | total / algorithmic |")
    print("|---|---|---|---|---|---|")
    for kern in sorted(set(fetch) & set(write)):
        if kern == COPY or kern.startswith("at::") or kern.startswith("void at::"):
            continue   # the calibration copy and torch's own set-up kernels
        fb = fetch[kern] * 1024.0 * ff
        wb = write[kern] * 1024.0 * wf
        alg, what = algorithmic(kern, probe)
        ratio = f"{(fb + wb) / alg:.2f}" if alg else "-"
        algs = f"{alg / 1e6:.2f}" if alg else "-"
        print(f"| `{kern}` | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {(fb + wb) / 1e6:.2f} | {algs} "
              f"| {ratio} |")
        src = "experts.hip" if "gemm" in kern or "fixup" in kern else (
            kern.split("_")[0] + ".hip")
        path = os.path.join(CSRC, src)
        out[f"{kern}/{a.workload}"] = {
            "bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
            "write_bytes": int(round(wb)), "algorithmic_bytes": alg, "algorithmic": what,
            "source_sha": source_sha(path) if os.path.exists(path) else None}
    with open(a.json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
