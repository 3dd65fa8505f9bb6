"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m sparse_attention_diffusion_block_amd.profiling stats KERNEL_STATS_CSV --command "..."
    python -m sparse_attention_diffusion_block_amd.profiling traffic --fetch CSV --write CSV \\
        --copy-fetch CSV --copy-write CSV --copy-bytes N --command "..."

`stats` condenses a `--kernel-trace --stats` kernel-statistics CSV.  `traffic`
turns FETCH_SIZE / WRITE_SIZE counter CSVs (KiB per dispatch) into HBM bytes
per launch, each scaled by what the same counter reads for a plain device copy
of known size, and records the hash of each kernel's source so that a reader
(the bench) can tell whether the counters still describe the current kernel.
"""
import argparse
import collections
import csv
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
# kernel symbol fragment -> source files that define it
KERNEL_SOURCES = {
    "sparse64_kernel": ["sparse64.hip", "common.h", "attn.h"],
    "calib_kernel": ["calib.hip", "common.h", "attn.h"],
    "attn_bf16_kernel": ["attn_bf16.hip", "common.h", "attn.h"],
    "attn_f32_kernel": ["attn_f32.hip", "common.h", "attn.h"],
    "sparse_wg_kernel": ["sparse_wg.hip", "common.h", "attn.h"],
    "dyn_pool_kernel": ["dynamic.hip", "common.h", "attn.h"],
    "dyn_topk_kernel": ["dynamic.hip", "common.h", "attn.h"],
    "index_": ["index.hip", "common.h", "attn.h"],
}


def kernel_source_hash(kernel):
    """sha256 over the source files of a kernel (short form), or None if unknown."""
    for frag, files in KERNEL_SOURCES.items():
        if frag in kernel:
            h = hashlib.sha256()
            for f in files:
                with open(os.path.join(CSRC, f), "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()[:16]
    return None


def short_name(name):
    name = name.replace("void ", "").replace("(rettn::AttnArgs)", "")
    return name.split("(")[0] if "rettn::" not in name else name.replace("rettn::", "")


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def cmd_stats(args):
    rows = _rows(args.csv)
    print(f"# rocprofv3 kernel statistics\n# command: {args.command}")
    print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'total_us':>11s} {'pct':>6s}")
    for r in rows:
        name = short_name(r.get("Name", r.get("KernelName", "?")))
        calls = int(float(r.get("Calls", 0)))
        avg = float(r.get("AverageNs", 0)) / 1e3
        tot = float(r.get("TotalDurationNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
        print(f"{name[:60]:60s} {calls:6d} {avg:10.2f} {tot:11.1f} {pct:6.2f}")


def _counter_means(path, counter):
    acc = collections.defaultdict(list)
    for r in _rows(path):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def cmd_traffic(args):
    cf = _counter_means(args.copy_fetch, "FETCH_SIZE")
    cw = _counter_means(args.copy_write, "WRITE_SIZE")
    copy_name = max(cf, key=lambda k: cf[k])          # the copy kernel: the largest reader
    fetch_scale = args.copy_bytes / (cf[copy_name] * 1024.0)
    write_scale = args.copy_bytes / (cw[max(cw, key=lambda k: cw[k])] * 1024.0)
    fetch = _counter_means(args.fetch, "FETCH_SIZE")
    write = _counter_means(args.write, "WRITE_SIZE")
    print("# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch)")
    print(f"# command: {args.command}")
    print(f"# copy reference: {short_name(copy_name)} moving {args.copy_bytes} bytes each way;"
          f" scale fetch x{fetch_scale:.4f}, write x{write_scale:.4f}")
    print("# kernel | source_sha256 | fetch_kib_raw | write_kib_raw | fetch_bytes | write_bytes | traffic_bytes")
    for k in sorted(set(fetch) & set(write)):
        sha = kernel_source_hash(k)
        if sha is None:
            continue
        fb = fetch[k] * 1024.0 * fetch_scale
        wb = write[k] * 1024.0 * write_scale
        print(f"{short_name(k)} | {sha} | {fetch[k]:.1f} | {write[k]:.1f} | {fb:.0f} | {wb:.0f} | {fb + wb:.0f}")


def read_traffic(path):
    """{kernel short name: (source sha, traffic bytes)} from a `traffic` summary."""
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            if line.startswith("#") or "|" not in line:
                continue
            parts = [p.strip() for p in line.split("|")]
            if len(parts) == 7:
                out[parts[0]] = (parts[1], float(parts[6]))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--command", default="")
    args = ap.parse_args(argv)
    (cmd_stats if args.cmd == "stats" else cmd_traffic)(args)


if __name__ == "__main__":
    sys.exit(main())
