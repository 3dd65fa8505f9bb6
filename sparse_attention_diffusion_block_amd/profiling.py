"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m sparse_attention_diffusion_block_amd.profiling stats KERNEL_STATS_CSV --command "..."
    python -m sparse_attention_diffusion_block_amd.profiling traffic --fetch CSV --write CSV \\
        --copy-fetch CSV --copy-write CSV --copy-bytes N --command "..."
    python -m sparse_attention_diffusion_block_amd.profiling counters CSV [CSV ...] --command "..."

`stats` condenses a `--kernel-trace --stats` kernel-statistics CSV.  `traffic`
turns FETCH_SIZE / WRITE_SIZE counter CSVs (KiB per dispatch) into HBM bytes
per launch, each scaled by what the same counter reads for a plain device copy
of known size, and records the hash of each kernel's source so that a reader
(the bench) can tell whether the counters still describe the current kernel.
`counters` tabulates SQ / GRBM counters (one CSV per collection pass) as the
mean per dispatch of each kernel, with the utilisations derived from them.
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
    "sparse64_kernel": ["sparse64.hip", "common.h", "attn.h", "args.h"],
    "calib_kernel": ["calib.hip", "common.h", "attn.h", "args.h"],
    "v16_kernel": ["calib.hip", "common.h", "attn.h", "args.h"],
    "calib_merge_kernel": ["calib.hip", "common.h", "attn.h", "args.h"],
    "attn_bf16_kernel": ["attn_bf16.hip", "common.h", "attn.h", "args.h"],
    "attn_f32_kernel": ["attn_f32.hip", "common.h", "attn.h", "args.h"],
    "sparse_wg_kernel": ["sparse_wg.hip", "common.h", "attn.h", "args.h"],
    "dyn_pool_kernel": ["dynamic.hip", "common.h", "attn.h", "args.h"],
    "dyn_topk_kernel": ["dynamic.hip", "common.h", "attn.h", "args.h"],
    "index_": ["index.hip", "common.h", "attn.h", "args.h"],
}


def _pad_d(d):
    return 32 if d <= 32 else 64 if d <= 64 else 96 if d <= 96 else 128


def dispatched_kernels(dtype, block, d, L, stride_l=None):
    """(calibration kernel, sparse-step kernel) that the library launches for contiguous
    [B, H, L, d] tensors (row pitch stride_l, default d), named as rocprofv3 reports them in short
    form.  Follows the dispatch of the bf16 and fp32 launchers: the fast kernels take a slice only if
    its 32-bit buffer offsets cannot wrap (rows rounded up to 256, times the pitch in bytes, at most
    2^31 - 256)."""
    sl = d if stride_l is None else stride_l
    fits = -(-L // 256) * 256 * sl * 2 <= (1 << 31) - 256
    dp = _pad_d(d)
    if dtype == "f32":
        return f"attn_f32_kernel<{block}, {dp}, true>", f"attn_f32_kernel<{block}, {dp}, false>"
    # the binding's calibrate passes a workspace, so V is streamed in float16 (the third argument)
    cal = (f"calib_kernel<{block}, {dp}, true>" if block in (64, 128) and fits
           else f"attn_bf16_kernel<{block}, {dp}, true>")
    if block == 64 and d <= 64 and fits:
        sp = f"sparse64_kernel<{dp}>"
    elif (block == 128 or (block == 64 and d > 64)) and fits:
        sp = f"sparse_wg_kernel<{block}, {(96 if dp <= 96 else 128) if block == 64 else dp}>"
    else:
        sp = f"attn_bf16_kernel<{block}, {dp}, false>"
    return cal, sp


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


# SIMDs and compute units of the chip (MI355X: 256 CUs of 4 SIMDs)
CU_NUM, SIMD_NUM = 256, 1024


def _all_counter_means(path):
    """{kernel: {counter: mean value per dispatch}} over every counter in one CSV."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _rows(path):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def derived(c):
    """Utilisations from raw counters, with the definitions rocprofv3 documents for its derived
    metrics.  GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's active cycles are 1/8 of it.
    Missing inputs give no entry."""
    out = {}
    gui = c.get("GRBM_GUI_ACTIVE")
    if not gui:
        return out
    cyc = gui / 8.0                                       # busy cycles of the GPU
    out["gpu_cycles"] = cyc
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out["mfma_busy_pct"] = 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMD_NUM)
    if "SQ_ACTIVE_INST_VALU" in c:                        # quad-cycles, per SE sum
        out["valu_busy_pct"] = 100.0 * 4 * c["SQ_ACTIVE_INST_VALU"] / (cyc * SIMD_NUM)
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out["coexec_pct_of_mfma_busy"] = 100.0 * c["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(c["SQ_VALU_MFMA_BUSY_CYCLES"], 1)
    if "SQ_WAVE_CYCLES" in c:                             # quad-cycles: resident waves per SIMD
        out["waves_per_simd"] = 4 * c["SQ_WAVE_CYCLES"] / (cyc * SIMD_NUM)
    if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c:
        out["lds_bank_conflict_pct_of_active"] = 100.0 * c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1)
    if "SQ_LDS_IDX_ACTIVE" in c:
        out["lds_active_pct"] = 100.0 * c["SQ_LDS_IDX_ACTIVE"] / (cyc * CU_NUM)
    if "SQ_INSTS_VALU" in c and "SQ_WAVES" in c:
        out["valu_insts_per_wave"] = c["SQ_INSTS_VALU"] / c["SQ_WAVES"]
    if "SQ_INSTS_MFMA" in c and "SQ_WAVES" in c:
        out["mfma_insts_per_wave"] = c["SQ_INSTS_MFMA"] / c["SQ_WAVES"]
    return out


def cmd_counters(args):
    merged = collections.defaultdict(dict)
    for path in args.csv:
        for k, cs in _all_counter_means(path).items():
            merged[k].update(cs)
    print(f"# rocprofv3 counters, mean per dispatch (one collection pass per CSV)\n# command: {args.command}")
    for k in sorted(merged):
        if kernel_source_hash(k) is None:
            continue
        c = merged[k]
        print(f"\n## {short_name(k)} | source_sha256 {kernel_source_hash(k)}")
        for name in sorted(c):
            print(f"{name:34s} {c[name]:18.1f}")
        for name, val in derived(c).items():
            print(f"{'= ' + name:34s} {val:18.2f}")


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
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--command", default="")
    args = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
