"""Turns rocprofv3 output into the text summaries kept under profiles/.

Commands (run from the repository root):

  python -m gpt_pre_norm_amd.profiling calibrate [--mib 1024]
      One device-to-device copy of a known size; profile it with the same
      counters as the workload to get the scale from counter KiB to bytes.

  python -m gpt_pre_norm_amd.profiling stats STATS_CSV OUT_TXT --command "..." [--trace TRACE_CSV]
      Per-kernel table (calls, average, median and total duration) from
      rocprofv3 --kernel-trace --stats (the median from the kernel trace).

  python -m gpt_pre_norm_amd.profiling traffic --fetch CSV --write CSV
         --cal-fetch CSV --cal-write CSV --cal-mib N --out profiles/traffic.json
         --command "..."
      HBM-side bytes per launch for each kernel kind from two --pmc runs
      (FETCH_SIZE, WRITE_SIZE), each scaled by what the same counter reads for
      the calibration copy.  The record carries a hash of the kernel sources,
      so bench.py ignores it once the kernels change.

  python -m gpt_pre_norm_amd.profiling core --pmc CSV --trace CSV --out TXT
         --command "..."
      Per kernel kind, from one --pmc run with --kernel-trace: matrix-core
      busy cycles against the launch's duration (at the nominal 2.4 GHz, so a
      lower bound on the busy fraction), the bf16 MFMA work the counters saw
      against the algorithmic flops, and LDS bank-conflict cycles against LDS
      active cycles.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def sources_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gpt_pre_norm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    n = name.replace("void ", "").replace("gpt2::", "")
    n = re.sub(r"\(.*", "", n)
    n = n.replace("unsigned short", "bf16")
    return n


def kind_of(name: str, prev_kind: str | None) -> str:
    """Maps a kernel symbol to the kind names gpt2_timing_end reports."""
    n = short_name(name)
    if "embed" in n:
        return "embed"
    if "layernorm_kernel" in n or "layernorm_reduce" in n:
        # the reduce form also adds the residual product's partial sums
        return "layernorm"
    if "attn_prefill" in n:
        return "attn_prefill"
    if "attn_decode" in n:
        return "attn_decode"
    if "attn_rows" in n:
        return "attn_rows"
    if "EpiQKV" in n:
        return "gemm_c_attn"
    if "EpiBiasGelu" in n:
        return "gemm_c_fc"
    if "EpiLoss" in n:
        return "gemm_lm_head_loss"
    if "EpiStoreF32" in n:
        return "gemm_lm_head"
    if "EpiResidInPlace" in n or "EpiBiasResid" in n or "EpiPartial" in n:
        # the block's two residual products: after attention, after c_fc
        return "gemm_mlp_c_proj" if prev_kind == "gemm_c_fc" else "gemm_attn_c_proj"
    return n


def read_pmc(path: str, counter: str):
    """[(dispatch_id, kernel_name, grid_size, value)] in dispatch order."""
    agg = collections.OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            if key not in agg:
                agg[key] = [r["Kernel_Name"], int(r["Grid_Size"]), 0.0]
            agg[key][2] += float(r["Counter_Value"])
    return [(k, v[0], v[1], v[2]) for k, v in sorted(agg.items())]


def classify(rows):
    """Adds (phase, kind) to each dispatch.  bench.py runs the forward first and
    the decode step second; the first decode-only kernel (the weight-streaming
    product or the decode attention) starts the decode phase."""
    out = []
    prev = None
    phase = "forward"
    for did, name, grid, val in rows:
        # the decode step starts with its embedding of 64 tokens (64 one-wave
        # workgroups: a small grid)
        if ("embed" in name and grid < 65536) or "skinny" in name or "attn_decode" in name:
            phase = "decode"
        k = kind_of(name, prev)
        out.append((did, phase, k, grid, val))
        if k != "layernorm":
            prev = k
    return out


def cmd_calibrate(args):
    import torch
    n = args.mib << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(f"calibration copy of {n} bytes done", flush=True)


def cmd_stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    # per-kernel median launch duration from the kernel trace, when given:
    # the average of the stats table also counts the first (cold) launches
    med = {}
    if args.trace:
        durs = collections.defaultdict(list)
        for r in csv.DictReader(open(args.trace)):
            durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        for name, d in durs.items():
            d.sort()
            med[name] = d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"# command: {args.command}", "#",
             f"{'kernel':80s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} {'max_us':>10s} "
             f"{'total_ms':>9s} {'pct':>6s}"]
    for r in rows:
        m = med.get(r["Name"])
        lines.append(f"{short_name(r['Name'])[:80]:80s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{(f'{m:10.2f}' if m is not None else f'{chr(45):>10s}')} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['TotalDurationNs']) / 1e6:9.3f} {float(r['Percentage']):6.2f}")
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[:30]))


def cmd_traffic(args):
    cal_bytes = args.cal_mib << 20

    def cal_scale(path, counter):
        rows = read_pmc(path, counter)
        # the calibration copy is the largest dispatch in its run
        kib = max(v for _, _, _, v in rows)
        return cal_bytes / (kib * 1024.0), kib

    sf, f_kib = cal_scale(args.cal_fetch, "FETCH_SIZE")
    sw, w_kib = cal_scale(args.cal_write, "WRITE_SIZE")
    fetch = classify(read_pmc(args.fetch, "FETCH_SIZE"))
    write = classify(read_pmc(args.write, "WRITE_SIZE"))
    per = collections.defaultdict(lambda: {"fetch": [], "write": []})
    for _, phase, k, grid, v in fetch:
        if k.startswith(("gemm", "attn", "layernorm", "embed")):
            per[(phase, k)]["fetch"].append(v * 1024.0 * sf)
    for _, phase, k, grid, v in write:
        if k.startswith(("gemm", "attn", "layernorm", "embed")):
            per[(phase, k)]["write"].append(v * 1024.0 * sw)
    out = {"source_sha": sources_sha(), "command": args.command,
           "calibration": {"bytes": cal_bytes, "fetch_kib": f_kib, "write_kib": w_kib,
                           "fetch_scale": sf, "write_scale": sw},
           "forward": {}, "decode": {}}
    for (phase, k), d in sorted(per.items()):
        if not d["fetch"] or not d["write"]:
            continue
        fb = sum(d["fetch"]) / len(d["fetch"])
        wb = sum(d["write"]) / len(d["write"])
        out[phase][k] = {"launches": len(d["fetch"]), "fetch_bytes": fb, "write_bytes": wb,
                         "bytes_per_launch": fb + wb}
    json.dump(out, open(args.out, "w"), indent=1)
    for phase in ("forward", "decode"):
        for k, v in out[phase].items():
            print(f"{phase:8s} {k:20s} {v['launches']:5d} fetch {v['fetch_bytes'] / 1e6:10.2f} MB  "
                  f"write {v['write_bytes'] / 1e6:10.2f} MB")


CORE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT",
                 "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS")
N_SIMD = 1024      # 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9   # nominal peak engine clock


def cmd_core(args):
    from gpt_pre_norm_amd import roofline as R
    from gpt_pre_norm_amd.workloads import WORKLOADS
    dur = {}
    for r in csv.DictReader(open(args.trace)):
        dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    vals = {c: {did: v for did, _, _, v in read_pmc(args.pmc, c)} for c in CORE_COUNTERS}
    base = read_pmc(args.pmc, CORE_COUNTERS[0])
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for did, phase, k, grid, _ in classify(base):
        if did not in dur or not k.startswith(("gemm", "attn", "layernorm", "embed")):
            continue
        d = per[(phase, k)]
        d["n"] += 1
        d["sec"] += dur[did]
        for c in CORE_COUNTERS:
            d[c] += vals[c].get(did, 0.0)
    fw, dw = WORKLOADS["gpt2s_fwd_b8_t1024"], WORKLOADS["gpt2s_decode_b64_p1023"]
    lines = ["# matrix-core and LDS counters per kernel kind (rocprofv3 --pmc with --kernel-trace)",
             f"# command: {args.command}",
             "# mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x duration x 2.4 GHz), a lower bound",
             "# mops_vs_alg: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / algorithmic flops of the launch",
             "# lds_conflict: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
             "#",
             f"{'phase':8s} {'kernel':18s} {'launches':>8s} {'avg_us':>9s} {'mfma_busy':>10s} {'mops_vs_alg':>12s} "
             f"{'lds_conflict':>13s} {'lds_insts/launch':>17s}"]
    for (phase, k), d in sorted(per.items()):
        n = int(d["n"])
        avg = d["sec"] / n
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * d["sec"] * CLOCK_HZ)
        wl = fw if phase == "forward" else dw
        B, T = (wl.B, wl.T) if phase == "forward" else (wl.B, 1)
        f, _ = R.kernel_work(k, B=B, T=T, d=wl.d, h=wl.h, V=wl.n_vocab, l_past=getattr(wl, "l_past", 0))
        mops = d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / (f * n) if f else float("nan")
        conf = d["SQ_LDS_BANK_CONFLICT"] / d["SQ_LDS_IDX_ACTIVE"] if d["SQ_LDS_IDX_ACTIVE"] else 0.0
        lines.append(f"{phase:8s} {k:18s} {n:8d} {avg * 1e6:9.2f} {busy:10.3f} {mops:12.3f} {conf:13.4f} "
                     f"{d['SQ_INSTS_LDS'] / n:17.4g}")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("calibrate")
    c.add_argument("--mib", type=int, default=1024)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--trace", default=None, help="kernel_trace.csv of the same run (adds median_us)")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write", "--out", "--command"):
        t.add_argument(a, required=True)
    t.add_argument("--cal-mib", type=int, default=1024)
    c2 = sub.add_parser("core")
    for a in ("--pmc", "--trace", "--out", "--command"):
        c2.add_argument(a, required=True)
    args = ap.parse_args(argv)
    {"calibrate": cmd_calibrate, "stats": cmd_stats, "traffic": cmd_traffic, "core": cmd_core}[args.cmd](args)


if __name__ == "__main__":
    main(sys.argv[1:])
