"""Turn rocprofv3 output into the short records bench.py and the profiles
folder keep.

    # a plain copy of known size, for the counters' scale factor
    python -m quantized_expert_ffn_amd.profiling copy --mib 256

    # per-launch HBM bytes of a kernel from two counter runs (FETCH_SIZE,
    # WRITE_SIZE), scaled by what the same counters read for the copy
    python -m quantized_expert_ffn_amd.profiling traffic --key gateup_gemv_olmoe_b16 \\
        --kernel "gemv_kernel<0, true" --source quantized_expert_ffn_amd/csrc/gemv.hip \\
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv --copy-mib 256 \\
        --command "..." [--out profiles/traffic.json]

    # a kernel-trace --stats table as markdown
    python -m quantized_expert_ffn_amd.profiling stats run_kernel_stats.csv --command "..."

    # the mean per dispatch of every counter of one kernel, from --pmc runs
    python -m quantized_expert_ffn_amd.profiling pmc A.csv B.csv --kernel "q8_mfma_kernel<1, true" --command "..."

Only rocprofv3's CSV files are read; nothing here touches the GPU except the
copy command.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def strip_comments(src: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed, so
    that the digest below changes with the code only."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(strip_comments(open(p, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def counter_per_dispatch(path: str, counter: str, kernel_substr: str):
    """Mean value (and dispatch count) of `counter` over the dispatches whose
    kernel name contains kernel_substr, from a --pmc CSV."""
    vals = []
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") == counter and kernel_substr in r.get("Kernel_Name", ""):
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for a kernel matching {kernel_substr!r} in {path}")
    return sum(vals) / len(vals), len(vals)


def cmd_copy(args):
    import torch
    n = args.mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[copy] {args.reps} copies of {args.mib} MiB done", flush=True)


def cmd_traffic(args):
    copy_bytes = args.copy_mib << 20
    cf, _ = counter_per_dispatch(args.copy_fetch, "FETCH_SIZE", args.copy_kernel)
    cw, _ = counter_per_dispatch(args.copy_write, "WRITE_SIZE", args.copy_kernel)
    f, nf = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    w, nw = counter_per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    # the copy reads and writes copy_bytes each: bytes per counter unit
    fetch_factor = copy_bytes / cf
    write_factor = copy_bytes / cw
    rec = {
        "bytes_per_launch": round(f * fetch_factor + w * write_factor),
        "fetch_bytes": round(f * fetch_factor),
        "write_bytes": round(w * write_factor),
        "fetch_counter_per_launch": f,
        "write_counter_per_launch": w,
        "dispatches": [nf, nw],
        "copy_calibration": {"bytes": copy_bytes, "fetch_counter": cf, "write_counter": cw,
                             "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4)},
        "kernel_match": args.kernel,
        "source_digest": source_digest(args.source),
        "sources": [os.path.relpath(p, ROOT) for p in args.source],
        "command": args.command,
    }
    out = args.out
    data = {}
    if os.path.exists(out):
        data = json.load(open(out))
    data[args.key] = rec
    with open(out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({args.key: rec}, indent=1))


def cmd_stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    print(f"Command: `{args.command}`\n")
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows[: args.top]:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")


def cmd_pmc(args):
    """Mean per dispatch of every counter in one or more --pmc CSVs, for the
    dispatches of one kernel, as a markdown table."""
    sums, counts = {}, {}
    for path in args.csv:
        for r in csv.DictReader(open(path)):
            if args.kernel not in r.get("Kernel_Name", ""):
                continue
            k = r["Counter_Name"]
            sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
            counts[k] = counts.get(k, 0) + 1
    if not sums:
        raise SystemExit(f"no rows for a kernel matching {args.kernel!r}")
    print(f"Command: `{args.command}`\n")
    print(f"Kernel: `{args.kernel}`\n")
    print("| counter | mean per dispatch | dispatches |")
    print("|---|---:|---:|")
    for k in sorted(sums):
        print(f"| {k} | {sums[k] / counts[k]:.6g} | {counts[k]} |")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=256)
    c.add_argument("--reps", type=int, default=3)
    t = sub.add_parser("traffic")
    t.add_argument("--key", required=True)
    t.add_argument("--kernel", required=True, help="substring of the kernel name")
    t.add_argument("--source", action="append", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, default=256)
    t.add_argument("--copy-kernel", default="elementwise")
    t.add_argument("--command", required=True)
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=14)
    m = sub.add_parser("pmc")
    m.add_argument("csv", nargs="+")
    m.add_argument("--kernel", required=True, help="substring of the kernel name")
    m.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    {"copy": cmd_copy, "traffic": cmd_traffic, "stats": cmd_stats, "pmc": cmd_pmc}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
