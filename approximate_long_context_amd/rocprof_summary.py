"""Summaries of rocprofv3 output for the measurement record.

    python -m approximate_long_context_amd.rocprof_summary stats \\
        --csv DIR/..._kernel_stats.csv --command "..." --out profiles/NAME.md

writes the per-kernel duration table of a `rocprofv3 --kernel-trace --stats`
run (with the command that produced it) as markdown.

    python -m approximate_long_context_amd.rocprof_summary traffic \\
        --fetch DIR --write DIR --calib-fetch DIR --calib-write DIR \\
        --calib-bytes N --kernel attn_mfma_kernel --workload NAME \\
        --kernel-sha SHA --algorithmic-bytes B --commands FILE \\
        --out-md profiles/NAME.md --out-json profiles/traffic.json

turns two counter runs of the benchmark (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) into HBM bytes per launch of the named kernel.  Each counter is
scaled by what it reads for a plain copy of known size (`bench.py
--copy-calibration`), which reads and writes exactly N bytes.

    python -m approximate_long_context_amd.rocprof_summary mfma \
        --run DIR --kernel attn_mfma_kernel --workload NAME --kernel-sha SHA \
        --issued-pairs P --flops-per-pair F --command "..." \
        --out-md profiles/NAME.md --out-json profiles/mfma.json

turns a counter run with SQ_INSTS_VALU_MFMA_MOPS_BF16 and
SQ_VALU_MFMA_BUSY_CYCLES into the bf16 matrix-core work per launch.  The
counter counts units of 512 flops; the run is checked against the pairs the
kernel issues by construction (P pairs of F flops each, from the tables).

    python -m approximate_long_context_amd.rocprof_summary sweep \
        --jsonl FILE --command "python bench.py --sweep" --out profiles/NAME.md

turns the JSON lines of `bench.py --sweep` into a markdown table (and keeps
the lines themselves below it).

    python -m approximate_long_context_amd.rocprof_summary crossover \
        --jsonl FILE --command "python bench.py --crossover" --out profiles/NAME.md

does the same for the estimator-against-exact-ALiBi lines of `bench.py
--crossover`.
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        sys.exit(f"no file matches {pattern}")
    return hits[0]


def kernel_stats_md(csv_path: str, command: str) -> str:
    rows = list(csv.DictReader(open(csv_path)))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share (%) |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("|", "\\|")
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "Command:\n\n```\n" + command + "\n```\n\n" + "\n".join(out) + "\n"


def counter_per_dispatch(run_dir: str, counter: str, kernel_substr: str, largest: bool = False):
    """Mean value of `counter` per dispatch of kernels whose name contains
    kernel_substr (largest=True: only the dispatches with the largest value,
    i.e. the calibration copies rather than small incidental copies)."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
            continue
        key = r["Dispatch_Id"]
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        sys.exit(f"{path}: no {counter} for kernels matching {kernel_substr!r}")
    vals = list(per.values())
    if largest:
        top = max(vals)
        vals = [v for v in vals if v >= 0.99 * top]
    return statistics.mean(vals), len(vals)


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("--csv", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--out", required=True)
    a.add_argument("--title", default="rocprofv3 kernel trace")
    t = sub.add_parser("traffic")
    for f in ("fetch", "write", "calib_fetch", "calib_write"):
        t.add_argument("--" + f.replace("_", "-"), required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--calib-kernel", default="copyBuffer")
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--kernel-sha", required=True)
    t.add_argument("--algorithmic-bytes", type=float, required=True)
    t.add_argument("--commands", required=True, help="text file with the commands of the four runs")
    t.add_argument("--out-md", required=True)
    t.add_argument("--out-json", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--run", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--kernel-sha", required=True)
    m.add_argument("--issued-pairs", type=float, required=True)
    m.add_argument("--flops-per-pair", type=float, required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--out-md", required=True)
    m.add_argument("--out-json", required=True)
    w = sub.add_parser("sweep")
    w.add_argument("--jsonl", required=True)
    w.add_argument("--command", required=True)
    w.add_argument("--out", required=True)
    x = sub.add_parser("crossover")
    x.add_argument("--jsonl", required=True)
    x.add_argument("--command", required=True)
    x.add_argument("--out", required=True)
    args = ap.parse_args(argv)

    if args.cmd == "crossover":
        recs = [json.loads(l) for l in open(args.jsonl) if l.startswith("{")]
        out = ["# Estimator against dense exact ALiBi over n (`bench.py --crossover`)", "",
               "Mistral shape: B = 1, H = 32 / H_kv = 8, d = 128, causal, s = 20, sigma_h = 2^(h/4). "
               "`estimator` is one `plsh_alibi_attention` call (pre-pass + kernel), tables resident; "
               "`exact` is one `plsh_exact_alibi_attention` call; TFLOP/s counts the dense causal "
               "work (4 d flops per visited pair) over the exact kernel's time. `torch SDPA flash` is "
               "torch.nn.functional.scaled_dot_product_attention forced to its flash backend, causal, "
               "without any bias: a lower bound on what dense exact attention costs on this stack.",
               "", "Command:", "", "```",
               args.command, "```", "",
               "| n | estimator call (ms) | estimator kernel (ms) | exact call (ms) | exact TFLOP/s | exact / estimator "
               "| torch SDPA flash, no bias (ms) | its TFLOP/s |",
               "|---|---|---|---|---|---|---|---|"]
        for r in recs:
            fa = r.get("torch_sdpa_flash_no_bias_ms")
            out.append(f"| {r['n']} | {r['lsh_call_ms']:.3f} | {r['lsh_attention_kernel_ms']:.3f} | "
                       f"{r['exact_ms']:.3f} | {r['exact_tflops']:.0f} | {r['exact_over_lsh']:.2f} | "
                       f"{'n/a' if fa is None else format(fa, '.3f')} | "
                       f"{'n/a' if fa is None else format(r['torch_sdpa_flash_tflops'], '.0f')} |")
        out += ["", "The JSON lines:", "", "```"] + [json.dumps(r) for r in recs] + ["```", ""]
        open(args.out, "w").write("\n".join(out))
        print("\n".join(out[:20]))
        return

    if args.cmd == "sweep":
        recs = [json.loads(l) for l in open(args.jsonl) if l.startswith("{")]
        out = ["# Every workload on one MI355X (`bench.py --sweep`)", "", "Command:", "", "```",
               args.command, "```", "",
               "| workload | s | call (ms) | kernel (ms) | warm median / min kernel (ms) | query-rows*samples/s "
               "| HBM frac (kernel) | useful TFLOP/s (kernel) | % of attainable | rel. error vs exact "
               "| backward from saved forward (ms) | graph-replayed call (ms) |",
               "|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for r in recs:
            rf = r.get("roofline") or {}
            wm = r.get("warm") or {}
            err = r.get("error_vs_exact_alibi")
            bw = r.get("backward")
            att = rf.get("attainable_useful_tflops")
            frac_att = (100.0 * rf["useful_tflops_in_kernel"] / att) if att else float("nan")
            out.append(f"| {r['workload']} | {r['s']} | {r['ms_per_call']:.4f} | {r['kernel_ms']:.4f} | "
                       f"{wm.get('kernel_ms_median', float('nan')):.4f} / {wm.get('kernel_ms_min', float('nan')):.4f} | "
                       f"{r['rows_samples_per_s']:.3g} | {r['hbm_frac_kernel']:.3f} | "
                       f"{rf.get('useful_tflops_in_kernel', float('nan')):.0f} | {frac_att:.1f} | "
                       f"{'n/a' if err is None else format(err['rel_fro'], '.3f')} | "
                       f"{'n/a' if bw is None else format(bw['saved_forward_backward_ms'], '.3f')} | "
                       f"{'n/a' if r.get('graph_replay_ms_per_call') is None else format(r['graph_replay_ms_per_call'], '.4f')} |")
        shas = sorted({r.get("kernel_sha", "?") for r in recs})
        out += ["", f"Forward kernel source sha256[:16]: {', '.join(shas)}.", "", "The JSON lines:", "", "```"]
        out += [json.dumps(r) for r in recs] + ["```", ""]
        open(args.out, "w").write("\n".join(out))
        print("\n".join(out[:20]))
        return

    if args.cmd == "mfma":
        mops, nd = counter_per_dispatch(args.run, "SQ_INSTS_VALU_MFMA_MOPS_BF16", args.kernel)
        busy, _ = counter_per_dispatch(args.run, "SQ_VALU_MFMA_BUSY_CYCLES", args.kernel)
        flops = mops * 512.0
        want = args.issued_pairs * args.flops_per_pair
        rec = {"kernel": args.kernel, "kernel_sha": args.kernel_sha, "dispatches": nd,
               "mops_bf16_per_dispatch": mops, "flops_per_mop": 512,
               "bf16_flops_per_launch": flops, "issued_pair_flops_per_launch": want,
               "mfma_busy_cycles_per_dispatch": busy}
        try:
            allrec = json.load(open(args.out_json))
        except (OSError, ValueError):
            allrec = {}
        allrec[args.workload] = rec
        json.dump(allrec, open(args.out_json, "w"), indent=1, sort_keys=True)
        md = (f"# bf16 matrix-core work of `{args.kernel}` on {args.workload}\n\n"
              f"Command:\n\n```\n{args.command}\n```\n\n"
              f"| quantity | value |\n|---|---|\n"
              f"| SQ_INSTS_VALU_MFMA_MOPS_BF16 per dispatch | {mops:.0f} ({nd} dispatches) |\n"
              f"| bf16 MFMA flops per launch (512 per MOP) | {flops / 1e9:.3f} GFLOP |\n"
              f"| pairs issued by construction x {args.flops_per_pair:.0f} flops | {want / 1e9:.3f} GFLOP |\n"
              f"| SQ_VALU_MFMA_BUSY_CYCLES per dispatch | {busy:.0f} |\n"
              f"| kernel source sha256[:16] | `{args.kernel_sha}` |\n")
        open(args.out_md, "w").write(md)
        print(md)
        return

    if args.cmd == "stats":
        path = _one(args.csv)
        md = f"# {args.title}\n\n" + kernel_stats_md(path, args.command)
        open(args.out, "w").write(md)
        print(md)
        return

    fetch_kib, nf = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    write_kib, nw = counter_per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    cf_kib, ncf = counter_per_dispatch(args.calib_fetch, "FETCH_SIZE", args.calib_kernel, largest=True)
    cw_kib, ncw = counter_per_dispatch(args.calib_write, "WRITE_SIZE", args.calib_kernel, largest=True)
    f_fetch = args.calib_bytes / (cf_kib * 1024.0)
    f_write = args.calib_bytes / (cw_kib * 1024.0)
    read_b = fetch_kib * 1024.0 * f_fetch
    write_b = write_kib * 1024.0 * f_write
    total = read_b + write_b
    rec = {"kernel": args.kernel, "kernel_sha": args.kernel_sha,
           "bytes_per_launch": total, "read_bytes": read_b, "write_bytes": write_b,
           "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
           "dispatches": [nf, nw],
           "calibration": {"bytes": args.calib_bytes, "fetch_kib": cf_kib, "write_kib": cw_kib,
                           "fetch_scale": f_fetch, "write_scale": f_write},
           "algorithmic_bytes": args.algorithmic_bytes,
           "traffic_over_algorithmic": total / args.algorithmic_bytes}
    try:
        allrec = json.load(open(args.out_json))
    except (OSError, ValueError):
        allrec = {}
    allrec[args.workload] = rec
    json.dump(allrec, open(args.out_json, "w"), indent=1, sort_keys=True)
    cmds = open(args.commands).read().strip()
    md = (f"# HBM traffic of `{args.kernel}` on {args.workload}\n\n"
          f"Commands (FETCH_SIZE and WRITE_SIZE passes of the benchmark, then of the copy "
          f"calibration):\n\n```\n{cmds}\n```\n\n"
          f"| quantity | value |\n|---|---|\n"
          f"| FETCH_SIZE per dispatch (KiB) | {fetch_kib:.1f} ({nf} dispatches) |\n"
          f"| WRITE_SIZE per dispatch (KiB) | {write_kib:.1f} ({nw} dispatches) |\n"
          f"| copy of {args.calib_bytes} B: FETCH_SIZE / WRITE_SIZE (KiB) | {cf_kib:.1f} / {cw_kib:.1f} |\n"
          f"| scale factors (fetch, write) | {f_fetch:.4f}, {f_write:.4f} |\n"
          f"| HBM bytes read / written per launch | {read_b / 1e6:.2f} MB / {write_b / 1e6:.2f} MB |\n"
          f"| traffic per launch | {total / 1e6:.2f} MB |\n"
          f"| algorithmic bytes per launch | {args.algorithmic_bytes / 1e6:.2f} MB |\n"
          f"| traffic / algorithmic | {total / args.algorithmic_bytes:.3f} |\n"
          f"| kernel source sha256[:16] | `{args.kernel_sha}` |\n")
    open(args.out_md, "w").write(md)
    print(md)


if __name__ == "__main__":
    main()
