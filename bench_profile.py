"""rocprofv3 summaries of the benchmark, written under profiles/.

    python bench_profile.py run        [--out DIR]   # on the GPU machine (default prof_out/)
    python bench_profile.py summarize  [--out DIR]   # anywhere, from run's CSVs

Runs bench.py (no CPU baseline, ending with one plain 1 GiB device copy) as a
child process under rocprofv3, once per pass. Counters are never combined
with tracing:
  1. --kernel-trace --stats                    per-kernel calls and durations
  2. --pmc FETCH_SIZE                          HBM read KiB per dispatch
  3. --pmc WRITE_SIZE                          HBM write KiB per dispatch
  4. --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA   MFMA work per dispatch
  5. --kernel-trace --stats of bench.py --rows-only     the per-row kernels on their workloads
  6-8. --kernel-trace --stats, --pmc FETCH_SIZE, --pmc WRITE_SIZE of
       bench.py --mtp-only: the 1 + 3 token fused decode step on its own (its
       kernel is the single-token step's, so it needs runs of its own)
  9. --pmc TCP_TCC_READ_REQ_sum TCC_HIT_sum TCC_MISS_sum   L2 -> L1 read requests
       (bytes per request from the copy, which reads each byte once) and L2 hits
The copy gives the calibration factors: true bytes / counter reading for a
copy of known size, applied to every kernel's reading.

Writes
  profiles/bench_prefill_t8k_decode_256seq_kernel_stats.md
  profiles/hbm_traffic_prefill_t8k_decode_256seq.md   (its traffic_json line is
      read by bench.py, with the hash of the kernel sources it was taken on)
  profiles/rows_long_prefill_t256k_decode_256seq_kernel_stats.md
(the 1 + 3 token step's figures go into the traffic summary)
This process itself never touches the GPU.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (top level imports no GPU library)

BENCH_ARGS = ["--steps", "200", "--warmup", "100", "--skip-cpu-baseline", "--skip-mtp", "--skip-rows",
              "--calibrate-copy"]
COPY_BYTES = 1 << 30
KERNELS = {  # what one call of each measured entry point launches (bf16 in, fp32 out); the
    # chunk table kernel runs only with cu_seqlens, so it is counted when present
    "chunk": ["chunk_offsets_kernel?", "chunk_prep_kernel<unsigned short, 1, false, false>",
              "chunk_state_bf16_kernel<float, false, false>"],
    "recurrent": ["recurrent_kernel<unsigned short, float"],
    "fused": ["decode_fused_kernel<unsigned short, float"],
}
MTP_ARGS = ["--steps", "200", "--warmup", "100", "--mtp-only", "--calibrate-copy"]


def launched(table, names):
    return [k.rstrip("?") for k in names if not k.endswith("?") or any(k.rstrip("?") in n for n in table)]


PASSES = [  # name, rocprofv3 arguments
    ("ktrace", ["--kernel-trace", "--stats"]),
    ("fetch", ["--pmc", "FETCH_SIZE"]),
    ("write", ["--pmc", "WRITE_SIZE"]),
    ("mfma", ["--pmc", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA"]),
    ("rows", ["--kernel-trace", "--stats"]),     # bench.py --rows-only
    ("mtp_ktrace", ["--kernel-trace", "--stats"]),   # bench.py --mtp-only
    ("mtp_fetch", ["--pmc", "FETCH_SIZE"]),
    ("mtp_write", ["--pmc", "WRITE_SIZE"]),
    ("l2l1", ["--pmc", "TCP_TCC_READ_REQ_sum", "TCC_HIT_sum", "TCC_MISS_sum"]),   # L2 -> L1 reads, L2 hits
]
ROWS_SUMMARY = os.path.join(ROOT, "profiles", "rows_long_prefill_t256k_decode_256seq_kernel_stats.md")


def bench_args(name):
    return ["--rows-only"] if name == "rows" else MTP_ARGS if name.startswith("mtp") else BENCH_ARGS


def pass_command(name, prof_args):
    return " ".join(["rocprofv3", *prof_args, "-f", "csv", "-d", f"<out>/{name}", "-o", name, "--",
                     "python3", "bench.py", *bench_args(name)])


def run_pass(out, name, prof_args, timeout):
    d = os.path.join(out, name)
    cmd = ["rocprofv3", *prof_args, "-f", "csv", "-d", d, "-o", name, "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_args(name)]
    print("[pass]", name, " ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=timeout)
    with open(os.path.join(out, name + ".log"), "w") as fh:
        fh.write(r.stdout + r.stderr)
    if not [l for l in r.stdout.splitlines() if l.startswith("{")]:
        raise RuntimeError(f"pass {name}: bench.py printed no result (rc={r.returncode}); see {name}.log")


def bench_line(out, name):
    with open(os.path.join(out, name + ".log")) as fh:
        return json.loads([l for l in fh.read().splitlines() if l.startswith("{")][-1])


def kernel_stats(d):
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0]
    return list(csv.DictReader(open(f)))


def counters(d):
    """{kernel name: {counter: [value per dispatch]}}"""
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def pick(table, key):
    hits = [n for n in table if key in n]
    if len(hits) != 1:
        raise RuntimeError(f"kernel {key!r}: {len(hits)} matches in the profile")
    return hits[0]


def avg(v):
    return sum(v) / len(v)


def summarize_rows(out):
    """Kernel trace of the per-row measurements: each row kernel launched on its own workload."""
    d = os.path.join(out, "rows")
    b = bench_line(out, "rows")["rows"]
    ks = kernel_stats(d)
    by_name = {r["Name"]: r for r in ks}
    lines = ["# Kernel trace: the per-row kernels on their own workloads (bench.py --rows-only)", "",
             "Long prefill T=262144 (16->64 heads, conv_dim 12288, bf16) for the conv, gating, chunk and",
             "gated RMSNorm; the 256-sequence decode batch for the conv update. Command (from /tmp,",
             "TMPDIR=/tmp; `python bench_profile.py run`, summarised by `python bench_profile.py summarize`):", "",
             "    " + pass_command("rows", dict(PASSES)["rows"]), "",
             "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in sorted(ks, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines += ["", "Agreement with the HIP-event figures bench.py printed in the same run:", ""]
    for row, key in (("causal_conv1d", "causal_conv1d_kernel"), ("gating", "gating_kernel"),
                     ("gated_rmsnorm", "gated_rmsnorm_kernel"), ("causal_conv1d_update", "conv_update")):
        names = [n for n in by_name if key in n]
        avg_us = sum(float(by_name[n]["TotalDurationNs"]) for n in names) / max(1, sum(int(by_name[n]["Calls"]) for n in names)) / 1e3
        kn = sorted({re.search(r"(\w+)<", n).group(1) for n in names})
        lines.append(f"- {row}: trace average {avg_us:.1f} us over {', '.join(kn)}"
                     f" (all its launches in the run); events {b[row]['avg_ms'] * 1e3:.1f} us, "
                     f"{b[row]['achieved']:.0f} GB/s = {100 * b[row]['frac']:.1f} % of HBM peak")
    for key in ("chunk_fwd", "chunk_fwd_varlen"):
        c = b[key]
        lines.append(f"- {key}: events {c['avg_ms'] * 1e3:.1f} us per call, {c['achieved']:.1f} TFLOP/s algorithmic "
                     f"({100 * c['frac']:.2f} % of the bf16 MFMA peak), {c['tokens_per_s'] / 1e6:.2f} M tokens/s")
    lines += ["", "bench.py line of this run:", "", "    " + json.dumps({"rows": b}), ""]
    with open(ROWS_SUMMARY, "w") as fh:
        fh.write("\n".join(lines))
    print("[profile] wrote", ROWS_SUMMARY, flush=True)


def l2l1_lines(out):
    """L2 -> L1 read traffic of the chunk call's kernels (the operand stream of the state kernel)."""
    d = os.path.join(out, "l2l1")
    if not os.path.isdir(d):
        return []
    c = counters(d)
    copy_req = max(c[pick(c, "copyBuffer")]["TCP_TCC_READ_REQ_sum"])
    bpr = COPY_BYTES / copy_req
    lines = ["L2 -> L1 reads of the chunk call (one run: " + pass_command("l2l1", dict(PASSES)["l2l1"]) + "); the",
             f"1 GiB copy made {copy_req:.0f} read requests, {bpr:.1f} bytes each:", "",
             "| kernel | L2 -> L1 read requests | L2 -> L1 bytes | L2 hit rate |", "|---|---|---|---|"]
    for k in launched(c, KERNELS["chunk"]):
        r = c[pick(c, k)]
        req, hit, miss = avg(r["TCP_TCC_READ_REQ_sum"]), avg(r["TCC_HIT_sum"]), avg(r["TCC_MISS_sum"])
        lines.append(f"| `{k}` | {req:.3e} | {req * bpr / 1e6:.1f} MB | {100 * hit / max(1.0, hit + miss):.1f} % |")
    return lines + [""]


def summarize(out):
    d1, d2, d3, d4 = (os.path.join(out, n) for n, _ in PASSES[:4])
    cmd1, cmd2, cmd3, cmd4 = (pass_command(n, a) for n, a in PASSES[:4])
    b1 = bench_line(out, "ktrace")

    # ---- kernel trace
    ks = kernel_stats(d1)
    by_name = {r["Name"]: r for r in ks}
    lines = ["# Kernel trace: bench.py, prefill T=8192 (16->32 heads, bf16) and decode 256 seqs (separate and fused)", "",
             "Command (from /tmp, TMPDIR=/tmp; written by `python bench_profile.py run`, summarised by",
             "`python bench_profile.py summarize`):", "", "    " + cmd1, "",
             "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in sorted(ks, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    chunk_names = launched(by_name, KERNELS["chunk"])
    chunk_sum = sum(float(by_name[pick(by_name, k)]["AverageNs"]) for k in chunk_names) / 1e3
    rec_avg = float(by_name[pick(by_name, KERNELS["recurrent"][0])]["AverageNs"]) / 1e3
    fus_avg = float(by_name[pick(by_name, KERNELS["fused"][0])]["AverageNs"]) / 1e3
    lines += ["", "Agreement with the HIP-event figures bench.py printed in the same run:", "",
              f"- gdn_chunk_fwd_gated = {' + '.join(k.split('<')[0] for k in chunk_names)}: sum of averages {chunk_sum:.1f} us; "
              f"events {b1['roofline']['avg_ms'] * 1e3:.1f} us per call",
              f"- recurrent_kernel: average {rec_avg:.1f} us; events {b1['decode']['roofline']['avg_ms'] * 1e3:.1f} us",
              f"- decode_fused_kernel: average {fus_avg:.1f} us; events "
              f"{b1['decode_fused']['roofline']['avg_ms'] * 1e3:.1f} us",
              "", "bench.py line of this run:", "", "    " + json.dumps(b1), ""]
    with open(os.path.join(ROOT, "profiles", "bench_prefill_t8k_decode_256seq_kernel_stats.md"), "w") as fh:
        fh.write("\n".join(lines))

    # ---- traffic and MFMA counters
    cf, cw, cm = counters(d2), counters(d3), counters(d4)
    copy_f = max(cf[pick(cf, "copyBuffer")]["FETCH_SIZE"])
    copy_w = max(cw[pick(cw, "copyBuffer")]["WRITE_SIZE"])
    kf, kw = COPY_BYTES / 1024 / copy_f, COPY_BYTES / 1024 / copy_w
    rec = {}
    rows = ["| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read bytes | write bytes | MFMA ops (x512 flop) |",
            "|---|---|---|---|---|---|"]
    for part, names in KERNELS.items():
        total = 0.0
        flops = 0.0
        for k in launched(cf, names):
            f_kib = avg(cf[pick(cf, k)]["FETCH_SIZE"])
            w_kib = avg(cw[pick(cw, k)]["WRITE_SIZE"])
            mops = avg(cm[pick(cm, k)]["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
            rb, wb = f_kib * 1024 * kf, w_kib * 1024 * kw
            total += rb + wb
            flops += mops * 512
            rows.append(f"| `{k}` | {f_kib:.1f} | {w_kib:.1f} | {rb / 1e6:.1f} MB | {wb / 1e6:.1f} MB | {mops:.3e} |")
        rec[part] = dict(bytes_per_call=round(total), mfma_flops_per_call=flops, source_hash=bench.source_hash(part))
    # the 1 + 3 token step, from its own runs (calibrated by their own copy)
    mf, mw = counters(os.path.join(out, "mtp_fetch")), counters(os.path.join(out, "mtp_write"))
    mkf = COPY_BYTES / 1024 / max(mf[pick(mf, "copyBuffer")]["FETCH_SIZE"])
    mkw = COPY_BYTES / 1024 / max(mw[pick(mw, "copyBuffer")]["WRITE_SIZE"])
    k = KERNELS["fused"][0]
    f_kib, w_kib = avg(mf[pick(mf, k)]["FETCH_SIZE"]), avg(mw[pick(mw, k)]["WRITE_SIZE"])
    rb, wb = f_kib * 1024 * mkf, w_kib * 1024 * mkw
    rows.append(f"| `{k}` (1 + 3 tokens) | {f_kib:.1f} | {w_kib:.1f} | {rb / 1e6:.1f} MB | {wb / 1e6:.1f} MB | 0 |")
    rec["mtp"] = dict(bytes_per_call=round(rb + wb), mfma_flops_per_call=0.0, source_hash=bench.source_hash("mtp"))
    mks = {r["Name"]: r for r in kernel_stats(os.path.join(out, "mtp_ktrace"))}
    mtp_avg = float(mks[pick(mks, k)]["AverageNs"]) / 1e3
    bm = bench_line(out, "mtp_ktrace")["decode_mtp_fused"]
    cmd_m = [pass_command(n, a) for n, a in PASSES if n.startswith("mtp")]
    lines = ["# HBM traffic and MFMA work per call: prefill T=8192 (bf16, 16->32 heads) and decode 256 seqs", "",
             "Commands (from /tmp, TMPDIR=/tmp), one counter set per run:", "",
             "    " + cmd2, "    " + cmd3, "    " + cmd4, *["    " + c for c in cmd_m[1:]], "",
             "Calibration on the plain 1 GiB device copy (`copyBuffer`) in the same runs:", "",
             f"- FETCH_SIZE read {copy_f:.1f} KiB for {COPY_BYTES // 1024} KiB: read bytes = {kf:.4f} x 1024 x FETCH_SIZE",
             f"- WRITE_SIZE read {copy_w:.1f} KiB for {COPY_BYTES // 1024} KiB: write bytes = {kw:.4f} x 1024 x WRITE_SIZE",
             "", *rows, "",
             f"- gdn_chunk_fwd_gated (all its launches): {rec['chunk']['bytes_per_call'] / 1e6:.1f} MB per call "
             f"(algorithmic {bench.chunk_bytes(8192, 16, 32, gate_bytes=4) / 1e6:.1f} MB); MFMA work "
             f"{rec['chunk']['mfma_flops_per_call'] / 1e9:.2f} GFLOP executed (hi/lo passes included) vs "
             f"{bench.chunk_flops_per_token_head() * 8192 * 32 / 1e9:.2f} GFLOP algorithmic",
             f"- recurrent_kernel: {rec['recurrent']['bytes_per_call'] / 1e6:.1f} MB per call "
             f"(algorithmic {bench.recurrent_bytes(256, 16, 32) / 1e6:.1f} MB)",
             f"- decode_fused_kernel: {rec['fused']['bytes_per_call'] / 1e6:.1f} MB per call "
             f"(algorithmic {bench.fused_decode_bytes(256, 256, 16, 32) / 1e6:.1f} MB)",
             f"- decode_fused_kernel, 1 + 3 tokens per sequence: {rec['mtp']['bytes_per_call'] / 1e6:.1f} MB per call "
             f"(algorithmic {bench.fused_decode_bytes(1024, 256, 16, 32) / 1e6:.1f} MB); kernel trace average "
             f"{mtp_avg:.1f} us ({cmd_m[0]}), events {bm['roofline']['avg_ms'] * 1e3:.1f} us, "
             f"{100 * bm['roofline']['frac']:.1f} % of HBM peak", "",
             *l2l1_lines(out),
             "Source hashes are of the kernel sources the counters were taken on; bench.py reports traffic",
             "only while they match.", "",
             "traffic_json: " + json.dumps(rec), ""]
    with open(bench.TRAFFIC_SUMMARY, "w") as fh:
        fh.write("\n".join(lines))
    print("[profile] wrote", bench.TRAFFIC_SUMMARY, flush=True)
    summarize_rows(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["run", "summarize"])
    ap.add_argument("--out", default=os.path.join(ROOT, "prof_out"))
    ap.add_argument("--timeout", type=int, default=240)
    args = ap.parse_args()
    if args.mode == "run":
        os.makedirs(args.out, exist_ok=True)
        for name, prof_args in PASSES:
            run_pass(args.out, name, prof_args, args.timeout)
        print("[profile] passes done in", args.out, flush=True)
    else:
        summarize(args.out)


if __name__ == "__main__":
    main()
