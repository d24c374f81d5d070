"""Benchmark of one TiDAR decode step on one MI355X.

A step is the whole hot path over one batch: structured-mask step attention
(one layer), greedy verification with next-draft selection, and the KV
commit / evict.  The workload is the 8B-shaped step (batch 16, 32 query / 8
KV heads of 128, settled prefix 4096, k = 8 candidates + 64 draft slots,
verify over a 128256-entry vocabulary with planted accept lengths U{0..8}),
bf16, synthetic seeded inputs already resident in HBM.

Timing: W untimed warmup steps, then K steps between HIP events on the
launch stream (step_us), and the same K steps replayed from HIP graphs
(step_us_graph).  Inputs rotate over replicas totalling >= 2 GB so the 256 MB
Infinity Cache cannot serve them warm.  After each step the settled lengths
are restored (a 64-byte device copy) so every step is the same workload.
The attention calls alone, and the verify + commit calls alone, are then
timed as K calls in a row queued behind a spin kernel, so the host has
enqueued them all before the GPU starts, and after 40 ms of untimed calls of
the same work: the part boosts its clock after an idle spell and its power
controller clamps it a few ms later, so the timed calls run at the clock it
settles at under continuous load, as in a serving loop (--clock-trace shows
the transient; the *_after_idle keys time the same calls straight after the
spin).  One event pair around the K calls gives the GPU time per call (the
value and the roofline figure; it agrees with the kernel's rocprofv3
durations for the calls made that far into a run, which each trace summary
lists), an event pair around each call gives p50/p99.

Prints ONE JSON line.  Options:
  --gpus N          only N = 1 is supported (one GPU per process, no collectives)
  --steps K --warmup W
  --no-cpu-baseline skip the oracle timing (for profiler runs)
  --paged           settled keys/values in shared 64-position page pools under
                    a shuffled block table (tidar_step_attention_paged and
                    tidar_kv_commit_paged) instead of per-sequence caches
  --verify lmhead   the LM head fused with greedy verification: hidden states
                    and a random-init head of the workload's model size in,
                    no logits stored (tidar_lmhead_verify_greedy_packed on
                    the head packed before timing; --lm-layout rowmajor for
                    tidar_lmhead_verify_greedy on the [V][d] head)
  --verify sample   stochastic verification (temperature --temperature, Philox
                    stream of --seed and the step number) in place of greedy;
                    inputs from the sampling generator, accept lengths as drawn
  --loop N          the serving loop: N consecutive steps on one cache whose
                    lengths the commit advances in place (no restore); per-step
                    p50/p99 and mean GB/s as the lengths grow (e.g. with
                    --workload ragged_8b --loop 256)
  --clock-trace N   print the attention time of N back-to-back calls after an
                    idle spell, per 10 calls, in call order, then exit
  --workload NAME   step_8b (default), step_1p5b, step_8b_long, ragged_8b,
                    train_8b (the training-mask attention alone)
  --calibrate-copy  run only a plain device copy of known size (for scaling
                    the FETCH_SIZE / WRITE_SIZE counters)
  --summarize DIR   turn rocprofv3 outputs under DIR (kt/, pmc_FETCH_SIZE/,
                    pmc_WRITE_SIZE/, pmc_copy_FETCH_SIZE/, pmc_copy_WRITE_SIZE/)
                    into the summaries kept under profiles/
  --summarize-lmhead DIR  the same for the fused LM head's FETCH_SIZE /
                    WRITE_SIZE runs (pmc_FETCH_SIZE/, pmc_WRITE_SIZE/ of
                    --verify lmhead); its bench line then carries the traffic
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

SUSTAIN_MS = 40.0         # untimed load before the queued timed calls (the clock settles after ~30 ms)
MAX_SUSTAIN_CALLS = 5000
HOST_US_PER_CALL = 60.0   # the host's enqueue time per call, generously: sizes the spin that gives it a head start
METRIC = "KV-cache GB/s and decode-step latency (µs) for TiDAR step attention, % of HBM peak"
HBM_PEAK_GBPS = 8000.0
COPY_CALIB_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_step_8b_traffic.txt")
ATTN_SOURCES = [os.path.join(ROOT, "diffusion_drafted_self_amd", "csrc", n)
                for n in ("attention.hip", "attention_pp.hip", "attn_tile.h", "check.h", "common.h", "launch.h", "lds_dma.h")]
LM_SOURCES = [os.path.join(ROOT, "diffusion_drafted_self_amd", "csrc", n)
              for n in ("lmhead.hip", "check.h", "common.h", "launch.h", "lds_dma.h")]
LM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_verify_8b_traffic.txt")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cold-bytes", type=float, default=2.0e9)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--kv-chunk", type=int, default=0, help="key positions per attention chunk (0: library plan)")
    p.add_argument("--summarize", metavar="DIR", help="write profiles/ summaries from rocprofv3 outputs in DIR")
    p.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "NAME"),
                   help="write profiles/NAME_kernel_trace.md from the kernel-trace run under DIR/kt")
    p.add_argument("--summarize-counters", metavar="DIR",
                   help="write the attention counter summary of --workload from the passes under DIR")
    p.add_argument("--counters-kernel", default="", help="TIDAR_ATTN_KERNEL value the counter runs used")
    p.add_argument("--summarize-lmhead", metavar="DIR",
                   help="write the fused LM head's traffic summary from FETCH_SIZE / WRITE_SIZE runs in DIR")
    p.add_argument("--verify", default="greedy", choices=["greedy", "sample", "lmhead"])
    p.add_argument("--lm-layout", default="packed", choices=["packed", "rowmajor"],
                   help="layout of W for --verify lmhead (packed once, before timing, as at weight load)")
    p.add_argument("--temperature", type=float, default=1.0)
    p.add_argument("--separate", action="store_true",
                   help="greedy verify and the commit as two calls (tidar_verify_greedy, tidar_kv_commit) "
                        "instead of the fused tidar_verify_commit_greedy")
    p.add_argument("--paged", action="store_true")
    p.add_argument("--loop", type=int, default=0, metavar="N",
                   help="serving loop: N consecutive steps on one cache whose lengths the commit advances in "
                        "place (no restore), per-step p50/p99 and mean GB/s as the lengths grow")
    p.add_argument("--clock-trace", type=int, default=0, metavar="N",
                   help="print the attention time of N back-to-back calls after an idle spell, per 10 calls, in "
                        "call order (how the part's clock moves with the time under load), then exit")
    p.add_argument("--workload", default="step_8b",
                   choices=["step_8b", "step_1p5b", "step_8b_long", "ragged_8b", "train_8b"],
                   help="synthetic workload (the reported line is the 8B-shaped step; ragged_8b is one step of "
                        "the serving loop's batch of 32 at its initial lengths; train_8b is the training-mask "
                        "attention over a duplicated sequence, 8B heads, 4 x 2 x 4096 positions, block 8)")
    p.add_argument("--compare", nargs="+", metavar="LIB",
                   help="paired timing of the workload's attention call across library builds (libtidar.so "
                        "first, then each LIB, e.g. a build of another revision): all are loaded in this "
                        "process and take turns, --steps calls each per round, over --rounds rounds in "
                        "rotating order after 0.3 s of sustaining calls, so every build runs at the same clock; "
                        "checks that every build's output equals the first's; one JSON line")
    p.add_argument("--rounds", type=int, default=40, help="rounds of --compare")
    p.add_argument("--probes", action="store_true",
                   help="only the matrix-core issue probe (tidar_mfma_probe): cycles per MFMA with one and two "
                        "waves per SIMD, operands in registers or read from LDS; one JSON line")
    p.add_argument("--compare-call", default="attention", choices=["attention", "verify_commit"],
                   help="the call --compare times: the step attention, or the fused greedy verify + commit "
                        "(with the 64-byte restore of the settled lengths after each call, as in the step)")
    return p.parse_args()


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace: a counter summary stays
    valid across edits that do not touch the code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def attention_source_sha() -> str:
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def _kv_file(path):
    kv = {}
    if os.path.exists(path):
        for line in open(path):
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    return kv


def read_traffic(path=None, sha=None, key="hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    kv = _kv_file(path or TRAFFIC_FILE)
    if kv.get("kernel_source_sha") != (sha or attention_source_sha)():
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def lmhead_source_sha() -> str:
    h = hashlib.sha256()
    for f in LM_SOURCES:
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def summarize_lmhead(dirname):
    """HBM traffic of the fused LM head (packed W, 8B-shaped step) from
    FETCH_SIZE / WRITE_SIZE runs under dirname; written under profiles/."""
    import statistics
    cal = _kv_file(TRAFFIC_FILE)
    f_fetch, f_write = float(cal["copy_scale_fetch"]), float(cal["copy_scale_write"])
    out = ["# HBM traffic of the fused LM head + greedy verify, packed W, 8B-shaped step (rocprofv3 counters)",
           "# Commands (from the repository root, MI355X), one counter per run:",
           "#   rocprofv3 --pmc FETCH_SIZE -d DIR/pmc_FETCH_SIZE -o p --output-format csv -- "
           "python3 bench.py --verify lmhead --steps 3 --warmup 1 --no-cpu-baseline",
           "#   rocprofv3 --pmc WRITE_SIZE -d DIR/pmc_WRITE_SIZE -o p --output-format csv -- "
           "python3 bench.py --verify lmhead --steps 3 --warmup 1 --no-cpu-baseline",
           "# Counter values are KiB per dispatch, scaled by the plain-copy factors of the attention traffic",
           "# summary (the same counters on a 1 GiB device copy).",
           f"copy_scale_fetch = {f_fetch:.4f}",
           f"copy_scale_write = {f_write:.4f}"]
    total = 0.0
    for mt, what in ((9, "ar_pass"), (7, "draft_pass")):
        key = f"lmhead_argmax_kernel<{mt}, true>"
        res = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [float(r["Counter_Value"]) for r in
                    _csv_rows(os.path.join(dirname, f"pmc_{counter}", "*counter_collection.csv"))
                    if key in r["Kernel_Name"]]
            res[counter] = statistics.mean(vals)
        hbm = res["FETCH_SIZE"] * 1024 * f_fetch + res["WRITE_SIZE"] * 1024 * f_write
        total += hbm
        out += [f"{what}_fetch_kib = {res['FETCH_SIZE']:.1f}", f"{what}_write_kib = {res['WRITE_SIZE']:.1f}",
                f"{what}_hbm_bytes = {hbm:.0f}"]
    out += [f"hbm_bytes_per_verify = {total:.0f}", f"kernel_source_sha = {lmhead_source_sha()}", ""]
    with open(LM_TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def step_bytes(shape, V, accept, verify_kind="greedy", d_model=0):
    """Algorithmic bytes of one step (each byte moved once).
    attention: settled K+V + step K+V + Q + O; greedy verify: (k+1) AR rows
    and k-1 draft rows of f32 logits; sampling verify: k AR and k proposal
    rows (softmax statistics), the k drawn rows, and the proposal row of the
    residual where a candidate was rejected; commit: accepted K/V rows read
    and written."""
    s = shape
    esz = 2
    kv_prefix = sum(s.lens) * s.Hkv * 2 * s.D * esz
    kv_step = s.B * s.R * s.Hkv * 2 * s.D * esz
    qo = 2 * s.B * s.R * s.Hq * s.D * esz
    attn = kv_prefix + kv_step + qo
    if verify_kind == "sample":
        verify = (s.B * 3 * s.k + sum(1 for a in accept if a < s.k)) * V * 4
    elif verify_kind == "lmhead":  # W read once per pass, plus the hidden rows of both passes
        verify = 2 * V * d_model * 2 + s.B * 2 * s.k * d_model * 2
    else:
        verify = s.B * (2 * s.k) * V * 4
    commit = int(sum(accept)) * s.Hkv * s.D * esz * 2 * 2
    flops = 4 * s.D * s.Hq * sum(s.R * L for L in s.lens)
    return attn, verify, commit, kv_prefix + kv_step, flops


def attention_roofline(attn_bytes, attn_flops, attn_ms, traffic):
    """Roofline entry of the step-attention kernel: against HBM when its
    arithmetic intensity (flops per algorithmic byte) is below the ridge of
    the dense bf16 MFMA peak over the HBM peak (2500 TFLOP/s / 8 TB/s =
    312.5 flop/B), against the MFMA peak above it."""
    ai = attn_flops / attn_bytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    gbps = attn_bytes / (attn_ms * 1e-3) / 1e9
    tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    common = {"kernel": "tidar_step_attention", "traffic": traffic, "algorithmic_bytes": int(attn_bytes),
              "algorithmic_flops": int(attn_flops), "arithmetic_intensity": round(ai, 1), "ridge": round(ridge, 1)}
    if ai > ridge:
        return dict(bound="mfma", achieved=round(tflops, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), **common)
    return dict(bound="hbm", achieved=round(gbps, 2), peak=HBM_PEAK_GBPS, unit="GB/s",
                frac=round(gbps / HBM_PEAK_GBPS, 4), **common)


def visible_step_pairs(k, n_groups):
    """Visible (row, step key) pairs of the step block: candidates k(k+1)/2,
    group g: k*(g+1) own-candidate + k*k own-group entries."""
    return k * (k + 1) // 2 + sum(k * (g + 1) + k * k for g in range(n_groups))


def calibrate_copy():
    import torch
    dev = torch.device("cuda:0")
    n = COPY_CALIB_BYTES // 2
    a = torch.ones(n, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_each_way": COPY_CALIB_BYTES, "launches": 5}))


def _csv_rows(pattern):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(pattern)):
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize(dirname):
    """Summaries of a profiling session (see the module docstring for the
    commands); written under profiles/: the 8B step's kernel trace (under
    dirname/kt) and the attention kernel's HBM traffic."""
    import statistics
    summarize_trace(dirname, "attention_step_8b")

    def per_dispatch(counter, kernel_key):
        vals = [float(r["Counter_Value"]) for r in _csv_rows(os.path.join(dirname, f"pmc_{counter}", "*counter_collection.csv"))
                if kernel_key in r["Kernel_Name"] and "merge" not in r["Kernel_Name"]]
        return statistics.mean(vals) if vals else None, len(vals)

    def copy_factor(counter):
        vals = [float(r["Counter_Value"]) for r in
                _csv_rows(os.path.join(dirname, f"pmc_copy_{counter}", "*counter_collection.csv"))
                if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536]
        return (COPY_CALIB_BYTES / 1024.0) / statistics.mean(vals)

    f_fetch, f_write = copy_factor("FETCH_SIZE"), copy_factor("WRITE_SIZE")
    fetch, nf = per_dispatch("FETCH_SIZE", "attn_")
    write, nw = per_dispatch("WRITE_SIZE", "attn_")
    hbm = fetch * 1024 * f_fetch + write * 1024 * f_write
    out = ["# HBM traffic of the step-attention kernel, 8B-shaped workload (rocprofv3 counters)",
           "# Commands (from the repository root, MI355X), one counter per run:",
           "#   rocprofv3 --pmc FETCH_SIZE -d DIR/pmc_FETCH_SIZE -o p --output-format csv -- "
           "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline",
           "#   rocprofv3 --pmc WRITE_SIZE -d DIR/pmc_WRITE_SIZE -o p --output-format csv -- "
           "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline",
           "#   the same two counters on: python3 bench.py --calibrate-copy  (1 GiB device copy)",
           "# Counter values are KiB per dispatch; each is scaled by (known bytes / counter) of the copy.",
           f"fetch_kib_per_launch = {fetch:.1f}",
           f"write_kib_per_launch = {write:.1f}",
           f"dispatches = {nf}",
           f"copy_scale_fetch = {f_fetch:.4f}",
           f"copy_scale_write = {f_write:.4f}",
           f"hbm_bytes_per_launch = {hbm:.0f}",
           f"kernel_source_sha = {attention_source_sha()}", ""]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


# Kernel-trace summaries kept under profiles/: name -> (title, bench
# arguments of the traced run, the workload, where the calls come from)
_STEP_CALLS = ("The step's kernels run in the warm-up and timed eager steps, once per input replica before its graph "
               "capture, in the graph replays (warm-up and timed), and in the queued runs of the attention calls "
               "alone and the verify + commit calls alone (each straight after an idle spin, and after 40 ms of "
               "untimed calls of the same work).")
TRACES = {
    "attention_step_8b": ("one TiDAR step on the 8B-shaped workload", "--steps 20 --warmup 5",
                          "B=16, 32/8 heads of 128, prefix 4096, k=8 (+64 draft slots), greedy verify over 128256 "
                          "entries with planted accept lengths, fused verify + commit.", _STEP_CALLS),
    "step_1p5b": ("one TiDAR step on the 1.5B-shaped workload", "--workload step_1p5b --steps 20 --warmup 5",
                  "B=8, 12/2 heads of 128, prefix 2048, k=4 (+16 draft slots), greedy verify over 151936 entries, "
                  "fused verify + commit.", _STEP_CALLS),
    "step_8b_long": ("one long-context TiDAR step, 8B heads", "--workload step_8b_long --steps 10 --warmup 3",
                     "B=4, 32/8 heads of 128, prefix 32768, k=16 (+256 draft slots), greedy verify over 128256 "
                     "entries, fused verify + commit.", _STEP_CALLS),
    "train_attention_8b": ("training-mask attention, 8B heads", "--workload train_8b --steps 10 --warmup 3",
                           "B=4, Hq=32, Hkv=8, D=128, N=4096 clean + 4096 masked positions (T=8192), block 8.",
                           "One call per warm-up and timed step (3 + 10)."),
    "verify_sample_step_8b": ("one TiDAR step with stochastic verification, 8B-shaped workload",
                              "--verify sample --steps 20 --warmup 5",
                              "the 8B step with the rejection-sampling verify at T=1 (inputs from the sampling "
                              "generator) and the separate commit.",
                              "Eager steps only (the draw counter is a launch argument, so nothing is replayed); "
                              "after the timed steps the verification runs once more per timed step to read the "
                              "accept lengths the bytes depend on."),
    "lmhead_verify_8b": ("one TiDAR step with the LM head fused into greedy verification, 8B-shaped workload",
                         "--verify lmhead --steps 10 --warmup 3",
                         "the 8B step with hidden states and a random-init head of d_model 4096 x 128256 packed "
                         "before timing; two passes over the head per step.",
                         "The step's kernels run in the warm-up and timed eager steps, once per input replica before "
                         "its graph capture, and in the graph replays (warm-up and timed)."),
    "attention_ragged_loop": ("the ragged serving loop, 256 steps",
                              "--workload ragged_8b --loop 256 --warmup 5",
                              "batch 32, 32/8 heads of 128, lengths drawn U{512..8192} and advanced in place by "
                              "each step's commit, k=8, greedy verify over 128256 entries.",
                              "5 ordinary warm-up steps (lengths restored), then the 256 loop steps."),
}


def attention_calls_by_load(dirname, gap_ns=20_000, sustained_ms=SUSTAIN_MS):
    """The attention kernel's calls of a kernel-trace run, grouped by how
    long the GPU had been running attention back to back when each started
    (a run: each call starting within gap_ns of the previous one's end).
    The bench times the calls at least sustained_ms into such a run."""
    rows = _csv_rows(os.path.join(dirname, "kt", "*kernel_trace.csv"))
    calls = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                   if "attn_" in r["Kernel_Name"] and "merge" not in r["Kernel_Name"])
    if not calls:
        return []
    groups = {"first 2 ms": [], f"2 to {sustained_ms:.0f} ms": [], f"{sustained_ms:.0f} ms on (what the bench times)": []}
    keys = list(groups)
    t_run = calls[0][0]
    prev_end = None
    for s_ns, e_ns in calls:
        if prev_end is not None and s_ns - prev_end >= gap_ns:
            t_run = s_ns
        into = (s_ns - t_run) / 1e6
        groups[keys[0] if into < 2 else keys[1] if into < sustained_ms else keys[2]].append((e_ns - s_ns) / 1e3)
        prev_end = e_ns
    out = ["", "Attention calls by time under load (the part's clock boosts after an idle spell, is clamped by "
           "its power controller a few ms later and settles after ~30 ms; a run is a sequence of attention calls "
           f"each starting within {gap_ns / 1e3:.0f} us of the previous one's end):", "",
           "| time into the run | calls | average us |", "|---|---|---|"]
    for k, v in groups.items():
        out.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} |" if v else f"| {k} | 0 | - |")
    return out


def summarize_trace(dirname, name):
    """profiles/<name>_kernel_trace.md from the kernel-trace run under
    dirname/kt (the command in TRACES[name])."""
    title, bench_args, what, calls = TRACES[name]
    cmd = (f"rocprofv3 --kernel-trace --stats -d DIR/kt -o kt --output-format csv -- python3 bench.py {bench_args} "
           "--no-cpu-baseline")
    lines = [f"# Kernel trace: {title}", "", f"Command (from the repository root, MI355X): `{cmd}`", "",
             f"Workload: {what}", "",
             "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in _csv_rows(os.path.join(dirname, "kt", "*kernel_stats.csv")):
        if "tidar" not in r["Name"] and "copyBuffer" not in r["Name"]:
            continue
        kname = r["Name"].replace("(anonymous namespace)::", "").replace("tidar::", "")
        lines.append(f"| `{kname[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    lines += attention_calls_by_load(dirname)
    lines += ["", calls + " `copyBuffer` is the settled lengths' 64-byte "
              "restore after each step and the replicas' set-up copies (harness). `read_probe_kernel` is the "
              "achievable-bandwidth measurement (a streaming read of 4 GiB, six calls). Other rows of the run "
              "(torch elementwise kernels) are the harness's input generation and checks.", ""]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{name}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


# Counter passes of the attention kernel (one rocprofv3 --pmc run each, at
# most 8 SQ counters and GRBM_GUI_ACTIVE per pass).
COUNTER_PASSES = {
    "busy": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CU_CYCLES",
             "GRBM_GUI_ACTIVE"],
    "insts": ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE"],
    "wait": ["SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "SQ_LDS_DATA_FIFO_FULL", "GRBM_GUI_ACTIVE"],
}
N_CU, N_XCD, N_SIMD = 256, 8, 4


def summarize_counters(dirname, workload, kernel_env):
    """Derived utilisation figures of the step-attention kernel from the
    counter passes under dirname/pmc_<pass>/; written under profiles/."""
    import statistics
    vals, durs = {}, []
    for pas, names in COUNTER_PASSES.items():
        for r in _csv_rows(os.path.join(dirname, f"pmc_{pas}", "*counter_collection.csv")):
            if "attn_" not in r["Kernel_Name"] or "merge" in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if pas == "busy" and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
            kname = r["Kernel_Name"]
    m = {k: statistics.mean(v) for k, v in vals.items()}
    gui = m["GRBM_GUI_ACTIVE"] / N_XCD  # cycles per XCD (the counter sums the XCDs)
    simd_cycles = gui * N_CU * N_SIMD
    dur_us = statistics.mean(durs) if durs else float("nan")
    mfma_busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles
    rows = [
        ("kernel", kname.replace("(anonymous namespace)::", "").split("(")[0]),
        ("dispatches averaged", len(durs)),
        ("duration under counters, us", f"{dur_us:.2f}"),
        ("GRBM_GUI_ACTIVE per XCD, cycles", f"{gui:.0f}"),
        ("shader clock over the dispatch, MHz (cycles / duration)", f"{gui / dur_us:.0f}"),
        ("MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x CUs x 4))", f"{100 * mfma_busy:.1f} %"),
        ("MFMA busy cycles with VALU co-issue (COEXEC / MFMA_BUSY)",
         f"{100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:.1f} %"),
        ("VALU active (SQ_ACTIVE_INST_VALU / (cycles x CUs))",
         f"{100 * m['SQ_ACTIVE_INST_VALU'] / (gui * N_CU):.1f} %"),
        ("CU busy (SQ_BUSY_CU_CYCLES x 4 / (cycles x CUs))", f"{100 * 4 * m['SQ_BUSY_CU_CYCLES'] / (gui * N_CU):.1f} %"),
        ("LDS active (SQ_LDS_IDX_ACTIVE / (cycles x CUs))", f"{100 * m['SQ_LDS_IDX_ACTIVE'] / (gui * N_CU):.1f} %"),
        ("LDS bank-conflict cycles / LDS active cycles",
         f"{100 * m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_LDS_IDX_ACTIVE'], 1):.2f} %"),
        ("wave-cycles waiting for LDS issue / wave cycles",
         f"{100 * 4 * m['SQ_WAIT_INST_LDS'] / max(m['SQ_WAVE_CYCLES'], 1):.1f} %"),
        ("wave-cycles waiting for any issue / wave cycles",
         f"{100 * 4 * m['SQ_WAIT_INST_ANY'] / max(m['SQ_WAVE_CYCLES'], 1):.1f} %"),
        ("LDS data FIFO full / (cycles x CUs)", f"{100 * m['SQ_LDS_DATA_FIFO_FULL'] / (gui * N_CU):.1f} %"),
        ("instructions per dispatch: VALU / MFMA / LDS",
         f"{m['SQ_INSTS_VALU']:.3e} / {m['SQ_INSTS_MFMA']:.3e} / {m['SQ_INSTS_LDS']:.3e}"),
        ("bf16 MFMA flops per dispatch (MOPS x 512)", f"{m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4e}"),
    ]
    cmd = (f"{'TIDAR_ATTN_KERNEL=' + kernel_env + ' ' if kernel_env else ''}rocprofv3 --pmc <pass counters> "
           f"-d DIR/pmc_<pass> -o p --output-format csv -- python3 bench.py --workload {workload} "
           "--steps 3 --warmup 1 --no-cpu-baseline")
    lines = [f"# Counters of the step-attention kernel, workload {workload}"
             + (f" (TIDAR_ATTN_KERNEL={kernel_env})" if kernel_env else " (library plan)"), "",
             f"Command (from the repository root, MI355X), one run per pass: `{cmd}`", "",
             "Passes: " + "; ".join(f"`{p}`: {', '.join(c)}" for p, c in COUNTER_PASSES.items()), "",
             "| figure | value |", "|---|---|"] + [f"| {a} | {b} |" for a, b in rows] + [
             "", "Raw means per dispatch:", ""] + [f"- {k} = {v:.6g}" for k, v in sorted(m.items())] + [
             "", f"kernel_source_sha = {attention_source_sha()}", ""]
    tag = workload + (f"_{kernel_env}" if kernel_env else "")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"attention_{tag}_counters.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def clock_trace(N, name, reps, n_rep, attention, torch, stream):
    """N attention calls back to back on the rotating replicas after a ~20 ms
    idle spin, an event between consecutive calls; prints the mean time per
    call of each group of 10 against the time since the first call."""
    for i in range(5):
        attention(reps[i % n_rep])
    print(f"# attention per call on {name}, back to back after an idle spin (mean of each 10 calls)")
    for trial in range(2):
        torch.cuda.synchronize()
        torch.cuda._sleep(40_000_000)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(N + 1)]
        ev[0].record(stream)
        for i in range(N):
            attention(reps[i % n_rep])
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        d = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(N)]
        print(f"trial {trial}: | ms since the first call | us per call |")
        t = 0.0
        for i in range(0, N, 10):
            grp = d[i:i + 10]
            print(f"| {t / 1e3:.1f} | {sum(grp) / len(grp):.1f} |")
            t += sum(grp)
        sys.stdout.flush()


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the oracle baseline."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, d, v, a_planted, args):
    """The oracle (as it stands) on the same workload: three full steps."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle
    import workloads as W

    cores = len(os.sched_getaffinity(0))
    s = wl.attn
    f = {n: W.to_f32(x, "bf16") for n, x in d.items() if n != "lens"}
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1) if threadpool_limits else cores
        # warm-up on one sequence
        oracle.attention_ref(f["q"], f["k_step"], f["v_step"], f["k_cache"], f["v_cache"], d["lens"], s.k,
                             s.n_groups, s.sm_scale, pairs=[(0, h) for h in range(s.Hq)])
        n_steps = 3
        lm_seconds = 0.0
        if args.verify == "lmhead":
            # the head's oracle is a V x d float64 product per row: two
            # sequences timed, scaled to the batch
            wf = W.bf16_to_f32(v["w"])
            t_lm = time.perf_counter()
            oracle.lmhead_verify_ref(W.bf16_to_f32(v["h_ar"][:2]), W.bf16_to_f32(v["h_draft"][:2]), wf,
                                     v["cand"][:2])
            lm_seconds = (time.perf_counter() - t_lm) * s.B / 2
            lm_acc = v["planted"]
        t0 = time.perf_counter()
        for _ in range(n_steps):
            oracle.attention_ref(f["q"], f["k_step"], f["v_step"], f["k_cache"], f["v_cache"], d["lens"], s.k,
                                 s.n_groups, s.sm_scale)
            if args.verify == "sample":
                acc, _ = oracle.verify_sample_ref(v["ar_logits"], v["q_logits"], v["draft_logits"], v["cand"],
                                                  args.temperature, args.seed, 0)
            elif args.verify == "lmhead":
                acc = lm_acc
            else:
                acc, _ = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
            oracle.commit_ref(d["k_cache"], d["v_cache"], d["lens"], d["k_step"], d["v_step"], acc, s.k)
        dt = (time.perf_counter() - t0) / n_steps + lm_seconds
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    attn, ver, com, _, _ = step_bytes(s, wl.V, a_planted, args.verify, wl.d_model)
    return {"value": round((attn + ver + com) / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "seconds_per_step": round(dt, 3), "cpu_model": cpu_model(), "host_cores": cores,
            "sample": f"{n_steps} full {wl.name} steps (attention over all {s.B}x{s.Hq} heads, {args.verify} verify, "
                      "commit" + (", the LM head on 2 sequences scaled to the batch" if args.verify == "lmhead" else "")
                      + "), "
                      f"float64 NumPy, {threads} BLAS threads on {cores} host cores"}


TRAIN = {"B": 4, "Hq": 32, "Hkv": 8, "D": 128, "N": 4096, "block": 8}
MFMA_BF16_PEAK_TFLOPS = 2500.0


def train_pairs(N, bs):
    """Visible (row, key) pairs of one head of the training mask: N(N+1)/2
    for the clean half; each masked block of size s after lo clean tokens
    contributes s*(lo + s)."""
    masked = sum(min(bs, N - lo) * (lo + min(bs, N - lo)) for lo in range(0, N, bs))
    return N * (N + 1) // 2 + masked


def bench_train(args):
    """Training-mask attention: K calls between HIP events, inputs rotating
    over >= 2 GB of replicas; one JSON line with the MFMA roofline."""
    import numpy as np
    import torch

    import diffusion_drafted_self_amd as tidar
    import workloads as W

    c = TRAIN
    B, Hq, Hkv, D, N, bs = c["B"], c["Hq"], c["Hkv"], c["D"], c["N"], c["block"]
    dev = torch.device("cuda:0")
    d = W.train_inputs(B, Hq, Hkv, D, N, seed=args.seed)
    scale = 1.0 / math.sqrt(D)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    base = {n: to_dev(d[n]) for n in ("q", "k", "v")}
    per_rep = sum(t.numel() * t.element_size() for t in base.values()) * 2  # + the output
    n_rep = max(2, math.ceil(args.cold_bytes / per_rep))
    reps = [{**{n: t.clone() for n, t in base.items()}, "out": torch.empty_like(base["q"]),
             "lse": torch.empty((B, Hq, 2 * N), dtype=torch.float32, device=dev)} for _ in range(n_rep)]
    del base

    def call(r):
        tidar.train_attention(r["q"], r["k"], r["v"], N, bs, scale, out=r["out"], lse=r["lse"])

    K, Wu = args.steps, args.warmup
    for i in range(Wu):
        call(reps[i % n_rep])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(n_pre):  # K calls queued behind a spin, after n_pre untimed ones (see the step's queued timing)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2e6 * max(10.0, HOST_US_PER_CALL * (n_pre + K) / 1e3)))
        for i in range(n_pre):
            call(reps[(Wu + i) % n_rep])
        t0.record(stream)
        for i in range(K):
            call(reps[(Wu + n_pre + i) % n_rep])
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / K

    ms_after_idle = timed(0)
    ms = timed(int(min(MAX_SUSTAIN_CALLS, math.ceil(SUSTAIN_MS / ms_after_idle))))  # at the sustained clock
    assert torch.isfinite(reps[0]["out"].float()).all()
    flops = 4 * D * train_pairs(N, bs) * B * Hq
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "training-mask attention throughput (TFLOP/s over visible pairs)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": Wu,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "train_8b", "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "clean_positions": N, "sequence": 2 * N, "block": bs, "cold_replicas": n_rep},
        "attention_us": round(ms * 1e3, 2),
        "attention_us_after_idle": round(ms_after_idle * 1e3, 2),
        "timing": (f"attention_us: K calls queued after {SUSTAIN_MS:.0f} ms of untimed calls (the sustained clock); "
                   "attention_us_after_idle: the same K calls straight after an idle spin"),
        "roofline": {"bound": "mfma", "kernel": "tidar_train_attention", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_train(d, N, bs, scale, B, Hq, D)
    print(json.dumps(result))


def cpu_baseline_train(d, N, bs, scale, B, Hq, D):
    """The oracle (dense float64 over the whole T x T mask) on two of the
    B*Hq heads; the rate counts the visible-pair flops of those heads."""
    import numpy as np

    import oracle
    import workloads as W
    cores = len(os.sched_getaffinity(0))
    q, k, v = (W.bf16_to_f32(d[n]) for n in ("q", "k_nat", "v_nat"))
    heads = [(0, 0), (B - 1, Hq - 1)]
    G = Hq // k.shape[2]
    # the two heads as a batch of two single-head sequences: one call, one mask
    qs = np.stack([q[b, :, h] for b, h in heads])[:, :, None]
    ks = np.stack([k[b, :, h // G] for b, h in heads])[:, :, None]
    vs = np.stack([v[b, :, h // G] for b, h in heads])[:, :, None]
    t0 = time.perf_counter()
    oracle.train_attention_ref(qs, ks, vs, N, bs, scale)
    dt = time.perf_counter() - t0
    flops = 4 * D * train_pairs(N, bs) * len(heads)
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "seconds": round(dt, 2),
            "sample": f"{len(heads)} of {B * Hq} heads of train_8b (dense float64 over the full T x T mask)"}


def achievable_read_gbps(tidar, torch, dev, stream, gib: int = 4, reps: int = 5) -> float:
    """What the memory delivers to a plain streaming read, measured in the
    same run: the library's read helper over a buffer far beyond the caches
    (4 GiB against 256 MB of Infinity Cache)."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(tidar.READ_PROBE_BLOCKS, dtype=torch.int32, device=dev)
    tidar.read_probe(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        tidar.read_probe(buf, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    gbps = reps * buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    return gbps


def bench_loop(args, wl, d, v, a_planted, reps, n_rep, attention, verify_commit, tidar, torch, np, dev, stream):
    """The serving loop: args.loop consecutive steps on replica 0's cache.
    Each step's commit advances the device-side lengths in place; the host
    keeps the exact lengths (the accept lengths are planted) only to bound
    max_len and to count each step's algorithmic bytes.  Step rows and
    logits cycle over the input replicas, which all carry the same planted
    accept lengths."""
    s = wl.attn
    N = args.loop
    if args.paged or args.verify != "greedy":
        sys.exit("--loop runs the contiguous cache with greedy verification")
    lens_h = np.array(s.lens, dtype=np.int64)
    a = np.asarray(a_planted, dtype=np.int64)
    if int(lens_h.max()) + N * s.k > s.S_max:
        sys.exit(f"--loop {N}: the cache of this workload holds {s.S_max} positions, "
                 f"lengths reach up to {int(lens_h.max()) + N * s.k}")
    r0 = reps[0]
    for i in range(args.warmup):  # ordinary steps (lengths restored)
        r = reps[i % n_rep]
        attention(r)
        verify_commit(r, i)
    torch.cuda.synchronize()
    max_lens = [int(lens_h.max() + t * a.max()) for t in range(N)]
    ws = max(tidar.step_attention_workspace_bytes(0, s.B, s.Hq, s.Hkv, s.D, s.S_max, ml, s.k, s.n_groups,
                                                  args.kv_chunk) for ml in max_lens)
    ws_a = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(N)]
    step_b, attn_b, flops = [], [], []
    for t in range(N):
        r = reps[t % n_rep]
        sh = dataclasses.replace(s, lens=tuple(int(x) for x in lens_h))
        ab, vb, cb, _, fl = step_bytes(sh, wl.V, a, "greedy")
        step_b.append(ab + vb + cb)
        attn_b.append(ab)
        flops.append(fl + 4 * s.D * s.Hq * s.B * visible_step_pairs(s.k, s.n_groups))
        ev[t][0].record(stream)
        tidar.step_attention(r["q"], r["k_step"], r["v_step"], r0["k_cache"], r0["v_cache"], r0["lens"], s.k,
                             s.n_groups, s.sm_scale, max_len=max_lens[t], out=r["out"], lse=r["lse"],
                             workspace=ws_a, kv_chunk=args.kv_chunk)
        ev[t][1].record(stream)
        if args.separate:
            tidar.verify_greedy(r["ar_logits"], r["draft_logits"], r["cand"], accept_len=r0["acc"],
                                next_cand=r0["next"], workspace=r["ws_v"])
            tidar.kv_commit(r0["k_cache"], r0["v_cache"], r0["lens"], r["k_step"], r["v_step"], r0["acc"], s.k,
                            r0["err"])
        else:
            tidar.verify_commit_greedy(r["ar_logits"], r["draft_logits"], r["cand"], r0["k_cache"], r0["v_cache"],
                                       r0["lens"], r["k_step"], r["v_step"], accept_len=r0["acc"],
                                       next_cand=r0["next"], err_flags=r0["err"], state=r0["state"])
        ev[t][2].record(stream)
        lens_h = lens_h + a
    torch.cuda.synchronize()
    assert r0["acc"].cpu().numpy().tolist() == a.tolist(), "verify result differs from the planted accept lengths"
    assert r0["lens"].cpu().numpy().tolist() == lens_h.tolist() and int(r0["err"].abs().sum()) == 0
    step_ms = np.array([ev[t][0].elapsed_time(ev[t][2]) for t in range(N)])
    attn_ms = np.array([ev[t][0].elapsed_time(ev[t][1]) for t in range(N)])
    total_ms = ev[0][0].elapsed_time(ev[N - 1][2])
    step_gbps = sum(step_b) / (total_ms * 1e-3) / 1e9
    attn_gbps = sum(attn_b) / (attn_ms.sum() * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(attn_gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": N,
        "warmup": args.warmup, "ms_per_step": round(total_ms / N, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "_loop", "batch": s.B, "q_heads": s.Hq, "kv_heads": s.Hkv,
                   "head_dim": s.D, "prefix_start_mean": float(np.mean(s.lens)),
                   "prefix_end_mean": float(lens_h.mean()), "k": s.k, "draft_groups": s.n_groups,
                   "step_rows": s.R, "vocab": wl.V, "accept": wl.accept, "verify": "greedy",
                   "kv_layout": "contiguous", "input_replicas": n_rep,
                   "verify_commit": "separate" if args.separate else "fused"},
        "step_gbps": round(step_gbps, 2),
        "step_us_mean": round(total_ms / N * 1e3, 2),
        "step_us_p50": round(float(np.percentile(step_ms, 50)) * 1e3, 2),
        "step_us_p99": round(float(np.percentile(step_ms, 99)) * 1e3, 2),
        "attention_us_p50": round(float(np.percentile(attn_ms, 50)) * 1e3, 2),
        "attention_us_p99": round(float(np.percentile(attn_ms, 99)) * 1e3, 2),
        "attention_us_first": round(float(attn_ms[0]) * 1e3, 2),
        "attention_us_last": round(float(attn_ms[-1]) * 1e3, 2),
        "attention_gbps_mean": round(attn_gbps, 2),
        "attention_hbm_frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "attention_tflops_mean": round(sum(flops) / (attn_ms.sum() * 1e-3) / 1e12, 2),
        "attention_mfma_frac": round(sum(flops) / (attn_ms.sum() * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": attention_roofline(sum(attn_b) / N, sum(flops) / N, attn_ms.sum() / N, None),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, d, v, a_planted, args)
    print(json.dumps(result))


def bench_compare(args):
    """--compare: the attention call of args.workload timed across library
    builds in one process, interleaved so the part's clock (which moves with
    the time under load, see --clock-trace) is the same for all of them;
    single bench lines on one box vary by about +-2 us on the 8B step, more
    than the differences this resolves."""
    import statistics

    import numpy as np
    import torch

    import diffusion_drafted_self_amd as tidar
    import workloads as W

    dev = torch.device("cuda:0")
    libs = [tidar.LIB_PATH] + [os.path.abspath(x) for x in args.compare]

    def to_dev(x, bf16):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) if bf16 else torch.from_numpy(x).to(dev)

    cur = {"path": libs[0]}
    if args.compare_call == "verify_commit":
        wl = W.WORKLOADS[args.workload]()
        s = wl.attn
        d = W.attention_inputs(s, seed=args.seed, config_id=wl.config_id, tail="zero")
        v = W.verify_inputs(s.B, s.k, wl.V, seed=args.seed, config_id=wl.config_id, accept=wl.accept)
        base = {n: to_dev(d[n], n != "lens") for n in ("k_cache", "v_cache", "k_step", "v_step", "lens")}
        base.update({n: to_dev(v[n], False) for n in ("ar_logits", "draft_logits", "cand")})
        n_rep = max(2, math.ceil(args.cold_bytes / sum(t.numel() * t.element_size() for t in base.values())))
        reps = [{**{n: t.clone() for n, t in base.items()}, "lens0": base["lens"].clone(),
                 "acc": torch.empty(s.B, dtype=torch.int32, device=dev),
                 "out": torch.empty((s.B, s.k), dtype=torch.int32, device=dev),
                 "err": torch.empty(s.B, dtype=torch.int32, device=dev)} for _ in range(n_rep)]
        states = {}
        for path in libs:
            with tidar.library(path):
                states[path] = tidar.verify_commit_state(s.B, s.k, dev)

        def call(r):
            tidar.verify_commit_greedy(r["ar_logits"], r["draft_logits"], r["cand"], r["k_cache"], r["v_cache"],
                                       r["lens"], r["k_step"], r["v_step"], accept_len=r["acc"], next_cand=r["out"],
                                       err_flags=r["err"], state=states[cur["path"]])
            r["lens"].copy_(r["lens0"])
    elif args.workload == "train_8b":
        c = TRAIN
        d = W.train_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["N"], seed=args.seed)
        base = {n: to_dev(d[n], True) for n in ("q", "k", "v")}
        n_rep = 2
        reps = [{**{n: t.clone() for n, t in base.items()}, "out": torch.empty_like(base["q"]),
                 "lse": torch.empty((c["B"], c["Hq"], 2 * c["N"]), dtype=torch.float32, device=dev)}
                for _ in range(n_rep)]

        def call(r):
            tidar.train_attention(r["q"], r["k"], r["v"], c["N"], c["block"], 1.0 / math.sqrt(c["D"]), out=r["out"],
                                  lse=r["lse"])
    else:
        wl = W.WORKLOADS[args.workload]()
        s = wl.attn
        d = W.attention_inputs(s, seed=args.seed, config_id=wl.config_id, tail="zero")
        base = {n: to_dev(x, n != "lens") for n, x in d.items()}
        n_rep = max(2, math.ceil(args.cold_bytes / sum(t.numel() * t.element_size() for t in base.values())))
        ws = tidar.step_attention_workspace_bytes(0, s.B, s.Hq, s.Hkv, s.D, s.S_max, s.max_len, s.k, s.n_groups,
                                                  args.kv_chunk)
        reps = [{**{n: t.clone() for n, t in base.items()}, "out": torch.empty_like(base["q"]),
                 "lse": torch.empty((s.B, s.Hq, s.R), dtype=torch.float32, device=dev),
                 "ws": torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)} for _ in range(n_rep)]

        def call(r):
            tidar.step_attention(r["q"], r["k_step"], r["v_step"], r["k_cache"], r["v_cache"], r["lens"], s.k,
                                 s.n_groups, s.sm_scale, max_len=s.max_len, out=r["out"], lse=r["lse"],
                                 workspace=r["ws"], kv_chunk=args.kv_chunk)
    del base
    outs = []
    for path in libs:
        with tidar.library(path):
            cur["path"] = path
            call(reps[0])
            torch.cuda.synchronize()
            outs.append(reps[0]["out"].float().clone())
            if args.compare_call == "verify_commit":  # accept lengths too, and the cache rows written
                outs[-1] = torch.cat([outs[-1].flatten(), reps[0]["acc"].float(), reps[0]["err"].float()])
    diffs = [float((o - outs[0]).abs().max().item()) for o in outs[1:]]
    K, i = args.steps, 0
    with tidar.library(libs[0]):
        cur["path"] = libs[0]
        t0 = time.time()
        while time.time() - t0 < 0.3:  # sustaining calls: the clock the part settles at under load
            call(reps[i % n_rep])
            i += 1
    times = {p: [] for p in libs}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for rd in range(args.rounds):
        for path in libs[rd % len(libs):] + libs[:rd % len(libs)]:
            with tidar.library(path):
                cur["path"] = path
                for j in range(3):  # untimed: the change of code object
                    call(reps[(i + j) % n_rep])
                i += 3
                ev[0].record()
                for j in range(K):
                    call(reps[(i + j) % n_rep])
                ev[1].record()
                i += K
                torch.cuda.synchronize()
            times[path].append(ev[0].elapsed_time(ev[1]) * 1e3 / K)
    med0 = statistics.median(times[libs[0]])
    print(json.dumps({
        "metric": f"{args.compare_call} us per call, paired across library builds", "workload": args.workload,
        "calls_per_round": K, "rounds": args.rounds,
        "libraries": [{"path": os.path.relpath(p), "median_us": round(statistics.median(times[p]), 2),
                       "mean_us": round(statistics.mean(times[p]), 2), "min_us": round(min(times[p]), 2),
                       "vs_first_pct": round(100 * (statistics.median(times[p]) / med0 - 1), 2)} for p in libs],
        "max_abs_out_diff_vs_first": diffs}))


def bench_probes(args):
    """--probes: the matrix cores' issue interval (tidar_mfma_probe) with one
    and two waves per SIMD, operands in registers or read from LDS; one JSON
    line."""
    import statistics

    import numpy as np
    import torch

    import diffusion_drafted_self_amd as tidar

    dev = torch.device("cuda:0")
    iters = 4096
    res = {}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for lds in (0, 1):
        for w in (1, 2):
            tidar.mfma_probe(w, lds, 64, dev)  # warm-up (code object, clock)
            torch.cuda.synchronize()
            ev[0].record()
            c = tidar.mfma_probe(w, lds, iters, dev)
            ev[1].record()
            torch.cuda.synchronize()
            cyc = c.cpu().numpy()
            if (cyc < 0).any():
                raise RuntimeError("mfma probe: a record carries the impossible-sum mark")
            med, mx = float(np.median(cyc)), float(cyc.max())
            us = ev[0].elapsed_time(ev[1]) * 1e3
            # the waves of a SIMD start together; the SIMD's MFMAs are done when its last wave is
            res[f"{'lds' if lds else 'registers'}_{w}_waves_per_simd"] = {
                "simd_cycles_per_mfma": round(mx / (8 * iters * w), 2),
                "wave_cycles_per_mfma_median": round(med / (8 * iters), 2),
                "wave_cycles_median": int(med), "wave_cycles_max": int(mx),
                "kernel_us": round(us, 1), "shader_mhz": round(mx / us, 0)}
    print(json.dumps({"metric": "issue interval of v_mfma_f32_16x16x32_bf16 (shader-clock cycles)",
                      "iters": iters, "mfma_per_round": 8, "workgroups": tidar.MFMA_PROBE_BLOCKS, "results": res}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark runs on one GPU, with no "
              "collectives (each GPU would run the same step on its own share of the batch).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.summarize:
        summarize(args.summarize)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.counters_kernel)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_lmhead:
        summarize_lmhead(args.summarize_lmhead)
        return
    if args.probes:
        bench_probes(args)
        return
    if args.compare:
        bench_compare(args)
        return
    if args.workload == "train_8b":
        bench_train(args)
        return

    import numpy as np
    import torch

    import diffusion_drafted_self_amd as tidar
    import workloads as W

    if not os.path.exists(tidar.LIB_PATH):
        from __graft_entry__ import build
        build()
    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]()
    s = wl.attn

    d = W.attention_inputs(s, seed=args.seed, config_id=wl.config_id, tail="zero")
    if args.verify == "sample":
        v = W.sample_inputs(s.B, s.k, wl.V, seed=args.seed, config_id=wl.config_id)
        v_names = ("ar_logits", "q_logits", "draft_logits", "cand")
        a_planted = None
    elif args.verify == "lmhead":
        v = W.lmhead_inputs(s.B, s.k, wl.V, wl.d_model, seed=args.seed,
                            accept=wl.accept if wl.accept in ("uniform", "geometric") else "uniform")
        v_names = ("h_ar", "h_draft", "w", "cand")
        a_planted = v["planted"]
    else:
        v = W.verify_inputs(s.B, s.k, wl.V, seed=args.seed, config_id=wl.config_id, accept=wl.accept)
        v_names = ("ar_logits", "draft_logits", "cand")
        a_planted = v["planted"]

    def to_dev(x, bf16):
        x = np.ascontiguousarray(x)
        if bf16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    if args.paged:
        pg = W.to_pages(d["k_cache"], d["v_cache"], seed=args.seed, spare=0, config_id=wl.config_id)
        d_dev = {n: x for n, x in d.items() if n not in ("k_cache", "v_cache")}
        d_dev.update({"k_pool": pg["k_pool"], "v_pool": pg["v_pool"], "block_table": pg["block_table"]})
        del pg
    else:
        d_dev = d
    base = {n: to_dev(x, n not in ("lens", "block_table")) for n, x in d_dev.items()}
    del d_dev
    base.update({n: to_dev(v[n], n in ("h_ar", "h_draft", "w")) for n in v_names})
    per_rep = sum(t.numel() * t.element_size() for t in base.values())
    n_rep = max(2, math.ceil(args.cold_bytes / per_rep))
    ws_a = tidar.step_attention_workspace_bytes(0, s.B, s.Hq, s.Hkv, s.D, s.S_max, s.max_len, s.k, s.n_groups,
                                                args.kv_chunk)
    if args.verify == "lmhead":
        ws_v = tidar.lmhead_verify_workspace_bytes(s.B, s.k, wl.V, wl.d_model)
    else:
        ws_v = (tidar.verify_sample_workspace_bytes if args.verify == "sample" else tidar.verify_workspace_bytes)(
            s.B, s.k, wl.V)
    packed_w = args.verify == "lmhead" and args.lm_layout == "packed"
    reps = []
    for _ in range(n_rep):
        r = {n: t.clone() for n, t in base.items() if not (packed_w and n == "w")}
        if packed_w:  # the head is packed once, when weights are loaded
            r["wp"] = tidar.lmhead_pack(base["w"])
        r["lens0"] = base["lens"].clone()
        r["out"] = torch.empty_like(base["q"])
        r["lse"] = torch.empty((s.B, s.Hq, s.R), dtype=torch.float32, device=dev)
        r["ws_a"] = torch.zeros(max(ws_a, 256), dtype=torch.uint8, device=dev)
        r["ws_v"] = torch.empty(ws_v, dtype=torch.uint8, device=dev)
        r["acc"] = torch.empty(s.B, dtype=torch.int32, device=dev)
        r["next"] = torch.empty((s.B, s.k), dtype=torch.int32, device=dev)
        r["err"] = torch.empty(s.B, dtype=torch.int32, device=dev)
        r["state"] = tidar.verify_commit_state(s.B, s.k, dev)
        reps.append(r)
    del base
    torch.cuda.synchronize()

    def attention(r):
        if args.paged:
            tidar.step_attention_paged(r["q"], r["k_step"], r["v_step"], r["k_pool"], r["v_pool"], r["block_table"],
                                       r["lens"], s.k, s.n_groups, s.sm_scale, max_len=s.max_len, out=r["out"],
                                       lse=r["lse"], workspace=r["ws_a"], kv_chunk=args.kv_chunk)
            return
        tidar.step_attention(r["q"], r["k_step"], r["v_step"], r["k_cache"], r["v_cache"], r["lens"], s.k,
                             s.n_groups, s.sm_scale, max_len=s.max_len, out=r["out"], lse=r["lse"],
                             workspace=r["ws_a"], kv_chunk=args.kv_chunk)

    def verify(r, step_no):
        if packed_w:
            tidar.lmhead_verify_greedy_packed(r["h_ar"], r["h_draft"], r["wp"], wl.V, r["cand"], accept_len=r["acc"],
                                              next_cand=r["next"], workspace=r["ws_v"])
        elif args.verify == "lmhead":
            tidar.lmhead_verify_greedy(r["h_ar"], r["h_draft"], r["w"], r["cand"], accept_len=r["acc"],
                                       next_cand=r["next"], workspace=r["ws_v"])
        elif args.verify == "sample":
            tidar.verify_sample(r["ar_logits"], r["q_logits"], r["draft_logits"], r["cand"], args.temperature,
                                args.seed, step_no, accept_len=r["acc"], next_cand=r["next"], workspace=r["ws_v"])
        else:
            tidar.verify_greedy(r["ar_logits"], r["draft_logits"], r["cand"], accept_len=r["acc"],
                                next_cand=r["next"], workspace=r["ws_v"])

    def commit(r):
        if args.paged:
            tidar.kv_commit_paged(r["k_pool"], r["v_pool"], r["block_table"], r["lens"], r["k_step"], r["v_step"],
                                  r["acc"], s.k, r["err"])
        else:
            tidar.kv_commit(r["k_cache"], r["v_cache"], r["lens"], r["k_step"], r["v_step"], r["acc"], s.k,
                            r["err"])
        r["lens"].copy_(r["lens0"])

    fused = args.verify == "greedy" and not args.separate

    def verify_commit(r, step_no, ev=None):
        if fused:  # one call: greedy verify and the commit
            if args.paged:
                tidar.verify_commit_greedy_paged(r["ar_logits"], r["draft_logits"], r["cand"], r["k_pool"],
                                                 r["v_pool"], r["block_table"], r["lens"], r["k_step"], r["v_step"],
                                                 accept_len=r["acc"], next_cand=r["next"], err_flags=r["err"],
                                                 state=r["state"])
            else:
                tidar.verify_commit_greedy(r["ar_logits"], r["draft_logits"], r["cand"], r["k_cache"], r["v_cache"],
                                           r["lens"], r["k_step"], r["v_step"], accept_len=r["acc"],
                                           next_cand=r["next"], err_flags=r["err"], state=r["state"])
            r["lens"].copy_(r["lens0"])
            return
        verify(r, step_no)
        if ev is not None:
            ev.record(stream)
        commit(r)

    stream = torch.cuda.current_stream()
    K, Wu = args.steps, args.warmup
    if args.loop:
        bench_loop(args, wl, d, v, a_planted, reps, n_rep, attention, verify_commit, tidar, torch, np, dev, stream)
        return
    if args.clock_trace:
        clock_trace(args.clock_trace, wl.name, reps, n_rep, attention, torch, stream)
        return
    ev_a = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    # the fused LM head dominates its step: its own end event after verify
    ev_v = [torch.cuda.Event(enable_timing=True) if args.verify == "lmhead" else None for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(Wu):
        r = reps[i % n_rep]
        attention(r)
        verify_commit(r, i)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        r = reps[(Wu + i) % n_rep]
        ev_a[i][0].record(stream)
        attention(r)
        ev_a[i][1].record(stream)
        verify_commit(r, Wu + i, ev_v[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_end) / K
    attn_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev_a)
    attn_ms_mean = sum(attn_ms) / K

    assert int(reps[0]["err"].abs().sum()) == 0

    # The same steps replayed from HIP graphs (one captured step per input
    # replica, so the launches cost no host time between kernels): the
    # whole-step figure step_us_graph.  The sampling step takes its draw
    # counter as a launch argument and is not replayed.
    graph_ms = None
    if args.verify != "sample":
        side = torch.cuda.Stream()
        graphs = []
        for r in reps:
            side.wait_stream(stream)
            with torch.cuda.stream(side):  # a warm-up outside capture, on a side stream
                attention(r)
                verify_commit(r, 0)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                attention(r)
                verify_commit(r, 0)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(Wu):
            graphs[i % n_rep].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for i in range(K):
            graphs[(Wu + i) % n_rep].replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
        for r in reps:  # the replays did the step: planted accept lengths, lengths restored
            if a_planted is not None:
                assert r["acc"].cpu().numpy().tolist() == a_planted.tolist()
            assert torch.equal(r["lens"], r["lens0"]) and int(r["err"].abs().sum()) == 0
        del graphs

    # The attention calls alone and the verify + commit calls alone, each K
    # in a row on the rotating replicas, queued behind a spin kernel so the
    # host has enqueued all of them before the GPU reaches the first: an
    # event pair around the K calls then times the GPU's work (what
    # rocprofv3 reports for the kernels), not the host's launch overhead.
    # The clock the part runs at depends on how long it has been under load
    # (--clock-trace shows it): after an idle spell the first ~2 ms of calls
    # run boosted, the power controller then clamps for several ms, and the
    # clock settles after ~30 ms.  So the timed calls follow untimed
    # calls of the same work lasting SUSTAIN_MS and run at the clock the
    # part sustains under this load, as in a serving loop; the *_after_idle
    # figures time the same K calls straight after the spin instead.
    vc_ms = None
    attn_ms_pair_mean = None
    attn_ms_warm = attn_ms_after_idle = vc_ms_after_idle = None
    queued = args.verify == "greedy"
    if queued:
        def queued_run(fn, per_call, n_pre=0):
            torch.cuda.synchronize()
            # the host's head start: it enqueues the untimed and the timed calls while the GPU spins
            torch.cuda._sleep(int(2e6 * max(10.0, HOST_US_PER_CALL * (n_pre + K) / 1e3)))
            for i in range(n_pre):
                fn(reps[(Wu + i) % n_rep])
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
            q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            q0.record(stream)
            for i in range(K):
                r = reps[(Wu + n_pre + i) % n_rep]
                if per_call:
                    evs[i][0].record(stream)
                fn(r)
                if per_call:
                    evs[i][1].record(stream)
            q1.record(stream)
            torch.cuda.synchronize()
            return q0.elapsed_time(q1) / K, sorted(e0.elapsed_time(e1) for e0, e1 in evs) if per_call else None

        def sustain_calls(ms_per_call):  # untimed calls that keep the GPU busy for SUSTAIN_MS
            return int(min(MAX_SUSTAIN_CALLS, math.ceil(SUSTAIN_MS / max(ms_per_call, 1e-3))))

        attn_ms_after_idle, _ = queued_run(attention, False)
        n_pre = sustain_calls(attn_ms_after_idle)
        _, attn_ms = queued_run(attention, True, n_pre)
        attn_ms_pair_mean = sum(attn_ms) / K
        attn_ms_mean, _ = queued_run(attention, False, n_pre)
        # warm: the same replica every call (what caches keep of it between calls is reused)
        attn_ms_warm, _ = queued_run(lambda r: attention(reps[0]), False, n_pre)
        vc_ms_after_idle, _ = queued_run(lambda r: verify_commit(r, 0), False)
        vc_ms, _ = queued_run(lambda r: verify_commit(r, 0), False, sustain_calls(vc_ms_after_idle))
        for r in reps:
            if a_planted is not None:
                assert r["acc"].cpu().numpy().tolist() == a_planted.tolist()
            assert torch.equal(r["lens"], r["lens0"]) and int(r["err"].abs().sum()) == 0
    read_gbps = achievable_read_gbps(tidar, torch, dev, stream)
    if args.verify == "sample":
        # sampling is a function of (inputs, seed, step): replay the timed
        # steps' verification to get the accept lengths their bytes depend on
        accs = []
        for i in range(K):
            r = reps[(Wu + i) % n_rep]
            verify(r, Wu + i)
            accs.append(r["acc"].cpu().numpy())
        acc_all = np.stack(accs)
        assert ((acc_all >= 0) & (acc_all <= s.k)).all()
        a_planted = acc_all.mean(axis=0)
        b_steps = [step_bytes(s, wl.V, a, "sample") for a in acc_all]
        attn_b, kv_b, flops = b_steps[0][0], b_steps[0][3], b_steps[0][4]
        ver_b = sum(b[1] for b in b_steps) / K
        com_b = sum(b[2] for b in b_steps) / K
    else:
        # the accepted lengths the GPU produced must be the planted ones (exact by construction)
        acc = reps[0]["acc"].cpu().numpy()
        if a_planted is not None:
            assert acc.tolist() == a_planted.tolist(), "verify result differs from the planted accept lengths"
        else:
            a_planted = acc
        attn_b, ver_b, com_b, kv_b, flops = step_bytes(s, wl.V, a_planted, args.verify, wl.d_model)
    flops_step = 4 * s.D * s.Hq * s.B * visible_step_pairs(s.k, s.n_groups)
    step_gbps = (attn_b + ver_b + com_b) / (step_ms * 1e-3) / 1e9
    attn_gbps = attn_b / (attn_ms_mean * 1e-3) / 1e9
    traffic = read_traffic()
    result = {
        "metric": METRIC,
        "value": round(attn_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "kv_chunk": args.kv_chunk or "auto", "batch": s.B, "q_heads": s.Hq, "kv_heads": s.Hkv, "head_dim": s.D,
                   "prefix": s.lens[0], "k": s.k, "draft_groups": s.n_groups, "step_rows": s.R, "vocab": wl.V,
                   "accept": wl.accept if args.verify == "greedy" else "sampled", "verify": args.verify,
                   "kv_layout": "paged" if args.paged else "contiguous",
                   "verify_commit": "fused" if fused else "separate",
                   "attention_plan": tidar.step_attention_plan(0, s.B, s.Hq, s.Hkv, s.D, s.S_max, s.max_len, s.k,
                                                               s.n_groups, args.kv_chunk),
                   "cold_replicas": n_rep},
        "step_gbps": round(step_gbps, 2),
        "step_us": round(step_ms * 1e3, 2),
        "step_us_graph": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
        "attention_us": round(attn_ms_mean * 1e3, 2),
        "attention_us_p50": round(attn_ms[K // 2] * 1e3, 2),
        "attention_us_p99": round(attn_ms[min(K - 1, math.ceil(0.99 * K) - 1)] * 1e3, 2),
        "attention_kv_gbps": round(kv_b / (attn_ms_mean * 1e-3) / 1e9, 2),
        "attention_hbm_frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "achievable_read_gbps": round(read_gbps, 1),
        "attention_achievable_frac": round(attn_gbps / read_gbps, 4),
        "attention_tflops": round((flops + flops_step) / (attn_ms_mean * 1e-3) / 1e12, 2),
        "attention_mfma_frac": round((flops + flops_step) / (attn_ms_mean * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "attention_us_warm": None if attn_ms_warm is None else round(attn_ms_warm * 1e3, 2),
        "attention_us_after_idle": None if attn_ms_after_idle is None else round(attn_ms_after_idle * 1e3, 2),
        "verify_commit_us": round((vc_ms if vc_ms is not None else step_ms - attn_ms_mean) * 1e3, 2),
        "verify_commit_us_after_idle": None if vc_ms_after_idle is None else round(vc_ms_after_idle * 1e3, 2),
        "attention_us_event_pairs": round(attn_ms_pair_mean * 1e3, 2) if vc_ms is not None else None,
        "timing": (f"attention_us / verify_commit_us: each call alone, K in a row on the rotating (cold) replicas, "
                   f"queued (GPU time) after {SUSTAIN_MS:.0f} ms of untimed calls of the same work (the sustained "
                   "clock); *_after_idle: the same K calls straight after an idle spin; attention_us_warm: sustained, "
                   "one replica (warm); step_us: eager whole steps; step_us_graph: replayed whole steps"
                   if vc_ms is not None else "eager steps, an event pair around each attention call"),
        "roofline": attention_roofline(attn_b, flops + flops_step, attn_ms_mean,
                                       traffic if wl.name == "step_8b" and not args.paged else None),
    }
    if args.verify == "lmhead":
        lm_ms = sum(ev_a[i][1].elapsed_time(ev_v[i]) for i in range(K)) / K
        lm_gbps = ver_b / (lm_ms * 1e-3) / 1e9
        result["config"]["d_model"] = wl.d_model
        result["config"]["w_layout"] = args.lm_layout
        result["lmhead_verify_us"] = round(lm_ms * 1e3, 2)
        result["attention_roofline"] = result["roofline"]
        result["roofline"] = {"bound": "hbm",
                              "kernel": "tidar_lmhead_verify_greedy" + ("_packed" if packed_w else ""),
                              "achieved": round(lm_gbps, 2),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(lm_gbps / HBM_PEAK_GBPS, 4),
                              "traffic": (read_traffic(LM_TRAFFIC_FILE, lmhead_source_sha, "hbm_bytes_per_verify")
                                          if packed_w and wl.name == "step_8b" else None),
                              "algorithmic_bytes": ver_b}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, d, v, a_planted, args)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
