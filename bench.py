#!/usr/bin/env python3
"""KDA benchmark on one MI355X.

One step is one pass of the whole hot path:
  * kda_chunk_fwd over B=1, H=32, T=65536, d_k=d_v=128 (bf16 q/k/v/o, fp32
    gates, random fp32 initial state, final state returned), chunk 64; and
  * one kda_recurrent_step over 256 sequences x 32 heads, d=128, fp32 state
    (512 MiB) updated in place; step i consumes the i-th of 100 pre-generated
    token batches (the decode workload is 100 such steps).
All inputs are seeded synthetic data already resident in HBM.  HIP events on
the stream the kernels run on time each part; `value` is the chunk forward's
token-head throughput (B*H*T per second of kda_chunk_fwd), and the decode
step is reported as achieved HBM GB/s.

Prints ONE JSON line.  Flags:
  --gpus N --steps K --warmup W       (N must be 1: the benchmark runs on one GPU)
  --no-cpu-baseline                   skip the oracle timing
  --only fwd|decode|bwd               time one part only (profiler runs; bwd = the
                                      chunkwise backward on the forward's shape)
  --no-variants                       skip the measured peaks, the other gate forms
                                      and the backward line
  --copy-calibration                  run a plain 1 GiB device copy (used to
                                      scale rocprofv3 FETCH_SIZE/WRITE_SIZE)
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix cores, vendor figure
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix cores, vendor figure

# Algorithmic ledger per token-head of the chunk forward (d_k = d_v = 128):
# q, k, v, o in bf16 (4 x 256 B) + alpha fp32 (512 B) + beta fp32 (4 B).
FWD_BYTES_PER_TOKEN_HEAD = 4 * 2 * 128 + 4 * 128 + 4
# Useful flops per token-head at C = 64, d = 128: three d x d contractions
# (6 d^2) + C-dependent products (A, T.X, QK^T, P.U') + the triangular solve.
FWD_FLOPS_PER_TOKEN_HEAD = 6 * 128 * 128 + 64 * 128 + 64 * 256 + 64 * 128 + 64 * 128 + 64 * 64 // 3


def fwd_flops_per_token_head(C=64, dk=128, dv=128):
    """Useful flops per token-head of the chunk forward at chunk size C: the
    three d x d contractions plus the C-dependent products (A, T.X, QK^T,
    P.U') and the triangular solve."""
    return 6 * dk * dv + C * dk + C * (dk + dv) + C * dk + C * dv + C * C // 3


# Chunkwise backward, per token-head: reads q, k, v, dO (bf16), alpha, beta;
# writes dq, dk, dv (bf16), dalpha, dbeta (fp32).
BWD_BYTES_PER_TOKEN_HEAD = 4 * 2 * 128 + 128 * 4 + 4 + 3 * 2 * 128 + 128 * 4 + 4


def bwd_flops_split(C=64, dk=128, dv=128):
    """Useful flops (2 x multiply-adds, triangular products at half) per
    token-head of the chunkwise backward with the forward recomputed, split by
    the matrix cores that run them with 16-bit activations:
      fp16  the two state-chain passes and the value-side contractions:
            8 dk dv + 2.5 C dv per token (W S, Kt^T U', Kt dS, Qh^T dO, W^T dU',
            dO S^T, dU' S^T, U' dS^T; P^T dO, M, N, T^T dU')
      fp32  preparation and key side: 5.5 C dk + 0.5 C dv + 7/6 C^2 per token
            (A, P, W, U, T; dT, R, dY, dKh, dQh, dKb; Y1, dA).
    With fp32 activations every product runs on the fp32 matrix cores."""
    f16 = 2 * (8 * dk * dv + 2.5 * C * dv)
    f32 = 2 * (5.5 * C * dk + 0.5 * C * dv + (7.0 / 6.0) * C * C)
    return f16, f32


def bwd_flops_per_token_head(C=64, dk=128, dv=128):
    return sum(bwd_flops_split(C, dk, dv))


def bwd_mixed_peak(C=64, dk=128, dv=128):
    """Matrix-core roofline of the 16-bit backward: its useful flops over the
    time they take at the fp16 and fp32 peaks (each part at its own peak)."""
    f16, f32 = bwd_flops_split(C, dk, dv)
    return (f16 + f32) / (f16 / BF16_MFMA_PEAK_TFLOPS + f32 / FP32_MFMA_PEAK_TFLOPS)


# bytes of the forget gate per token-head, by form (gate= argument)
GATE_BYTES = {"alpha": 4 * 128, "softplus": 2 * 128, "scalar": 4}


def decode_bytes_per_step(N, H, Dk, Dv, gate="alpha"):
    state = 2 * N * H * Dk * Dv * 4                      # read + write, fp32
    gbytes = {"alpha": Dk * 4, "softplus": Dk * 2, "scalar": 4}[gate]
    io = N * H * (2 * Dk * 2 + Dv * 2 + Dv * 2 + gbytes + 4)   # q,k,v,o bf16, gate, beta
    return state + io


def time_events(fn, reps, warm=3):
    """Mean milliseconds of fn() over reps calls (HIP events on the current stream)."""
    import torch
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# the device code of the forward and decode kernels (host-side validation lives elsewhere)
KERNEL_SOURCES = ["gated_delta_rule_12_amd/csrc/kda_chunk.hip", "gated_delta_rule_12_amd/csrc/kda_decode.hip",
                  "gated_delta_rule_12_amd/csrc/kda_common.h", "gated_delta_rule_12_amd/csrc/kda_chunk.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                            "hbm_traffic_chunk_fwd_B1_H32_T65536_d128_bf16+decode_N256_H32_d128_bf16.txt")


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when the kernel sources changed since it was taken."""
    import hashlib
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if not line.startswith("#") and ":" in line:
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.split()[0]
        h = hashlib.sha256()
        for s in KERNEL_SOURCES:
            with open(os.path.join(ROOT, s), "rb") as f:
                h.update(f.read())
        if fields.get("sources_sha256") != h.hexdigest():
            return None
        return {"fwd": int(float(fields["fwd_traffic_bytes"])),
                "decode": int(float(fields["decode_traffic_bytes"]))}
    except (OSError, KeyError, ValueError):
        return None


# the device code of the backward kernels
BWD_KERNEL_SOURCES = ["gated_delta_rule_12_amd/csrc/kda_chunk_bwd.hip", "gated_delta_rule_12_amd/csrc/kda_mm32.h",
                      "gated_delta_rule_12_amd/csrc/kda_common.h", "gated_delta_rule_12_amd/csrc/kda_chunk.h"]
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_chunk_bwd_B1_H32_T65536_d128_bf16.txt")


def measured_bwd_traffic():
    """HBM bytes per backward launch from the committed rocprofv3 summary, or
    None when the backward's sources changed since it was taken."""
    import hashlib
    try:
        fields = {}
        with open(BWD_TRAFFIC_FILE) as f:
            for line in f:
                if not line.startswith("#") and ":" in line:
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.split()[0]
        h = hashlib.sha256()
        for s in BWD_KERNEL_SOURCES:
            with open(os.path.join(ROOT, s), "rb") as f:
                h.update(f.read())
        if fields.get("bwd_sources_sha256") != h.hexdigest():
            return None
        return int(float(fields["bwd_traffic_bytes"]))
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# Summaries of rocprofv3 output (no GPU needed): the text files under
# profiles/ are written by `python bench.py --summarize KIND ...` from the CSV
# files of the rocprofv3 runs named in each summary's header.
# ---------------------------------------------------------------------------
GEN_KERNELS = ("gprep_kernel", "gprep_general_kernel", "gchain_kernel", "gout_kernel")   # chunk sizes 32 / 128
LIB_KERNELS = ("plan_kernel", "prep_kernel", "prep_general_kernel", "state_kernel", "state_split_kernel", "decode_kernel",
               "bwd_prep_kernel", "bwd_prep_general_kernel", "bwd_ckpt_kernel", "bwd_ckpt16_kernel",
               "bwd_rev_kernel", "bwd_rev16_kernel", "bwd_grad_kernel", "bwd_grad_general_kernel") + GEN_KERNELS
FWD_KERNELS = ("plan_kernel", "prep_kernel", "prep_general_kernel", "state_kernel", "state_split_kernel")
BWD_KERNELS = ("plan_kernel", "bwd_prep_kernel", "bwd_prep_general_kernel", "bwd_ckpt_kernel",
               "bwd_ckpt16_kernel", "bwd_rev_kernel", "bwd_rev16_kernel", "bwd_grad_kernel",
               "bwd_grad_general_kernel")


def _kernel_base(name):
    """The kernel's identifier: 'void kda::(anonymous namespace)::prep_kernel<...>(...)' -> 'prep_kernel'."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("kda::(anonymous namespace)::", "").replace("kda::", "")
    cut = len(n)
    for ch in "<(":
        k = n.find(ch)
        if k >= 0:
            cut = min(cut, k)
    return n[:cut].split("::")[-1].strip()


def _kernel_short(name):
    """The identifier with its template arguments, without the parameter list."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("kda::(anonymous namespace)::", "").replace("kda::", "")
    depth = 0
    for k, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:k]
    return n


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for s in paths:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _csv_rows(pattern):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"bench.py --summarize: no rows in {pattern}")
    return rows


def _counter_means(pattern, counter):
    """Mean counter value per dispatch, per library kernel (short name)."""
    acc = {}
    for r in _csv_rows(pattern):
        if r["Counter_Name"] != counter or _kernel_base(r["Kernel_Name"]) not in LIB_KERNELS:
            continue
        v = acc.setdefault(_kernel_short(r["Kernel_Name"]), [])
        v.append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _copy_counter(pattern, counter):
    """Mean counter value over the device-copy dispatches of --copy-calibration."""
    vals = [float(r["Counter_Value"]) for r in _csv_rows(pattern)
            if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"bench.py --summarize: no copy dispatch with {counter} in {pattern}")
    return sum(vals) / len(vals)


def _chunk_arg(name):
    """The chunk size of a generic-path kernel: its third template argument."""
    short = _kernel_short(name)
    args = short[short.find("<") + 1:short.rfind(">")].split(",")
    return int(args[2]) if len(args) > 2 else 0


def summarize(kind, inputs, title, commands, kernels=None):
    """Print a profiles/ summary.  kind:
      trace    inputs = [kernel_stats.csv glob]
      traffic  inputs = [FETCH_SIZE csv glob, WRITE_SIZE csv glob, copy FETCH_SIZE glob, copy WRITE_SIZE glob]
      mfma     inputs = [MfmaUtil csv glob, MOPS csv glob]
      counters inputs = [counter csv glob, ...]: the mean per dispatch of every counter found"""
    print(f"# {title}")
    for c in commands:
        print(f"# {c}")
    fwd_sha, bwd_sha = sources_sha256(KERNEL_SOURCES), sources_sha256(BWD_KERNEL_SOURCES)
    if kind == "trace":
        keep = kernels or LIB_KERNELS
        rows = [r for r in _csv_rows(inputs[0]) if _kernel_base(r["Name"]) in LIB_KERNELS
                and _kernel_base(r["Name"]) in keep]
        print(f"# forward/decode sources sha256: {fwd_sha}")
        print(f"# backward sources sha256: {bwd_sha}")
        print("#")
        print(f"# {'kernel':48s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
        sums, seen = {}, set()
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            base, avg = _kernel_base(r["Name"]), float(r["AverageNs"]) / 1e3
            seen.add(base)
            print(f"  {_kernel_short(r['Name']):48s} {int(r['Calls']):6d} {avg:10.2f} "
                  f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")
            for grp, names in (("forward", FWD_KERNELS), ("backward", BWD_KERNELS), ("decode", ("decode_kernel",))):
                if base in names:
                    sums[grp] = sums.get(grp, 0.0) + avg
            if base in GEN_KERNELS:
                grp = f"chunk-{_chunk_arg(r['Name'])} forward (generic path)"
                sums[grp] = sums.get(grp, 0.0) + avg
        for grp, names in (("forward", FWD_KERNELS), ("backward", BWD_KERNELS), ("decode", ("decode_kernel",))):
            if any(n in seen and n != "plan_kernel" for n in names):
                print(f"# {grp} kernels, sum of averages: {sums[grp]:.2f} us")
        for grp in sorted(k for k in sums if k.startswith("chunk-")):
            print(f"# {grp} kernels (plan_kernel not included), sum of averages: {sums[grp]:.2f} us")
    elif kind == "traffic":
        fetch, write = _counter_means(inputs[0], "FETCH_SIZE"), _counter_means(inputs[1], "WRITE_SIZE")
        copy_bytes = 1 << 30
        fs = copy_bytes / (_copy_counter(inputs[2], "FETCH_SIZE") * 1024)
        ws = copy_bytes / (_copy_counter(inputs[3], "WRITE_SIZE") * 1024)
        print(f"# copy calibration: 1 GiB read and 1 GiB written per dispatch -> "
              f"FETCH_SIZE scale {fs:.6f}, WRITE_SIZE scale {ws:.6f}")
        print(f"sources_sha256: {fwd_sha}")
        print(f"bwd_sources_sha256: {bwd_sha}")
        print(f"fetch_scale: {fs:.6f}")
        print(f"write_scale: {ws:.6f}")
        tot = {}
        for k in sorted(set(fetch) | set(write)):
            rb, wb = fetch.get(k, 0.0) * 1024 * fs, write.get(k, 0.0) * 1024 * ws
            print(f"{k}: read_bytes {rb:.0f} write_bytes {wb:.0f} "
                  f"(FETCH_SIZE {fetch.get(k, 0.0):.0f} KiB, WRITE_SIZE {write.get(k, 0.0):.0f} KiB)")
            base = _kernel_base(k)
            for grp, names in (("fwd", FWD_KERNELS), ("bwd", BWD_KERNELS), ("decode", ("decode_kernel",))):
                if base in names:
                    tot[grp] = tot.get(grp, 0.0) + rb + wb
        kinds = {_kernel_base(k) for k in set(fetch) | set(write)}
        for grp, names in (("fwd", FWD_KERNELS), ("bwd", BWD_KERNELS), ("decode", ("decode_kernel",))):
            if any(n in kinds and n != "plan_kernel" for n in names):
                print(f"{grp}_traffic_bytes: {tot[grp]:.0f}")
    elif kind == "mfma":
        util = _counter_means(inputs[0], "MfmaUtil")
        mops = {c: _counter_means(inputs[1], c) for c in
                ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32")}
        print("# MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMD_NUM) (rocprofv3's "
              "derived metric); executed GFLOP = MOPS * 512 per dispatch")
        print(f"# forward/decode sources sha256: {fwd_sha}")
        print(f"# backward sources sha256: {bwd_sha}")
        print(f"# {'kernel':48s} {'MfmaUtil %':>10s} {'f16 GFLOP':>10s} {'bf16 GFLOP':>10s} {'f32 GFLOP':>10s}")
        for k in sorted(util):
            g = [mops[c].get(k, 0.0) * 512 / 1e9 for c in mops]
            print(f"  {k:48s} {util[k]:10.2f} {g[0]:10.1f} {g[1]:10.1f} {g[2]:10.1f}")
    elif kind == "counters":
        names = []
        for pattern in inputs:
            for r in _csv_rows(pattern):
                if r["Counter_Name"] not in names:
                    names.append(r["Counter_Name"])
        means = {}
        for c in names:
            for pattern in inputs:
                for k, v in _counter_means(pattern, c).items():
                    means.setdefault(k, {})[c] = v
        print(f"# forward/decode sources sha256: {fwd_sha}")
        print(f"# backward sources sha256: {bwd_sha}")
        print("# mean per dispatch, in millions")
        print(f"# {'kernel':48s} " + " ".join(f"{c:>28s}" for c in names))
        for k in sorted(means):
            print(f"  {k:48s} " + " ".join(f"{means[k].get(c, 0.0) / 1e6:28.3f}" for c in names))
    else:
        raise SystemExit(f"bench.py --summarize: unknown kind {kind}")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def copy_calibration(torch):
    n = 1 << 28                                   # 2^28 fp32 = 1 GiB
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 3}))


def measured_peaks(torch):
    """Achievable references on this GPU, reported beside the vendor peaks:
    a 512 MiB device-to-device copy (read + write bytes) and a dense bf16
    8192^3 matrix product through torch (hipBLASLt)."""
    res = {}
    n = 512 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        b.copy_(a)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    res["copy_GBps"] = round(2 * n * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    del a, b
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.mm(x, y)
    e0.record()
    for _ in range(10):
        torch.mm(x, y)
    e1.record()
    torch.cuda.synchronize()
    res["bf16_matmul_TFLOPs"] = round(2 * m ** 3 * 10 / (e0.elapsed_time(e1) / 1e3) / 1e12, 1)
    res["note"] = "achievable references measured on this GPU (copy = read + write bytes)"
    return res


def bench_bwd(kda, synth, torch, fi, wf, reps, warm):
    """Time kda_chunk_bwd on the forward workload's inputs (alpha gate, initial
    state, upstream dO and dS_T drawn N(0, 1)); outputs and workspace are
    allocated before timing."""
    B, T, H, Dk, Dv = wf.B, wf.T, wf.H, wf.Dk, wf.Dv
    up = synth.draw_upstream((B, T), B, H, Dk, Dv, wf.dtype, 1.0, 2, "cuda")
    nb = kda.kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, False, 0, 64, torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = {}

    def run():
        return kda.kda_chunk_bwd(fi["q"], fi["k"], fi["v"], fi["alpha"], fi["beta"], up["dout"],
                                 initial_state=fi["initial_state"], dfinal_state=up["dfinal_state"],
                                 workspace=ws, out=out)
    out = run()
    ms = time_events(run, reps, warm)
    units = B * H * T
    f16, f32 = bwd_flops_split(64, Dk, Dv)
    fl = (f16 + f32) * units
    peak = bwd_mixed_peak(64, Dk, Dv)
    tf = fl / (ms / 1e3) / 1e12
    byts = BWD_BYTES_PER_TOKEN_HEAD * units + 3 * B * H * Dk * Dv * 4
    del ws, out
    return {"value": round(units / (ms / 1e3), 1), "unit": "token-heads/s", "bwd_ms": round(ms, 3),
            "workspace_GiB": round(nb / 2 ** 30, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": round(peak, 1),
                         "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                         "dtype": "mixed: state passes and value side on the fp16 matrix cores "
                                  f"({f16 / (f16 + f32):.0%} of the flops, peak {BF16_MFMA_PEAK_TFLOPS:g}), "
                                  f"preparation and key side on fp32 (peak {FP32_MFMA_PEAK_TFLOPS:g}); "
                                  "peak = useful flops / their time with each part at its own peak",
                         "useful_flops_per_launch": round(fl)},
            "hbm_algorithmic": {"bytes_per_launch": byts,
                                "GBps": round(byts / (ms / 1e3) / 1e9, 1),
                                "traffic": measured_bwd_traffic(),
                                "traffic_unit": "bytes/launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated; "
                                                "null if the kernels changed since)"},
            "note": "gradients of sum(dO*o) + sum(dS_T*S_T) w.r.t. q, k, v, alpha, beta, S_0; "
                    "the forward is recomputed inside the call"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["fwd", "decode", "bwd"], default=None)
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize", choices=["trace", "traffic", "mfma", "counters"], default=None,
                    help="print a profiles/ summary from rocprofv3 CSV files (globs given by --inputs)")
    ap.add_argument("--inputs", nargs="*", default=[])
    ap.add_argument("--kernels", nargs="*", default=None,
                    help="--summarize trace: keep only these kernels (names without template arguments)")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the measured peaks and the other gate forms (profiler runs)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.inputs, args.title, args.command, args.kernels)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); a multi-GPU run is not part of it.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_12_amd as kda
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    kda.lib()                       # fail loudly if the HIP library is missing
    if args.copy_calibration:
        copy_calibration(torch)
        return

    K, W = args.steps, args.warmup
    dev = "cuda"
    wf = synth.WORKLOADS[2]
    wd = synth.WORKLOADS[3]
    do_fwd = args.only in (None, "fwd", "bwd")
    do_dec = args.only in (None, "decode")
    if args.only == "bwd":
        fi = synth.workload_inputs(2, device=dev)
        r = bench_bwd(kda, synth, torch, fi, wf, K, W)
        print(json.dumps({"metric": "KDA chunkwise backward token-heads/s", "n_gpus": 1, "steps": K,
                          "warmup": W, "bwd": r, "config": {"workload": wf.name, "chunk": 64}}))
        return

    # ---- inputs, outputs and workspace: all allocated before timing ----------
    if do_fwd:
        fi = synth.workload_inputs(2, device=dev)
        B, T, H, Dk, Dv = wf.B, wf.T, wf.H, wf.Dk, wf.Dv
        o = torch.empty((B, T, H, Dv), dtype=torch.bfloat16, device=dev)
        sT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        ws_bytes = kda.kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, False, 0, 64, torch.bfloat16)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def fwd():
            kda.kda_chunk_fwd(fi["q"], fi["k"], fi["v"], fi["alpha"], fi["beta"],
                              initial_state=fi["initial_state"], final_state=sT, o=o,
                              out_dtype=torch.bfloat16, workspace=ws)
    if do_dec:
        di = synth.workload_inputs(3, device=dev)
        state = di["state"].clone()
        od = torch.empty((wd.B, wd.H, wd.Dv), dtype=torch.bfloat16, device=dev)

        def dec(i):
            s = i % wd.steps
            kda.kda_recurrent_step(di["q"][s], di["k"][s], di["v"][s], di["alpha"][s],
                                   di["beta"][s], state, o=od, out_dtype=torch.bfloat16)

    # ---- warmup and timed loop ------------------------------------------------
    for i in range(W):
        if do_fwd:
            fwd()
        if do_dec:
            dec(i)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        if do_fwd:
            fwd()
        ev[i][1].record()
        if do_dec:
            dec(W + i)
        ev[i][2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) if do_fwd else None
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) if do_dec else None

    out = {"metric": "KDA fwd tokens/s (B*H*T/s) at d=128,T=64K; decode-step HBM GB/s",
           "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16xf32", "data": "synthetic"}
    cfg = {"workload": "", "chunk": 64}
    if do_fwd:
        units = wf.B * wf.H * wf.T
        fwd_s = fwd_ms / 1e3
        byts = FWD_BYTES_PER_TOKEN_HEAD * units + 2 * wf.B * wf.H * wf.Dk * wf.Dv * 4
        achieved = byts / fwd_s / 1e9
        out.update({"value": round(units / fwd_s, 1), "unit": "token-heads/s",
                    "fwd_ms": round(fwd_ms, 4)})
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                           "traffic": None, "kernel": "kda_chunk_fwd (plan+prep+state launches)",
                           "algorithmic_bytes_per_launch": byts}
        tflops = FWD_FLOPS_PER_TOKEN_HEAD * units / fwd_s / 1e12
        out["mfma"] = {"achieved_useful": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
        cfg["workload"] = wf.name
        cfg.update({"B": wf.B, "H": wf.H, "T": wf.T, "d_k": wf.Dk, "d_v": wf.Dv})
    else:
        out.update({"value": None, "unit": "token-heads/s"})
    if do_dec:
        dbytes = decode_bytes_per_step(wd.B, wd.H, wd.Dk, wd.Dv)
        gbps = dbytes / (dec_ms / 1e3) / 1e9
        out["decode"] = {"value": round(gbps, 1), "unit": "GB/s", "us_per_step": round(dec_ms * 1e3, 2),
                         "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                                      "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                                      "traffic": None, "kernel": "decode_kernel",
                                      "algorithmic_bytes_per_launch": dbytes}}
        cfg["decode_workload"] = wd.name
        if not do_fwd:
            cfg["workload"] = wd.name

    out["config"] = cfg

    # ---- parity and the CPU baseline: the fp64 oracle on the same inputs -------
    # The oracle runs on a bounded sample (by default the whole forward
    # workload: all heads, all tokens); its outputs check the timed forward
    # and decode results before any variant overwrites them.
    base = None
    o_ref = s_ref = None
    if not args.no_cpu_baseline and do_fwd:
        import oracle
        from tests.helpers import error_ratio
        S = min(args.cpu_sample_tokens, wf.T)
        sl = (slice(0, 1), slice(0, S))
        f64 = lambda x: x[sl].to("cpu").to(torch.float64).numpy()
        q, k, v, a, b = (f64(fi[key]) for key in ("q", "k", "v", "alpha", "beta"))
        s0 = fi["initial_state"].cpu().double().numpy()
        c0 = time.perf_counter()
        o_ref, s_ref, used = oracle.kda_fwd(q, k, v, a, b, initial_state=s0, return_threads=True)
        c1 = time.perf_counter()
        del q, k, v, a, b
        base = {"value": round(wf.H * S / (c1 - c0), 1), "unit": "token-heads/s", "cores": used,
                "kind": "oracle",
                "sample": f"first {S} of {wf.T} tokens, all {wf.H} heads of the forward workload "
                          f"(fp64 token-by-token recurrence, {c1 - c0:.2f} s)",
                "cpu": cpu_model()}
        full = S == wf.T
        out["parity"] = {
            "o": round(error_ratio(o[sl], o_ref, "bf16", stored_bf16=True), 4),
            "S_T": round(error_ratio(sT, s_ref, "bf16"), 4) if full else None,
            "unit": "max error / allowed error (<= 1 passes)",
            "tolerance": "max|err| <= 2e-2 x RMS(oracle) per tensor, plus half a bf16 ulp of each stored o",
            "reference": f"fp64 oracle on {'every element' if full else f'the first {S} tokens'} "
                         "of the timed forward's o and final state"}
        if not full:
            o_ref = s_ref = None        # the ablation below needs the whole reference
        if do_dec:
            s = W % wd.steps
            dq, dk, dv, da, db = (di[key][s].cpu().double().numpy()
                                  for key in ("q", "k", "v", "alpha", "beta"))
            dst = di["state"].cpu().double().numpy()
            c0 = time.perf_counter()
            od_ref, st_ref, dused = oracle.kda_step(dq, dk, dv, da, db, dst, return_threads=True)
            c1 = time.perf_counter()
            base["decode"] = {"value": round(decode_bytes_per_step(wd.B, wd.H, wd.Dk, wd.Dv)
                                             / (c1 - c0) / 1e9, 3),
                              "unit": "GB/s (fp32 byte ledger)", "cores": dused,
                              "sample": f"one full decode step ({c1 - c0:.2f} s)"}
            st_chk = di["state"].clone()
            od_chk = kda.kda_recurrent_step(di["q"][s], di["k"][s], di["v"][s], di["alpha"][s],
                                            di["beta"][s], st_chk, out_dtype=torch.bfloat16)
            torch.cuda.synchronize()
            out["decode"]["parity"] = {
                "o": round(error_ratio(od_chk, od_ref, "bf16", stored_bf16=True), 4),
                "state": round(error_ratio(st_chk, st_ref, "f32"), 4),
                "unit": "max error / allowed error (<= 1 passes)",
                "reference": "fp64 oracle step on all 8192 (sequence, head) pairs, from the workload's "
                             "initial state; state tolerance: fp32 (1e-4 relative)"}
            del dst, st_ref, st_chk
    if args.only is None and not args.no_variants:
        out["measured_peaks"] = measured_peaks(torch)
        # the other forget-gate forms on the same shapes (q, k, v, beta, states reused)
        var = {}
        units = wf.B * wf.H * wf.T
        for gate in ("softplus", "scalar"):
            g = synth.draw_gate(gate, (wf.B, wf.T), wf.H, wf.Dk, wf.mu, 2, dev)

            def fwd_g():
                kda.kda_chunk_fwd(fi["q"], fi["k"], fi["v"], g, fi["beta"],
                                  initial_state=fi["initial_state"], final_state=sT, o=o,
                                  out_dtype=torch.bfloat16, workspace=ws, gate=gate)
            ms = time_events(fwd_g, 10)
            byts = ((FWD_BYTES_PER_TOKEN_HEAD - GATE_BYTES["alpha"] + GATE_BYTES[gate]) * units
                    + 2 * wf.B * wf.H * wf.Dk * wf.Dv * 4)
            ach = byts / (ms / 1e3) / 1e9
            var[f"fwd_gate_{gate}"] = {"value": round(units / (ms / 1e3), 1), "unit": "token-heads/s",
                                       "fwd_ms": round(ms, 4),
                                       "roofline": {"bound": "hbm", "achieved": round(ach, 1),
                                                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                                    "frac": round(ach / HBM_PEAK_GBPS, 4),
                                                    "algorithmic_bytes_per_launch": byts}}
            del g
            gd = synth.draw_gate(gate, (wd.steps, wd.B), wd.H, wd.Dk, wd.mu, 3, dev)
            st2 = di["state"].clone()
            it = [0]

            def dec_g():
                s = it[0] % wd.steps
                it[0] += 1
                kda.kda_recurrent_step(di["q"][s], di["k"][s], di["v"][s], gd[s], di["beta"][s],
                                       st2, o=od, out_dtype=torch.bfloat16, gate=gate)
            ms = time_events(dec_g, 20)
            dbytes = decode_bytes_per_step(wd.B, wd.H, wd.Dk, wd.Dv, gate)
            gb = dbytes / (ms / 1e3) / 1e9
            var[f"decode_gate_{gate}"] = {"value": round(gb, 1), "unit": "GB/s",
                                          "us_per_step": round(ms * 1e3, 2),
                                          "roofline": {"bound": "hbm", "achieved": round(gb, 1),
                                                       "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                                       "frac": round(gb / HBM_PEAK_GBPS, 4),
                                                       "algorithmic_bytes_per_launch": dbytes}}
            del gd, st2
        var["note"] = ("forget gate given as the bf16 softplus pre-activation, or one fp32 alpha "
                       "per token and head; same shapes as the main lines")
        # chunk-size ablation: C = 32 and 128 run the generic fp32 path (C = 64 is the main line)
        for C in (32, 128):
            nbc = kda.kda_chunk_fwd_workspace_bytes(wf.B, wf.T, wf.H, wf.Dk, wf.Dv, False, 0, C, torch.bfloat16)
            wsc = torch.empty(nbc, dtype=torch.uint8, device=dev)

            def fwd_c():
                kda.kda_chunk_fwd(fi["q"], fi["k"], fi["v"], fi["alpha"], fi["beta"],
                                  initial_state=fi["initial_state"], final_state=sT, o=o,
                                  out_dtype=torch.bfloat16, workspace=wsc, chunk_size=C)
            ms = time_events(fwd_c, 5, 2)
            byts = FWD_BYTES_PER_TOKEN_HEAD * units + 2 * wf.B * wf.H * wf.Dk * wf.Dv * 4
            ach = byts / (ms / 1e3) / 1e9
            tf = fwd_flops_per_token_head(C, wf.Dk, wf.Dv) * units / (ms / 1e3) / 1e12
            par = None
            if o_ref is not None:
                fwd_c()
                torch.cuda.synchronize()
                par = {"o": round(error_ratio(o, o_ref, "bf16", stored_bf16=True), 4),
                       "S_T": round(error_ratio(sT, s_ref, "bf16"), 4)}
            var[f"fwd_chunk{C}"] = {"value": round(units / (ms / 1e3), 1), "unit": "token-heads/s",
                                    "fwd_ms": round(ms, 4), "workspace_GiB": round(nbc / 2 ** 30, 2),
                                    "parity": par,
                                    "roofline": {"bound": "hbm", "achieved": round(ach, 1),
                                                 "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                                 "frac": round(ach / HBM_PEAK_GBPS, 4),
                                                 "algorithmic_bytes_per_launch": byts},
                                    "mfma": {"achieved_useful": round(tf, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                                             "unit": "TFLOP/s", "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4),
                                             "dtype": "f32"}}
            del wsc
        var["chunk_note"] = ("chunk sizes 32 and 128 take the generic path (every product on the fp32 "
                             "matrix cores; at C = 32 the chain forms the output itself, at C = 128 an "
                             "output pass reads the stored state and U', fp16 with bf16 activations); "
                             "chunk 64 is the main line")
        # accuracy - memory - time of the chunk-size ablation, one row per C
        abl = {"64": {"fwd_ms": out["fwd_ms"], "workspace_GiB": round(ws_bytes / 2 ** 30, 2),
                      "parity": ({"o": out["parity"]["o"], "S_T": out["parity"]["S_T"]}
                                 if "parity" in out else None)}}
        for C in (32, 128):
            r = var[f"fwd_chunk{C}"]
            abl[str(C)] = {"fwd_ms": r["fwd_ms"], "workspace_GiB": r["workspace_GiB"], "parity": r["parity"]}
        var["chunk_ablation"] = {"rows": {c: abl[c] for c in ("32", "64", "128")},
                                 "parity_unit": "max error / allowed error against the fp64 oracle "
                                                "(bf16 o and fp32 final state of the forward workload)"}
        del o, sT, ws, fi
        torch.cuda.empty_cache()
        # the small dense workload (~0.1 GB, fits the 256 MB memory-side cache):
        # back to back ("hot"), and with a 512 MiB device write before each call
        # so that none of its inputs or records are still cached ("flushed")
        w1 = synth.WORKLOADS[1]
        f1 = synth.workload_inputs(1, device=dev)
        o1 = torch.empty((w1.B, w1.T, w1.H, w1.Dv), dtype=torch.bfloat16, device=dev)
        s1 = torch.empty((w1.B, w1.H, w1.Dk, w1.Dv), dtype=torch.float32, device=dev)
        ws1 = torch.empty(kda.kda_chunk_fwd_workspace_bytes(w1.B, w1.T, w1.H, w1.Dk, w1.Dv, False, 0, 64,
                                                            torch.bfloat16), dtype=torch.uint8, device=dev)

        def fwd1():
            kda.kda_chunk_fwd(f1["q"], f1["k"], f1["v"], f1["alpha"], f1["beta"], final_state=s1, o=o1,
                              out_dtype=torch.bfloat16, workspace=ws1)
        hot = time_events(fwd1, 50, 5)
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for n, (a, b) in enumerate(ev):
            scrub.fill_(n & 255)
            a.record()
            fwd1()
            b.record()
        torch.cuda.synchronize()
        cold = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
        u1 = w1.B * w1.H * w1.T
        b1 = FWD_BYTES_PER_TOKEN_HEAD * u1 + w1.B * w1.H * w1.Dk * w1.Dv * 4
        var["fwd_B2_H8_T4096"] = {
            "unit": "token-heads/s", "workload": w1.name, "algorithmic_bytes_per_launch": b1,
            "hot": {"value": round(u1 / (hot / 1e3), 1), "fwd_ms": round(hot, 4),
                    "hbm_frac": round(b1 / (hot / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "flushed": {"value": round(u1 / (cold / 1e3), 1), "fwd_ms": round(cold, 4),
                        "hbm_frac": round(b1 / (cold / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "note": "flushed: a 512 MiB device write before each timed call evicts the 256 MB memory-side cache"}
        del f1, o1, s1, ws1, scrub
        torch.cuda.empty_cache()
        # the packed variable-length workload: 64 sequences of 512..32768 tokens, 16 heads
        w4 = synth.WORKLOADS[4]
        f4 = synth.workload_inputs(4, device=dev)
        cu = f4["cu_seqlens"]
        T4 = f4["q"].shape[1]
        N4 = cu.numel() - 1
        o4 = torch.empty((1, T4, w4.H, w4.Dv), dtype=torch.bfloat16, device=dev)
        s4 = torch.empty((N4, w4.H, w4.Dk, w4.Dv), dtype=torch.float32, device=dev)
        ws4 = torch.empty(kda.kda_chunk_fwd_workspace_bytes(1, T4, w4.H, w4.Dk, w4.Dv, True, N4, 64,
                                                            torch.bfloat16), dtype=torch.uint8, device=dev)

        def fwd4():
            kda.kda_chunk_fwd(f4["q"], f4["k"], f4["v"], f4["alpha"], f4["beta"],
                              initial_state=f4["initial_state"], final_state=s4, cu_seqlens=cu, o=o4,
                              out_dtype=torch.bfloat16, workspace=ws4)
        ms4 = time_events(fwd4, 5, 2)
        u4 = w4.H * T4
        b4 = FWD_BYTES_PER_TOKEN_HEAD * u4 + 2 * N4 * w4.H * w4.Dk * w4.Dv * 4
        ach4 = b4 / (ms4 / 1e3) / 1e9
        var["fwd_varlen"] = {"value": round(u4 / (ms4 / 1e3), 1), "unit": "token-heads/s", "fwd_ms": round(ms4, 4),
                             "workload": w4.name, "tokens": T4, "sequences": N4,
                             "roofline": {"bound": "hbm", "achieved": round(ach4, 1), "peak": HBM_PEAK_GBPS,
                                          "unit": "GB/s", "frac": round(ach4 / HBM_PEAK_GBPS, 4),
                                          "algorithmic_bytes_per_launch": b4}}
        del f4, o4, s4, ws4, cu
        torch.cuda.empty_cache()
        fi = synth.workload_inputs(2, device=dev)
        var["bwd"] = bench_bwd(kda, synth, torch, fi, wf, 5, 2)
        out["variants"] = var
    traffic = measured_traffic()
    if traffic is not None:
        if do_fwd:
            out["roofline"]["traffic"] = traffic["fwd"]
            out["roofline"]["traffic_unit"] = "bytes/launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
        if do_dec:
            out["decode"]["roofline"]["traffic"] = traffic["decode"]
            out["decode"]["roofline"]["traffic_unit"] = "bytes/launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)"

    # ---- CPU baseline (the oracle runs above, with the parity checks) ---------
    if base is not None:
        import oracle
        if "variants" in out:
            Sb = min(4096, wf.T)
            slb = (slice(0, 1), slice(0, Sb))
            f64b = lambda x: x[slb].to("cpu").to(torch.float64).numpy()
            up = synth.draw_upstream((1, Sb), wf.B, wf.H, wf.Dk, wf.Dv, wf.dtype, 1.0, 2, "cpu")
            qb, kb, vb, ab, bb = (f64b(fi[key]) for key in ("q", "k", "v", "alpha", "beta"))
            dob = up["dout"].to(torch.float64).numpy()
            c0 = time.perf_counter()
            rb = oracle.kda_bwd(qb, kb, vb, ab, bb, dob, initial_state=s0,
                                dfinal_state=up["dfinal_state"].double().numpy())
            c1 = time.perf_counter()
            base["bwd"] = {"value": round(wf.H * Sb / (c1 - c0), 1), "unit": "token-heads/s",
                           "cores": rb["threads"], "kind": "oracle",
                           "sample": f"first {Sb} tokens, all {wf.H} heads, backward of the fp64 "
                                     f"recurrence ({c1 - c0:.2f} s)"}
            # the GPU backward on the same sample, against that oracle result
            from tests.helpers import error_ratio
            gs = lambda x: x[slb].contiguous()
            rg = kda.kda_chunk_bwd(gs(fi["q"]), gs(fi["k"]), gs(fi["v"]), gs(fi["alpha"]), gs(fi["beta"]),
                                   up["dout"].to(dev), initial_state=fi["initial_state"],
                                   dfinal_state=up["dfinal_state"].to(dev))
            torch.cuda.synchronize()
            par = {name: round(error_ratio(rg[name], rb[name], "bf16", stored_bf16=True), 4)
                   for name in ("dq", "dk", "dv")}
            par["dalpha"] = round(error_ratio(rg["dgate"], rb["dalpha"], "bf16"), 4)
            par["dbeta"] = round(error_ratio(rg["dbeta"], rb["dbeta"], "bf16"), 4)
            par["dS0"] = round(error_ratio(rg["dinitial_state"], rb["dinitial_state"], "bf16"), 4)
            par["unit"] = "max error / allowed error (<= 1 passes)"
            par["reference"] = (f"fp64 oracle backward on the first {Sb} tokens, all {wf.H} heads "
                                "(the CPU-baseline sample), against kda_chunk_bwd on the same sample")
            out["variants"]["bwd"]["parity"] = par
            del rg
        if np.isfinite(base["value"]) and out.get("value"):
            base["gpu_over_cpu"] = round(out["value"] / base["value"], 1)
        out["cpu_baseline"] = base

    print(json.dumps(out))


if __name__ == "__main__":
    main()
