#!/usr/bin/env python3
"""Benchmark of the quantized-weight prefill GEMM on one MI355X.

A step (the default workload, gate_up_T512_f16) is the fused gate/up SwiGLU GEMM of
one 512-token prefill chunk: Q4_0, 4096 -> 2 x 12288, f16 leg (fp16 inputs, fp32
accumulation), as pf_gemm_ws runs it: X rounded to fp16 once into the workspace
(pf_prepare_x), then the GEMM (pf_gemm_prepared); both calls are inside the step.
Inputs are synthetic (seeded N(0, 0.02) weights quantized to Q4_0 / Q8_0, N(0, 1)
activations) and resident in HBM before timing starts; the weights rotate over
enough copies (> 512 MB) that the 256 MB Infinity Cache does not hold them from
one step to the next.

Timing: --trials trials of --steps back-to-back steps, HIP events on the launch
stream around each trial and a synchronize on both sides; ms_per_step is the median
trial. Then each op, and the GEMM call of each op, run alone back to back for at
least --kernel-ms per trial (median of --trials): that gives the roofline entry of
the dominant kernel (its algorithmic FLOPs, or weight bytes where the weight stream
bounds it, over its average launch duration, against the MI355X spec peak). The
Q8_0 down projection with residual (12288 -> 4096) that follows in the FFN is timed
after the step, with it, as `ffn_chain`. The CPU oracle is timed on a bounded sample
of the step.

Prints one JSON line: value = FLOPs of the step / ms_per_step (TFLOP/s).

    python bench.py [--steps K] [--warmup W] [--trials N] [--workload NAME]
                    [--no-cpu-baseline] [--no-workspace]
    python bench.py --trace-summary KT_DIR | --traffic-summary F W CF CW |
                    --counter-summary PMC_DIR KT_DIR      (CPU only)
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill GEMM TFLOP/s at T=512 (Q4_0 4096->12288 gate/up); % MFMA peak"

# MI355X published peaks (dense): 256 CUs at 2.4 GHz.
PEAK = {
    "fp16_mfma_tflops": 2516.6,   # 256 CU x 4096 flop/clk x 2.4 GHz
    "fp32_mfma_tflops": 157.3,
    "hbm_gbs": 8000.0,
}

HIDDEN, INTER = 4096, 12288
VOCAB = 151936
LM_UNIQUE_ROWS = 16384  # lm_head weights: this many seeded rows, tiled to VOCAB
NORM_EPS = 1e-6
Q4_0, Q8_0, F16W, Q4_K, Q5_K, Q6_K, IQ4_XS = 0, 1, 2, 3, 4, 5, 6
PLAIN, RESIDUAL, SWIGLU = 0, 1, 2
BLOCK = {Q4_0: 18, Q8_0: 34, F16W: 64, Q4_K: 144, Q5_K: 176, Q6_K: 210, IQ4_XS: 136}
BLOCK_ELEMS = {Q4_0: 32, Q8_0: 32, F16W: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256, IQ4_XS: 256}


def weight_bytes(qtype, rows, k):
    return rows * (k // BLOCK_ELEMS[qtype]) * BLOCK[qtype]

# Sources whose change invalidates stored counter readings, per kernel family.
KERNEL_SOURCES = {
    "gemm_f16": ["pf_gemm_f16.hip", "pf_device.h"],
    "gemm_f32": ["pf_gemm_f32.hip", "pf_device.h"],
    "gemv": ["pf_gemv.hip", "pf_gemv_mfma.hip", "pf_device.h"],
    "xq": ["pf_xq.hip", "pf_device.h"],
}


def kernel_family(T, leg, qtype=0):
    if qtype not in (Q4_0, Q8_0):
        # on the f16 leg above the GEMV the further types take Q4_0's matrix-core GEMMs
        # (Q4_K, Q5_K, IQ4_XS and Q6_K with k % 512 == 0, as every workload here has, at
        # every T; F16 from 512 rows)
        return "gemm_f16" if leg == 1 and T > 8 and (qtype != F16W or T >= 512) else "xq"
    return "gemv" if T <= 8 else ("gemm_f16" if leg == 1 else "gemm_f32")


def kernel_source_sha(family):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "quantized_weight_prefill_gguf_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def gemv_sweep():
    """gemv_<qtype>_<n>x<k>_T<T>: one f32-leg PLAIN projection of T rows."""
    out = {}
    for qname, qtype in (("q4_0", Q4_0), ("q8_0", Q8_0)):
        for n, k, src in ((INTER, HIDDEN, "x"), (HIDDEN, INTER, "x12288")):
            for T in (1, 2, 4, 8):
                out["gemv_%s_%dx%d_T%d" % (qname, n, k, T)] = (
                    T, 0, [("gemv_" + qname, qtype, n, k, PLAIN, src, "out")], 1)
    return out


def workloads():
    """name -> (T, leg, ops, step_ops). op = (label, qtype, n, k, epilogue, input,
    output). A step is the first step_ops ops; any further ops are timed after the
    step, with it, as the FFN chain they form."""
    gu = ("gate_up_swiglu_q4_0", Q4_0, INTER, HIDDEN, SWIGLU, "x", "act")
    down = ("down_residual_q8_0", Q8_0, HIDDEN, INTER, RESIDUAL, "act", "res")
    return {
        # the metric's configuration: the fused gate/up SwiGLU GEMM at T = 512 (X
        # conversion included); the down projection follows as the FFN chain
        "gate_up_T512_f16": (512, 1, [gu, down], 1),
        "ffn_T512_f16": (512, 1, [gu, down], 2),
        "gate_up_T2048_f16": (2048, 1, [gu, down], 1),
        "ffn_T2048_f16": (2048, 1, [gu, down], 2),
        "down_T512_f16": (512, 1, [down], 1),
        # a short chunk (32 rows): the same two projections, bound by the weight stream
        "ffn_T32_f16": (32, 1, [gu, down], 2),
        # the FFN sublayer as the pages run it: RMSNorm, gate/up SwiGLU, down + residual,
        # with the norm inside the gate/up call (pf_gemm_rmsnorm)
        "ffn_rmsnorm_T512_f16": (512, 1, [
            ("rmsnorm_gate_up_swiglu_q4_0", Q4_0, INTER, HIDDEN, SWIGLU, "x", "act"), down], 2),
        "gate_up_T512_f32": (512, 0, [gu, down], 1),
        # the gate/up projection on a few rows (the GEMV twin's SwiGLU form)
        "gate_up_T4_f32": (4, 0, [gu], 1),
        "gate_up_T4_f16": (4, 1, [gu], 1),
        "gate_up_T8_f32": (8, 0, [gu], 1),
        "plain_q4_0_4096_T512_f16": (512, 1, [("plain_q4_0", Q4_0, HIDDEN, HIDDEN, PLAIN, "x", "out")], 1),
        "plain_q4_0_4096_T2048_f16": (2048, 1, [("plain_q4_0", Q4_0, HIDDEN, HIDDEN, PLAIN, "x", "out")], 1),
        # the small-T sweep: Q4_0 and Q8_0 at T in {1, 2, 4, 8} on both projection shapes
        **gemv_sweep(),
        # the further weight types (the same projections with F16 / Q4_K / Q6_K / IQ4_XS
        # weights)
        "gate_up_iq4_xs_T512_f16": (512, 1, [("gate_up_swiglu_iq4_xs", IQ4_XS, INTER, HIDDEN, SWIGLU, "x", "act")], 1),
        "gemv_iq4_xs_12288x4096_T1": (1, 0, [("gemv_iq4_xs", IQ4_XS, INTER, HIDDEN, PLAIN, "x", "out")], 1),
        "gate_up_q4_k_T512_f16": (512, 1, [("gate_up_swiglu_q4_k", Q4_K, INTER, HIDDEN, SWIGLU, "x", "act")], 1),
        "gate_up_q4_k_T512_f32": (512, 0, [("gate_up_swiglu_q4_k", Q4_K, INTER, HIDDEN, SWIGLU, "x", "act")], 1),
        "gate_up_q5_k_T512_f16": (512, 1, [("gate_up_swiglu_q5_k", Q5_K, INTER, HIDDEN, SWIGLU, "x", "act")], 1),
        "gate_up_f16w_T512_f16": (512, 1, [("gate_up_swiglu_f16w", F16W, INTER, HIDDEN, SWIGLU, "x", "act")], 1),
        "down_q6_k_T512_f16": (512, 1, [("down_residual_q6_k", Q6_K, HIDDEN, INTER, RESIDUAL, "act", "res")], 1),
        # the K-quant mix of a typical 4-bit file (gate/up Q4_K, down Q6_K) as the FFN at
        # 32 rows (the 4-wave GEMM's short-chunk tiles) and 512 (the cooperative kernel)
        "ffn_q4_k_q6_k_T32_f16": (32, 1, [("gate_up_swiglu_q4_k", Q4_K, INTER, HIDDEN, SWIGLU, "x", "act"),
                                          ("down_residual_q6_k", Q6_K, HIDDEN, INTER, RESIDUAL, "act", "res")], 2),
        "ffn_q4_k_q6_k_T512_f16": (512, 1, [("gate_up_swiglu_q4_k", Q4_K, INTER, HIDDEN, SWIGLU, "x", "act"),
                                            ("down_residual_q6_k", Q6_K, HIDDEN, INTER, RESIDUAL, "act", "res")], 2),
        "gemv_q4_k_12288x4096_T1": (1, 0, [("gemv_q4_k", Q4_K, INTER, HIDDEN, PLAIN, "x", "out")], 1),
        "gemv_q5_k_12288x4096_T1": (1, 0, [("gemv_q5_k", Q5_K, INTER, HIDDEN, PLAIN, "x", "out")], 1),
        "gemv_q6_k_4096x12288_T1": (1, 0, [("gemv_q6_k", Q6_K, HIDDEN, INTER, PLAIN, "x12288", "out")], 1),
        "gemv_q6_k_12288x4096_T1": (1, 0, [("gemv_q6_k", Q6_K, INTER, HIDDEN, PLAIN, "x", "out")], 1),
        "gemv_f16w_4096x12288_T1": (1, 0, [("gemv_f16w", F16W, HIDDEN, INTER, PLAIN, "x12288", "out")], 1),
        # the plain-read floor: one launch that only streams the same weight bytes as the
        # T = 1 GEMV of that shape (include/pf_probe.h)
        "read_floor_q4_0_12288x4096": (1, 0, [("read_floor_q4_0", Q4_0, INTER, HIDDEN, PLAIN, "x", "out")], 1),
        "read_floor_q8_0_4096x12288": (1, 0, [("read_floor_q8_0", Q8_0, HIDDEN, INTER, PLAIN, "x12288", "out")], 1),
        # lm_head GEMV on one row plus the greedy token (pf_lm_head_argmax); the pages
        # give no vocabulary size: 151936 rows stand in for it
        "lm_head_q8_0_151936x4096_T1": (1, 0, [("lm_head_q8_0", Q8_0, VOCAB, HIDDEN, PLAIN, "x", "logits")], 1),
        "lm_head_q4_0_151936x4096_T1": (1, 0, [("lm_head_q4_0", Q4_0, VOCAB, HIDDEN, PLAIN, "x", "logits")], 1),
    }


def op_rows(op):
    return 2 * op[2] if op[4] == SWIGLU else op[2]


def op_flops(op, T):
    return 2.0 * T * op_rows(op) * op[3]


def op_bytes(op, T):
    """Algorithmic HBM bytes of one launch: weight blocks once, X read, Y written
    (and read again for RESIDUAL)."""
    w = weight_bytes(op[1], op_rows(op), op[3])
    x = 4 * T * op[3]
    y = 4 * T * op[2] * (2 if op[4] == RESIDUAL else 1)
    return w + x + y


def cpu_baseline(T, ops, inputs, target_s=12.0):
    """The oracle, as it is, on a bounded sample: the same ops over the first t_s
    token rows (t_s chosen so that the run takes roughly target_s seconds)."""
    import numpy as np
    import oracle

    def run(ts):
        t0 = time.perf_counter()
        flops = 0.0
        for op in ops:
            label, qtype, n, k, epi, src, _ = op
            X = inputs[src][:ts]
            if label.startswith("rmsnorm_"):
                X = oracle.rmsnorm(X, inputs["norm_w"], NORM_EPS).astype(np.float32)
            R = inputs["res"][:ts] if epi == RESIDUAL else None
            Y = oracle.gemm(qtype, inputs["w_" + label], n, k, X, epi, R)
            if label.startswith("lm_head_"):
                oracle.argmax_last(Y[0].astype(np.float32))
            flops += op_flops(op, ts)
        return flops, time.perf_counter() - t0

    ts = min(T, 4)
    flops, dt = run(ts)
    if dt < target_s / 3 and ts < T:
        ts = int(min(T, max(ts + 1, ts * target_s / max(dt, 1e-3))))
        flops, dt = run(ts)
    reps = 1
    # The whole step is shorter than the target: repeat it (each run is the same work).
    while ts == T and dt < target_s * 0.8 and reps < 64:
        f2, d2 = run(ts)
        flops += f2
        dt += d2
        reps += 1
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "cpu": cpu,
        "kind": "oracle",
        "sample": "the step's %d ops on the first %d of %d token rows, %d run(s) (%.1f GFLOP, %.1f s)"
                  % (len(ops), ts, T, reps, flops / 1e9, dt),
    }


def load_traffic(workload, label, family, gemm_call_only=False):
    """HBM bytes per launch of the op from the stored counter passes (FETCH_SIZE and
    WRITE_SIZE, scaled by the copy calibration), or None when none were taken for
    this workload or the kernel sources changed since. gemm_call_only: leave out the
    X conversion kernels (the op's first call when it is timed as two)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload, {}).get(label)
    if not entry or entry.get("kernel_source_sha") != kernel_source_sha(family):
        return None
    if gemm_call_only:
        conv = ("x_to_frag_kernel", "x_to_f16_kernel")
        return sum(v["read_bytes"] + v["write_bytes"] for name, v in entry.get("kernels", {}).items()
                   if not name.startswith(conv))
    return entry.get("bytes_per_launch")


def copy_calibration(torch, mib=256, reps=3):
    """Plain device-to-device copies of `mib` MiB, each between buffers no cache
    holds (fresh pairs, > the 256 MB Infinity Cache apart). A counter pass over this
    run reads the known bytes, which scales the same counters for the GEMM."""
    n = mib * (1 << 20) // 4
    bufs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2 * reps)]
    for b in bufs:
        b.fill_(1.0)
    torch.cuda.synchronize()
    for r in range(reps):
        bufs[2 * r + 1].copy_(bufs[2 * r])
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "copies": reps, "bytes_read_per_copy": n * 4,
                      "bytes_written_per_copy": n * 4}), flush=True)


def _counter_csv(d):
    """{(dispatch id, kernel name): {counter: value}} from a rocprofv3 --pmc output
    directory (its *_counter_collection.csv, wherever rocprofv3 put it)."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    out = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                cs = out.setdefault(key, {})
                cs[r["Counter_Name"]] = cs.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _short_kernel(name):
    """'void pf::(anonymous namespace)::x_to_frag_kernel<1>(float const*, ...)' ->
    'x_to_frag_kernel<1>': no return type, namespaces or parameter list."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    return name[4:] if name.startswith("pf::") else name


def _op_of_kernel(short, ops):
    """Which op of a workload launched the library kernel `short` (None if not ours).
    Block-type templated kernels name the qtype first; split_sum_kernel names the
    epilogue; swiglu_apply_kernel belongs to the SwiGLU op."""
    import re
    m = re.match(r"(\w+)<(\d+)", short)
    base = m.group(1) if m else short
    for op in ops:
        if base == "split_sum_kernel":
            if int(m.group(2)) == op[4]:
                return op
        elif base == "swiglu_apply_kernel":
            if op[4] == SWIGLU:
                return op
        elif base in ("rms_inv_kernel", "rms_apply_kernel"):
            if op[0].startswith("rmsnorm_"):
                return op
        elif base == "argmax_kernel":
            if op[0].startswith("lm_head_"):
                return op
        elif base in ("x_to_frag_kernel", "x_to_f16_kernel", "gemm_f16_coop_kernel", "gemm_f16_kernel",
                      "gemm_f32_kernel", "gemv_kernel", "gemv_mfma_kernel") and m and int(m.group(2)) == op[1]:
            return op
    return None


def traffic_summary(workload, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """HBM bytes per launch of each op of `workload` from rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes over `bench.py --workload W`, each scaled by what the same
    counter reads for plain copies of known size (`bench.py --copy-calibration`).
    Updates profiles/traffic.json and prints a text summary. CPU only."""
    T, leg, ops, _ = workloads()[workload]
    cal_bytes = 256 * (1 << 20)
    cal = {}
    for cname, d in (("FETCH_SIZE", cal_fetch_dir), ("WRITE_SIZE", cal_write_dir)):
        vals = [cs[cname] for (_, kn), cs in _counter_csv(d).items() if "copyBuffer" in kn and cname in cs]
        cal[cname] = sum(vals) / len(vals)   # KiB per copy
    scale = {c: cal_bytes / (v * 1024.0) for c, v in cal.items()}
    per_kernel = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for (_, kn), cs in _counter_csv(d).items():
            short = _short_kernel(kn)
            if cname in cs and _op_of_kernel(short, ops) is not None:
                per_kernel.setdefault(short, {}).setdefault(cname, []).append(cs[cname] * 1024.0 * scale[cname])
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec["calibration"] = {"copy_bytes": cal_bytes, "fetch_size_kib": cal["FETCH_SIZE"],
                          "write_size_kib": cal["WRITE_SIZE"], "fetch_scale": scale["FETCH_SIZE"],
                          "write_scale": scale["WRITE_SIZE"]}
    wl = rec.setdefault("workloads", {})
    wl[workload] = {}
    lines = ["%-52s %12s %12s %12s" % ("kernel", "read MB", "write MB", "total MB")]
    for op in ops:
        total = 0.0
        kern = {}
        for short, cs in sorted(per_kernel.items()):
            if _op_of_kernel(short, ops) is not op:
                continue
            rd = sum(cs.get("FETCH_SIZE", [0.0])) / max(1, len(cs.get("FETCH_SIZE", [])))
            wr = sum(cs.get("WRITE_SIZE", [0.0])) / max(1, len(cs.get("WRITE_SIZE", [])))
            kern[short] = {"read_bytes": rd, "write_bytes": wr, "dispatches": len(cs.get("FETCH_SIZE", []))}
            total += rd + wr
            lines.append("%-52s %12.2f %12.2f %12.2f" % (short, rd / 1e6, wr / 1e6, (rd + wr) / 1e6))
        lines.append("%-52s %12s %12s %12.2f" % ("op " + op[0] + " (all its kernels)", "", "", total / 1e6))
        wl[workload][op[0]] = {"kernel_source_sha": kernel_source_sha(kernel_family(T, leg)),
                               "bytes_per_launch": total, "kernels": kern}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("Calibration: a plain device copy of 256 MiB reads FETCH_SIZE = %.1f KiB and WRITE_SIZE = "
          "%.1f KiB,\n  so FETCH_SIZE is scaled by %.4f and WRITE_SIZE by %.4f below.\n"
          % (cal["FETCH_SIZE"], cal["WRITE_SIZE"], scale["FETCH_SIZE"], scale["WRITE_SIZE"]))
    print("\n".join(lines))
    print("\nkernel_source_sha (%s): %s" % (" + ".join(KERNEL_SOURCES[kernel_family(T, leg)]),
                                           kernel_source_sha(kernel_family(T, leg))))


# Chip organisation used to turn chip-total counters into per-unit figures:
# 8 XCDs x 32 CUs x 4 SIMDs.
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def _trace_avg_ns(kt_dir):
    """{short kernel name: (calls, average ns)} from a --kernel-trace --stats run."""
    import csv
    import glob
    files = glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under %s" % kt_dir)
    out = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            out[_short_kernel(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]))
    return out


def counter_summary(workload, pmc_dir, kt_dir):
    """MFMA utilisation and shader clock of each op's GEMM kernel, CPU only: from a
    rocprofv3 --pmc pass with SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, SQ_CYCLES and
    GRBM_GUI_ACTIVE over `bench.py --workload W`, and the average launch duration of
    the same kernel from a --kernel-trace --stats run of the same command.

      sclk          = GRBM_GUI_ACTIVE / N_XCD / duration (GPU-busy cycles of one
                      XCD's clock over the launch)
      mfma_busy     = SQ_VALU_MFMA_BUSY_CYCLES / N_SIMD / (GRBM_GUI_ACTIVE / N_XCD)
      frac_at_sclk  = achieved / (spec peak x sclk / 2.4 GHz)

    Updates profiles/counters.json (keyed by the kernel sources' hash, as the
    traffic table) and prints the raw totals next to the derived figures."""
    T, leg, ops, _ = workloads()[workload]
    counters = _counter_csv(pmc_dir)
    trace = _trace_avg_ns(kt_dir)
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec["units"] = {"xcd": N_XCD, "cu": N_CU, "simd": N_SIMD, "spec_clock_ghz": 2.4}
    wl = rec.setdefault("workloads", {})
    wl[workload] = {}
    names = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_CYCLES", "GRBM_GUI_ACTIVE")
    peak = PEAK["fp16_mfma_tflops"] if leg == 1 else PEAK["fp32_mfma_tflops"]
    lines = ["%-46s %6s %11s %14s %14s %14s %14s %8s %9s %8s" % (
        "kernel", "disp", "avg_us", *names, "sclk", "mfma_busy", "frac@sclk")]
    gemm_kernels = ("gemm_f16_coop_kernel", "gemm_f16_kernel", "gemm_f32_kernel", "gemv_kernel",
                    "gemv_mfma_kernel")
    for op in ops:
        per = {}
        for (_, kn), cs in counters.items():
            short = _short_kernel(kn)
            if _op_of_kernel(short, ops) is op and short.startswith(gemm_kernels):
                per.setdefault(short, []).append(cs)
        for short, lst in sorted(per.items()):
            avg = {c: sum(cs.get(c, 0.0) for cs in lst) / len(lst) for c in names}
            if short not in trace:
                continue
            dur_ns = trace[short][1]
            cycles = avg["GRBM_GUI_ACTIVE"] / N_XCD
            sclk = cycles / dur_ns if dur_ns > 0 else 0.0
            busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cycles if cycles > 0 else 0.0
            achieved = op_flops(op, T) / (dur_ns * 1e-9) / 1e12
            frac_sclk = achieved / (peak * sclk / 2.4) if sclk > 0 else 0.0
            lines.append("%-46s %6d %11.2f %14.0f %14.0f %14.0f %14.0f %8.3f %9.3f %8.3f" % (
                short[:46], len(lst), dur_ns / 1e3, *[avg[c] for c in names], sclk, busy, frac_sclk))
            wl[workload][op[0]] = {"kernel_source_sha": kernel_source_sha(kernel_family(T, leg)),
                                   "kernel": short, "dispatches": len(lst), "avg_us": dur_ns / 1e3,
                                   "raw": avg, "sclk_ghz": sclk, "mfma_busy_frac": busy,
                                   "frac_of_spec_peak": achieved / peak, "frac_at_sclk": frac_sclk}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("Counters per dispatch (chip totals), averaged over the dispatches; sclk in GHz;\n"
          "mfma_busy = MFMA-busy cycles per SIMD over GPU-busy cycles per XCD.\n")
    print("\n".join(lines))
    print("\nkernel_source_sha (%s): %s" % (" + ".join(KERNEL_SOURCES[kernel_family(T, leg)]),
                                           kernel_source_sha(kernel_family(T, leg))))


def trace_summary(kt_dir):
    """CPU only: per-kernel launch statistics from a rocprofv3 --kernel-trace --stats
    output directory (its *kernel_stats.csv), in microseconds, with the median launch
    from the per-dispatch trace (*kernel_trace.csv) where it is there: the mean also
    averages the first, cold launches."""
    import csv
    import glob
    files = glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under %s" % kt_dir)
    durs = {}
    for tf in glob.glob(os.path.join(kt_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(tf) as fh:
            for r in csv.DictReader(fh):
                durs.setdefault(_short_kernel(r["Kernel_Name"]), []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("%-52s %8s %12s %12s %12s %12s %10s" % ("kernel", "calls", "avg_us", "median_us", "min_us", "max_us",
                                                   "std_us"))
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            name = _short_kernel(r["Name"])
            med = median(durs[name]) if name in durs else float("nan")
            print("%-52s %8d %12.2f %12.2f %12.2f %12.2f %10.2f" % (
                name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, med,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["StdDev"]) / 1e3))


def median(v):
    v = sorted(v)
    m = len(v) // 2
    return v[m] if len(v) % 2 else 0.5 * (v[m - 1] + v[m])


def load_counters(workload, label, family):
    """Stored counter-pass figures of the op's GEMM kernel (profiles/counters.json,
    written by --counter-summary), or None when none were taken for this workload or
    the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload, {}).get(label)
    if not entry or entry.get("kernel_source_sha") != kernel_source_sha(family):
        return None
    return {key: entry[key] for key in ("kernel", "mfma_busy_frac", "sclk_ghz", "frac_at_sclk")
            if key in entry}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed steps per trial")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--trials", type=int, default=5,
                    help="trials of --steps steps; the median trial is reported")
    ap.add_argument("--kernel-ms", type=float, default=200.0,
                    help="least GPU time per trial when an op or its GEMM call is timed alone")
    ap.add_argument("--workload", default="gate_up_T512_f16", choices=sorted(workloads()))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workspace", action="store_true",
                    help="call pf_gemm (X rounded inside the GEMM) instead of pf_gemm_ws")
    ap.add_argument("--single-call", action="store_true",
                    help="time each op as its one pf_gemm_ws call, not as pf_prepare_x then "
                         "pf_gemm_prepared")
    ap.add_argument("--rotate-mb", type=float, default=640.0,
                    help="minimum total bytes of rotated weight copies")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of a known size (the reference reading "
                         "for the FETCH_SIZE / WRITE_SIZE counters) and print them")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR",
                                                           "CAL_WRITE_DIR"),
                    help="CPU only: turn rocprofv3 FETCH_SIZE / WRITE_SIZE pass outputs over "
                         "--workload (and over --copy-calibration) into profiles/traffic.json")
    ap.add_argument("--counter-summary", nargs=2, metavar=("PMC_DIR", "KT_DIR"),
                    help="CPU only: turn a rocprofv3 --pmc pass (SQ_VALU_MFMA_BUSY_CYCLES "
                         "SQ_BUSY_CYCLES SQ_CYCLES GRBM_GUI_ACTIVE) and a --kernel-trace run over "
                         "--workload into profiles/counters.json")
    ap.add_argument("--trace-summary", metavar="KT_DIR",
                    help="CPU only: print the per-kernel table of a rocprofv3 --kernel-trace "
                         "--stats output directory")
    args = ap.parse_args()

    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.traffic_summary:
        traffic_summary(args.workload, *args.traffic_summary)
        return
    if args.counter_summary:
        counter_summary(args.workload, *args.counter_summary)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(each GPU would run its own independent share).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return

    import quantized_weight_prefill_gguf_amd as pf
    from quantized_weight_prefill_gguf_amd import synth

    pf.load()
    torch.cuda.set_device(0)
    T, leg, ops, step_ops = workloads()[args.workload]
    step = ops[:step_ops]

    # ---- inputs (host, seeded), then resident in HBM
    wid = 3
    inputs = {}
    for op in ops:
        label, qtype, n, k, epi, src, dst = op
        if epi == SWIGLU:
            inputs["w_" + label] = synth.gate_up_weight(qtype, n, k, workload_id=wid)
        elif label.startswith("lm_head_"):
            # quantising 620 M weights on the host takes minutes: seeded rows, tiled
            # (the timing does not depend on the values)
            base = synth.quantized_weight(qtype, LM_UNIQUE_ROWS, k, workload_id=wid).reshape(LM_UNIQUE_ROWS, -1)
            reps = -(-n // LM_UNIQUE_ROWS)
            inputs["w_" + label] = np.ascontiguousarray(np.tile(base, (reps, 1))[:n]).reshape(-1)
        else:
            tid = synth.TENSOR_W_DOWN if label.startswith("down") else synth.TENSOR_W
            inputs["w_" + label] = synth.quantized_weight(qtype, n, k, workload_id=wid, tensor_id=tid)
    inputs["x"] = synth.activations(T, HIDDEN, workload_id=wid)
    inputs["x12288"] = synth.activations(T, INTER, workload_id=wid)
    inputs["res"] = synth.activations(T, HIDDEN, workload_id=wid, tensor_id=synth.TENSOR_R)
    inputs["act"] = synth.activations(T, INTER, workload_id=wid, tensor_id=synth.TENSOR_W_UP)
    inputs["norm_w"] = np.random.default_rng([wid, 9]).uniform(0.5, 1.5, HIDDEN).astype(np.float32)

    log("inputs generated for %s" % args.workload)
    wbytes = sum(inputs["w_" + op[0]].size for op in ops)
    copies = max(2, int(np.ceil(args.rotate_mb * 1e6 / wbytes)) + 1)
    dev_w = [{op[0]: torch.from_numpy(inputs["w_" + op[0]]).cuda() for op in ops}]
    for _ in range(copies - 1):
        dev_w.append({key: t.clone() for key, t in dev_w[0].items()})
    bufs = {
        "x": torch.from_numpy(inputs["x"]).cuda(),
        "x12288": torch.from_numpy(inputs["x12288"]).cuda(),
        "act": torch.from_numpy(inputs["act"]).cuda(),
        "res": torch.from_numpy(inputs["res"]).cuda(),
        "out": torch.empty((T, max(HIDDEN, INTER)), dtype=torch.float32, device="cuda"),
        "norm_w": torch.from_numpy(inputs["norm_w"]).cuda(),
        "logits": torch.empty((VOCAB,), dtype=torch.float32, device="cuda"),
        "token": torch.zeros((1,), dtype=torch.int32, device="cuda"),
        "sink": torch.zeros((int(pf.load().pf_probe_read_sink_words()),), dtype=torch.int32, device="cuda"),
    }
    stream = torch.cuda.current_stream()
    use_ws = not args.no_workspace
    ws_bytes = max((pf.rmsnorm_workspace_bytes if op[0].startswith("rmsnorm_") else pf.workspace_bytes)(
        op[1], op[2], op[3], T, op[4], leg) for op in ops)
    workspace = (torch.empty(((ws_bytes + 15) // 16) * 16, dtype=torch.uint8, device="cuda")
                 if use_ws and ws_bytes > 0 else None)

    # Every call's ctypes arguments are marshalled once, here, so that the timed
    # loops are C-ABI calls only and a short kernel does not wait on Python.
    lib = pf.load()
    P = ctypes.c_void_p
    hstream = P(stream.cuda_stream)
    calls = {}
    for wset in range(copies):
        for op in ops:
            label, qtype, n, k, epi, src, dst = op
            Y = bufs[dst] if dst != "out" else bufs["out"].view(-1)[: T * n].view(T, n)
            w, x, y = P(dev_w[wset][label].data_ptr()), P(bufs[src].data_ptr()), P(Y.data_ptr())
            if label.startswith("read_floor_"):
                nb = weight_bytes(qtype, op_rows(op), k)
                calls[(op[0], wset)] = [(lib.pf_probe_read, (w, nb, P(bufs["sink"].data_ptr()), hstream))]
                continue
            if label.startswith("lm_head_"):
                pf.lm_head_argmax(qtype, dev_w[wset][label], n, k, bufs[src][0], bufs["logits"], bufs["token"])
                calls[(op[0], wset)] = [(lib.pf_lm_head_argmax, (
                    qtype, w, n, k, x, P(bufs["logits"].data_ptr()), P(bufs["token"].data_ptr()), hstream))]
                continue
            if label.startswith("rmsnorm_"):
                if workspace is None:
                    raise SystemExit("the RMSNorm prologue needs a workspace")
                pf.gemm_rmsnorm(qtype, dev_w[wset][label], n, k, bufs[src], bufs["norm_w"], NORM_EPS, Y, epi,
                                leg, workspace)
                calls[(op[0], wset)] = [(lib.pf_gemm_rmsnorm, (
                    qtype, w, n, k, x, T, P(bufs["norm_w"].data_ptr()), NORM_EPS, y, n, epi, leg,
                    P(workspace.data_ptr()), workspace.numel(), hstream))]
                continue
            # the checks the binding makes, once
            pf.gemm_ws(qtype, dev_w[wset][label], n, k, bufs[src], Y, epi, leg, workspace) if use_ws \
                else pf.gemm(qtype, dev_w[wset][label], n, k, bufs[src], Y, epi, leg)
            if use_ws and leg == 1 and qtype in (Q4_0, Q8_0) and not args.single_call and \
                    pf.select_path(qtype, n, k, T, epi, leg) == pf.PF_PATH_GEMM:
                # the same kernels as pf_gemm_ws in two calls, so that the GEMM's own
                # launch can be timed: X rounded to fp16 into the workspace, then the GEMM
                ws, wsb = P(workspace.data_ptr()), workspace.numel()
                calls[(op[0], wset)] = [(lib.pf_prepare_x, (qtype, k, x, T, ws, wsb, hstream)),
                                        (lib.pf_gemm_prepared, (qtype, w, n, k, T, y, n, epi, ws, wsb, hstream))]
            elif use_ws:
                ws = P(workspace.data_ptr()) if workspace is not None else P(0)
                wsb = workspace.numel() if workspace is not None else 0
                calls[(op[0], wset)] = [(lib.pf_gemm_ws, (qtype, w, n, k, x, T, y, epi, leg, ws, wsb, hstream))]
            else:
                calls[(op[0], wset)] = [(lib.pf_gemm, (qtype, w, n, k, x, T, y, epi, leg, hstream))]
    torch.cuda.synchronize()

    def run(fn, argv):
        st = fn(*argv)
        if st != 0:
            raise pf.PfError(st, fn.__name__)

    def launch(op, wset, parts=None):
        """The op's C-ABI calls (or the listed ones only)."""
        cl = calls[(op[0], wset)]
        for i in (range(len(cl)) if parts is None else parts):
            run(*cl[i])

    newev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(body, count, trials):
        """Median over trials of the GPU time of `count` back-to-back bodies, in ms per
        body: HIP events on the launch stream around each trial, a synchronize on
        both sides."""
        per = []
        for tr in range(trials):
            e0, e1 = newev(), newev()
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(count):
                body(tr * count + i)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / count)
        return median(per), per

    for i in range(args.warmup):
        for op in ops:
            launch(op, i % copies)
    torch.cuda.synchronize()
    log("warmup done (%d weight copies)" % copies)

    # ---- the timed region: trials x K steps (a step = the workload's first step_ops
    # ops, each its C-ABI calls), each trial bracketed by a synchronize.
    def one_step(i):
        for op in step:
            launch(op, i % copies)

    t0 = time.perf_counter()
    ms_per_step, trial_ms = timed(one_step, args.steps, args.trials)
    elapsed = time.perf_counter() - t0
    log("timed region done: %.4f ms/step (trials %s)" % (ms_per_step, ", ".join("%.4f" % v for v in trial_ms)))

    # ---- each op alone, and each op's last call alone (the GEMM, when X is converted
    # by a call of its own), back to back for at least --kernel-ms per trial.
    def count_for(ms_est):
        return int(max(100, min(20000, np.ceil(args.kernel_ms / max(ms_est, 1e-4)))))

    op_ms, kern_ms, kern_launches = [], [], []
    for op in ops:
        nparts = len(calls[(op[0], 0)])
        est, _ = timed(lambda i: launch(op, i % copies), 20, 1)
        m, _ = timed(lambda i: launch(op, i % copies), count_for(est), args.trials)
        op_ms.append(m)
        if nparts > 1:
            launch(op, 0, range(nparts - 1))  # the prepared X the GEMM call reads
            last = [nparts - 1]
            est, _ = timed(lambda i: launch(op, i % copies, last), 20, 1)
            cnt = count_for(est)
            m, _ = timed(lambda i: launch(op, i % copies, last), cnt, args.trials)
        else:
            cnt = count_for(est)
        kern_ms.append(m)
        kern_launches.append(cnt)
    log("per-op timing done")

    chain = None
    if len(ops) > step_ops:
        def one_chain(i):
            for op in ops:
                launch(op, i % copies)
        c_ms, _ = timed(one_chain, max(args.steps, 20), args.trials)
        cflops = sum(op_flops(op, T) for op in ops)
        chain = {"ops": [op[0] for op in ops], "ms": c_ms, "tflops": cflops / (c_ms * 1e-3) / 1e12}

    step_flops = sum(op_flops(op, T) for op in step)
    dom = int(np.argmax(kern_ms[:step_ops]))
    dop = step[dom]
    nparts_dom = len(calls[(dop[0], 0)])
    family = kernel_family(T, leg, dop[1])
    # the bound is whichever takes longer at peak: streaming the weights once from HBM,
    # or the op's matrix-core flops (the GEMV, and the GEMM on short chunks, are HBM-bound)
    wbytes = weight_bytes(dop[1], op_rows(dop), dop[3])
    mfma_peak = PEAK["fp16_mfma_tflops"] if leg == 1 else PEAK["fp32_mfma_tflops"]
    hbm_bound = wbytes / (PEAK["hbm_gbs"] * 1e9) > op_flops(dop, T) / (mfma_peak * 1e12)
    traffic = load_traffic(args.workload, dop[0], family, nparts_dom > 1)
    if hbm_bound:
        achieved = wbytes / (kern_ms[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK["hbm_gbs"], "unit": "GB/s",
                    "frac": achieved / PEAK["hbm_gbs"], "traffic": traffic}
        op_frac = wbytes / (op_ms[dom] * 1e-3) / 1e9 / PEAK["hbm_gbs"]
    else:
        achieved = op_flops(dop, T) / (kern_ms[dom] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": mfma_peak, "unit": "TFLOP/s",
                    "frac": achieved / mfma_peak, "traffic": traffic}
        op_frac = op_flops(dop, T) / (op_ms[dom] * 1e-3) / 1e12 / mfma_peak
    roofline["kernel"] = dop[0] + (" (GEMM call)" if nparts_dom > 1 else "")
    roofline["avg_launch_us"] = kern_ms[dom] * 1e3
    roofline["launches_per_trial"] = kern_launches[dom]
    roofline["trials"] = args.trials
    roofline["op_us"] = op_ms[dom] * 1e3
    roofline["op_frac"] = op_frac
    roofline["counters"] = load_counters(args.workload, dop[0], family)

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    unit = "TFLOP/s"
    if all(op[0].startswith("read_floor_") for op in step):
        # a plain read moves bytes, not FLOPs: the value is the weight bytes per second
        value = sum(weight_bytes(op[1], op_rows(op), op[3]) for op in step) / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if leg == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "hidden": HIDDEN, "intermediate": INTER,
                   "leg": "f16" if leg == 1 else "f32",
                   "step": [op[0] for op in step],
                   "frac_of_peak": (value / mfma_peak) if not hbm_bound else None,
                   "trials": args.trials, "trial_ms_per_step": trial_ms,
                   "timed_wall_s": elapsed,
                   "ops": [{"op": op[0], "n": op[2], "k": op[3], "avg_us": op_ms[j] * 1e3,
                            "gemm_call_us": kern_ms[j] * 1e3,
                            "tflops": op_flops(op, T) / (op_ms[j] * 1e-3) / 1e12,
                            "gbs": op_bytes(op, T) / (op_ms[j] * 1e-3) / 1e9,
                            "calls": [fn.__name__ for fn, _ in calls[(op[0], 0)]]}
                           for j, op in enumerate(ops)],
                   "weight_copies": copies,
                   "workspace_bytes": ws_bytes if use_ws else 0},
        "roofline": roofline,
    }
    if chain is not None:
        out["ffn_chain"] = chain
    if not args.no_cpu_baseline and not any(op[0].startswith("read_floor_") for op in step):
        out["cpu_baseline"] = cpu_baseline(T, step, inputs)
        log("cpu baseline done")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
