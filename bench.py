#!/usr/bin/env python3
"""Benchmark of the NVFP4 quantized-linear hot path on one MI355X.

A step is one pass of the whole path over the 3B model's FFN at 8192 tokens (hidden 3072,
FFN 9216), the workload the headline metric is quoted on:
  forward   Q(X) rowwise RNE + columnwise RHT16 copy, Q(W_up) 16x16 2D (both copies),
            GEMM H = bf16(X W_up^T) (8192x9216x3072) with its tile maxima, Q(H) rowwise
            (its tensor amax from those maxima: H is read once), Q(W_down) 2D,
            GEMM Y_down = H W_down^T (8192x3072x9216)
  backward  Q(dY) rowwise SR + columnwise RHT16 SR, dgrad GEMM dX = dY W_up
            (8192x3072x9216), wgrad GEMM dW = dY^T X on the rotated copies (9216x3072x8192)
  optimizer Q-AdamW second moment v (9216x3072) encode + decode
  decode    dequantize of the W_up rowwise copy to FP32
All inputs are seeded synthetic tensors resident in HBM before timing starts.

Output: one JSON line.  value = total GEMM FLOPs of a step / step time (TFLOP/s, all
quantization, optimizer-state and decode kernels included).  Per-kernel times come from
HIP events recorded on the stream the kernels are launched on.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 quantize GB/s + W4A4 GEMM TFLOP/s at 8192×3072×9216 (% of roofline)"
PEAK_HBM_GBPS = 8000.0
PEAK_F16_TFLOPS = 2500.0   # dense f16/bf16 MFMA, MI355X
PEAK_FP4_TFLOPS = 10100.0  # dense FP4 MFMA, MI355X: the hardware ceiling of a 4-bit GEMM
TOKENS, HIDDEN, FFN = 8192, 3072, 9216
SEED_WGRAD, SEED_QADAMW = 0x5EED4, 0x5EED5


def qbytes(n, k):
    """Bytes of one NVFP4 copy of an n x k matrix: codes, E4M3 scales, tensor scale."""
    return n * k // 2 + n * k // 16 + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager launches instead of replays of a HIP graph")
    ap.add_argument("--cpu-sample-rows", type=int, default=8192,
                    help="rows of X for the oracle's bounded CPU sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write profiles/ffn3b_step_kernel_stats.txt from a rocprofv3 "
                         "--kernel-trace --stats folder of one bench run")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="write profiles/gemm_mfma_busy.txt from a rocprofv3 --pmc GRBM_GUI_ACTIVE "
                         "SQ_VALU_MFMA_BUSY_CYCLES --kernel-trace folder of one bench step")
    ap.add_argument("--valu-summary", metavar="DIR",
                    help="write profiles/valu_busy.txt from a rocprofv3 --pmc GRBM_GUI_ACTIVE "
                         "SQ_INSTS_VALU SQ_ACTIVE_INST_VALU --kernel-trace folder of one bench step")
    ap.add_argument("--counter-summary", nargs=4, metavar="DIR",
                    help="write profiles/hbm_counters.txt from rocprofv3 --pmc folders: "
                         "FETCH_SIZE and WRITE_SIZE of one bench step, then of --copy-calibration")
    return ap.parse_args()


# Source files that define each kernel family, hashed together so that a counter entry is
# used only while none of them has changed.
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_quantize_amd", "csrc")
SOURCES = {
    "gemm": ["gemm.hip", "device_common.h"],
    "quant": ["quantize.hip", "quantize_kernels.h", "quantize_launch_bf16_lo.hip",
              "quantize_launch_bf16_hi.hip", "quantize_launch_f32_lo.hip",
              "quantize_launch_f32_hi.hip", "device_common.h"],
    "qadamw": ["qadamw.hip", "quantize_kernels.h", "device_common.h"],
}
FAMILY = {"gemm": "gemm", "quant": "quant", "qadamw_encode": "qadamw", "qadamw_decode": "qadamw",
          "qadamw_step": "qadamw", "dequant": "quant"}
# kernels each call of the step launches, in order (name prefixes; '?' marks optional)
CALL_KERNELS = {"quant": ["?k_amax", "k_encode|k_quant"], "gemm": ["k_gemm", "?k_gemm_half"],
                "qadamw_encode": ["k_qv_pass1", "k_max_partials", "k_qv_pass2"],
                "qadamw_decode": ["k_qv_decode"],
                "qadamw_step": ["k_qs_pass1", "k_max_partials", "k_qs_pass2"],
                "dequant": ["k_dequant"]}


STEP_ORDER = [("quant_X_row+colRHT", "quant"), ("quant_Wup_2d", "quant"), ("gemm_ffn_up", "gemm"),
              ("quant_H_row", "quant"), ("quant_Wdown_2d", "quant"), ("gemm_ffn_down", "gemm"),
              ("quant_dY_rowSR+colRHTSR", "quant"), ("gemm_dgrad", "gemm"), ("gemm_wgrad", "gemm"),
              ("qadamw_encode", "qadamw_encode"), ("qadamw_decode", "qadamw_decode"),
              ("qadamw_step_Wup", "qadamw_step"), ("dequant_Wup", "dequant")]


def split_step(names):
    """Assign dispatch names (our kernels only, in order) to the step's calls; returns
    [(key, [dispatch indices])] per call, for every whole step present.  Set-up launches
    before the first step and the extra measurements after the last are skipped."""
    def one_step(i):
        got = []
        for key, kind in STEP_ORDER:
            idx = []
            for pat in CALL_KERNELS[kind]:
                alts = pat.lstrip("?").split("|")
                if i < len(names) and any(a in names[i] for a in alts):
                    idx.append(i)
                    i += 1
                elif not pat.startswith("?"):
                    return None, i
            got.append((key, idx))
        return got, i

    out, i = [], 0
    while i < len(names):
        got, j = one_step(i)
        if got is None:
            if out:
                break
            i += 1
            continue
        out += got
        i = j
    if not out:
        raise SystemExit("no whole step found in the dispatch list")
    return out


def trace_summary(d):
    """Write profiles/ffn3b_step_kernel_stats.txt from a rocprofv3 --kernel-trace --stats
    folder of `bench.py --steps 10 --warmup 2 --no-cpu-baseline`: the per-kernel statistics
    and, from the dispatch trace, the average duration of each call of the step."""
    import csv
    import glob as _glob
    stats = list(csv.DictReader(open(_glob.glob(os.path.join(d, "*kernel_stats.csv"))[0])))
    raw = list(csv.DictReader(open(_glob.glob(os.path.join(d, "*kernel_trace.csv"))[0])))
    trace = [r for r in raw if "nvfp4::" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace]
    per = {}
    for key, idx in split_step([r["Kernel_Name"] for r in trace]):
        per.setdefault(key, []).append(sum(dur[i] for i in idx))
    lines = ["# rocprofv3 kernel-trace summary: 3B FFN linear hot-path step (bench.py workload)",
             "# commands (from the repository root on one MI355X; cd /tmp && TMPDIR=/tmp first):",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d <kt> -o bench \\",
             "#       -- python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline",
             "#   python3 bench.py --trace-summary <kt>",
             "# per kernel (all steps, warm-up included):",
             f"# {'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}"]
    alld = {}
    for r in raw:
        alld.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for r in stats:
        v = sorted(alld.get(r["Name"], [])) or [float("nan")]
        lines.append(f"{r['Name'][:62]:62s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{v[len(v) // 2]:9.2f} {int(r['MinNs']) / 1e3:9.2f} {int(r['MaxNs']) / 1e3:9.2f} "
                     f"{float(r['Percentage']):7.2f}")
    lines.append("# per call of the step (sum of its kernels' durations), from the dispatch trace:")
    lines.append(f"# {'call':28s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for key, _ in STEP_ORDER:
        v = sorted(per.get(key, []))
        if v:
            lines.append(f"{key:30s} {len(v):6d} {sum(v) / len(v):9.2f} {v[len(v) // 2]:9.2f} "
                         f"{min(v):9.2f} {max(v):9.2f}")
    out = os.path.join(ROOT, "profiles", "ffn3b_step_kernel_stats.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def source_digest(family):
    h = hashlib.sha256()
    for f in SOURCES[family]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def counters_for(key, kind):
    """HBM bytes per launch (fetch + write) from the committed rocprofv3 counter summary, or
    None if a source of that kernel changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.txt")
    if not os.path.exists(path):
        return None
    digest = source_digest(FAMILY[kind])
    for line in open(path):
        t = line.split()
        if len(t) >= 4 and not line.startswith("#") and t[0] == key and t[1] == digest:
            return float(t[2]) + float(t[3])
    return None


def counter_summary(dirs):
    """Write profiles/hbm_counters.txt from four rocprofv3 --pmc output folders: FETCH_SIZE and
    WRITE_SIZE of `bench.py --steps 1 --warmup 0 --no-cpu-baseline`, then of
    `bench.py --copy-calibration`.  Counters are KiB per dispatch (summed over the L2
    instances); each is scaled by (bytes a plain 256 MiB device copy moves) / (what the same
    counter reads for that copy)."""
    import csv
    import glob as _glob

    def per_dispatch(d):
        f = _glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
        agg, name = {}, {}
        for r in csv.DictReader(open(f)):
            k = int(r["Dispatch_Id"])
            agg[k] = agg.get(k, 0.0) + float(r["Counter_Value"])
            name[k] = r["Kernel_Name"]
        return [(name[k], agg[k] * 1024.0) for k in sorted(agg)]

    fetch, write, cfetch, cwrite = (per_dispatch(d) for d in dirs)
    copy_bytes = 256 << 20
    fc = [v for n, v in cfetch if "copyBuffer" in n or "copy" in n.lower()]
    wc = [v for n, v in cwrite if "copyBuffer" in n or "copy" in n.lower()]
    f_scale = copy_bytes / (sum(fc[-5:]) / 5)
    w_scale = copy_bytes / (sum(wc[-5:]) / 5)
    ours = [(n, fv, wv) for (n, fv), (_, wv) in zip(fetch, write) if "nvfp4::" in n]
    order = STEP_ORDER
    lines = ["# HBM traffic per launch from rocprofv3 --pmc (TCC FETCH_SIZE, WRITE_SIZE; one pass each)",
             "# commands (from the repository root, cd /tmp && TMPDIR=/tmp first):",
             "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <f> -o bench -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --eager",
             "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <w> -o bench -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --eager",
             "#   rocprofv3 --pmc FETCH_SIZE ... -d <cf> -o copy -- python3 bench.py --copy-calibration   (and WRITE_SIZE -> <cw>)",
             "#   python3 bench.py --counter-summary <f> <w> <cf> <cw>",
             f"# calibration: a 256 MiB device copy reads {sum(fc[-5:]) / 5 / 2**20:.1f} MiB FETCH_SIZE and "
             f"{sum(wc[-5:]) / 5 / 2**20:.1f} MiB WRITE_SIZE -> scale fetch x{f_scale:.3f}, write x{w_scale:.3f}",
             "# key  source-digest  fetch_bytes  write_bytes  (per launch, calibrated)"]
    kinds = dict(order)
    for key, idx in split_step([n for n, _, _ in ours])[:len(order)]:
        fb = sum(ours[i][1] for i in idx)
        wb = sum(ours[i][2] for i in idx)
        lines.append(f"{key} {source_digest(FAMILY[kinds[key]])} {fb * f_scale:.0f} {wb * w_scale:.0f}")
    out = os.path.join(ROOT, "profiles", "hbm_counters.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma_summary(d):
    """Write profiles/gemm_mfma_busy.txt from a rocprofv3 --pmc GRBM_GUI_ACTIVE
    SQ_VALU_MFMA_BUSY_CYCLES --kernel-trace folder of `bench.py --steps 1 --warmup 1
    --no-cpu-baseline`: per GEMM call of the last step (the first one also pays the process's
    first launches), the duration under counter collection, the
    effective clock (GRBM_GUI_ACTIVE over the eight XCDs / duration) and the fraction of SIMD
    cycles the matrix cores were busy (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles))."""
    import csv
    import glob as _glob
    agg, name = {}, {}
    for r in csv.DictReader(open(_glob.glob(os.path.join(d, "*counter_collection.csv"))[0])):
        k = int(r["Dispatch_Id"])
        agg.setdefault(k, {}).setdefault(r["Counter_Name"], 0.0)
        agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
        name[k] = r["Kernel_Name"]
    dur = {}
    for r in csv.DictReader(open(_glob.glob(os.path.join(d, "*kernel_trace.csv"))[0])):
        dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    ids = [k for k in sorted(agg) if "nvfp4::" in name[k]]
    lines = ["# Matrix-core busy fraction and effective clock of the step's GEMMs (rocprofv3 --pmc)",
             "# commands (from the repository root, cd /tmp && TMPDIR=/tmp first):",
             "#   rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES --kernel-trace --output-format csv \\",
             "#       -d <m> -o bench -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --eager",
             "#   python3 bench.py --mfma-summary <m>   (the last of the two steps)",
             "# clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs",
             "# x GRBM_GUI_ACTIVE / 8); durations are longer than uncounted ones (collection overhead)",
             f"# {'call':16s} {'kernel':28s} {'us':>8s} {'clock_GHz':>10s} {'mfma_busy':>10s}"]
    kinds = dict(STEP_ORDER)
    for key, idx in split_step([name[k] for k in ids])[-len(STEP_ORDER):]:
        if kinds[key] != "gemm":
            continue
        for i in idx:
            k = ids[i]
            cyc = agg[k].get("GRBM_GUI_ACTIVE", 0.0) / 8
            t = dur.get(k, float("nan"))
            busy = agg[k].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * cyc) if cyc else float("nan")
            lines.append(f"{key:18s} {name[k].split('(')[0].replace('void nvfp4::', ''):28s} {t * 1e6:8.1f} "
                         f"{cyc / t / 1e9:10.2f} {busy:10.3f}")
    out = os.path.join(ROOT, "profiles", "gemm_mfma_busy.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# input elements of each non-GEMM call of the step
CALL_ELEMS = {"quant_X_row+colRHT": TOKENS * HIDDEN, "quant_Wup_2d": FFN * HIDDEN,
              "quant_H_row": TOKENS * FFN, "quant_Wdown_2d": HIDDEN * FFN,
              "quant_dY_rowSR+colRHTSR": TOKENS * FFN, "qadamw_encode": FFN * HIDDEN,
              "qadamw_decode": FFN * HIDDEN, "qadamw_step_Wup": FFN * HIDDEN,
              "dequant_Wup": FFN * HIDDEN}


def valu_summary(d):
    """Write profiles/valu_busy.txt from a rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_INSTS_VALU
    SQ_ACTIVE_INST_VALU --kernel-trace folder of `bench.py --steps 1 --warmup 0
    --no-cpu-baseline`.  Per kernel of each non-GEMM call of the step:
      valu/elem   vector instructions per input element, SQ_INSTS_VALU x 64 lanes / elements;
      issue_us    their issue time at 2 cycles per wave64 instruction on each of the 1024
                  SIMDs at the 2.4 GHz peak clock (the rate of fp32 adds and integer adds with
                  two or more waves per SIMD on gfx950; 64-bit integer products take about 4
                  cycles, square roots and reciprocals about 8, and one wave alone issues at
                  most every 4-5 cycles);
      issue/us    the share of the kernel's time those issue cycles fill."""
    import csv
    import glob as _glob
    agg, name = {}, {}
    for r in csv.DictReader(open(_glob.glob(os.path.join(d, "*counter_collection.csv"))[0])):
        k = int(r["Dispatch_Id"])
        agg.setdefault(k, {}).setdefault(r["Counter_Name"], 0.0)
        agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
        name[k] = r["Kernel_Name"]
    dur = {}
    for r in csv.DictReader(open(_glob.glob(os.path.join(d, "*kernel_trace.csv"))[0])):
        dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    ids = [k for k in sorted(agg) if "nvfp4::" in name[k]]
    clk, cyc = 2.4e9, 2
    lines = ["# Vector-ALU work of the step's quantize, optimizer-state and decode kernels (rocprofv3 --pmc)",
             "# commands (from the repository root, cd /tmp && TMPDIR=/tmp first):",
             "#   rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_ACTIVE_INST_VALU --kernel-trace \\",
             "#       --output-format csv -d <v> -o bench -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --eager",
             "#   python3 bench.py --valu-summary <v>",
             "# valu/elem = SQ_INSTS_VALU x 64 / input elements; issue_us = SQ_INSTS_VALU x 2 cycles / 1024 SIMDs",
             "# / 2.4 GHz (fp32-add rate; 64-bit integer products ~4 cycles, sqrt/rcp ~8); issue/us = issue_us / us.",
             "# Durations are under counter collection, somewhat longer than uncounted ones.",
             f"# {'call':24s} {'kernel':24s} {'us':>7s} {'valu/elem':>10s} {'issue_us':>9s} {'issue/us':>9s}"]
    kinds = dict(STEP_ORDER)
    for key, idx in split_step([name[k] for k in ids])[:len(STEP_ORDER)]:
        if kinds[key] == "gemm":
            continue
        for i in idx:
            k = ids[i]
            t = dur.get(k, float("nan"))
            insts = agg[k].get("SQ_INSTS_VALU", 0.0)
            issue = insts * cyc / 1024 / clk
            kern = name[k].split("(")[0].replace("void ", "").replace("nvfp4::", "")
            lines.append(f"{key:26s} {kern:24s} {t * 1e6:7.1f} {insts * 64 / CALL_ELEMS[key]:10.1f} "
                         f"{issue * 1e6:9.1f} {issue / t:9.2f}")
    out = os.path.join(ROOT, "profiles", "valu_busy.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.valu_summary:
        valu_summary(args.valu_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU path is a design note only)", file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_block_scaled_quantize_amd as nv
    from nvfp4_block_scaled_quantize_amd import synthetic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nv.load_library()
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 256 << 20, "launches": 5}))
        return

    # ------------------------------------------------------------ inputs (seeded, in HBM)
    ffn = synthetic.ffn()
    wg = synthetic.wgrad()
    X = ffn["X"].to(dev)
    W_up = ffn["W_up"].to(dev)
    W_down = ffn["W_down"].to(dev)
    dY = wg["dY"].to(dev)
    v = synthetic.qadamw()["v"].to(dev)

    P = nv.quant_params
    p_x = P(rowwise=True, colwise=True, rht_col=True, seed=SEED_WGRAD)
    p_w = P(rowwise=True, colwise=True, block2d=True)
    p_h = P(rowwise=True)
    p_wd = P(rowwise=True, block2d=True)
    p_dy = P(rowwise=True, colwise=True, round_row=nv.NVFP4_SR, round_col=nv.NVFP4_SR,
             rht_col=True, seed=SEED_WGRAD)

    def alloc(R, C, params):
        row = nv.QTensor.empty(R, C, dev) if params.rowwise else None
        col = nv.QTensor.empty(C, R, dev) if params.colwise else None
        ws = torch.empty(max(nv.nvfp4_quantize_workspace_bytes(R, C, params), 16),
                         dtype=torch.uint8, device=dev)
        return row, col, ws

    qx = alloc(TOKENS, HIDDEN, p_x)
    qw = alloc(FFN, HIDDEN, p_w)
    qh = alloc(TOKENS, FFN, p_h)
    qwd = alloc(HIDDEN, FFN, p_wd)
    qdy = alloc(TOKENS, FFN, p_dy)
    H = torch.empty((TOKENS, FFN), dtype=torch.bfloat16, device=dev)   # the up projection's output
    T_up = torch.empty((nv.load_library().nvfp4_gemm_tiles(TOKENS, FFN),), dtype=torch.float32,
                       device=dev)
    Y_down = torch.empty((TOKENS, HIDDEN), dtype=torch.float32, device=dev)
    dX = torch.empty((TOKENS, HIDDEN), dtype=torch.float32, device=dev)
    dW = torch.empty((FFN, HIDDEN), dtype=torch.float32, device=dev)
    mu = torch.empty((FFN // 16, HIDDEN // 16), dtype=torch.int16, device=dev)
    qv = nv.QTensor.empty(FFN, HIDDEN, dev)
    ws_v = torch.empty(max(nv.qadamw_v_workspace_bytes(FFN, HIDDEN), 16), dtype=torch.uint8,
                       device=dev)
    v_out = torch.empty_like(v)
    w_dec = torch.empty((FFN, HIDDEN), dtype=torch.float32, device=dev)
    # full Q-AdamW step on W_up: fp32 master weights, bf16 gradient, states out of place
    w_master = W_up.float()
    g_up = synthetic.normal((FFN, HIDDEN), SEED_QADAMW + 1, 1e-3).to(torch.bfloat16).to(dev)
    p_step = nv.qadamw_step_params(1.5e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, 1 / (1 - 0.9 ** 10),
                                   1 / (1 - 0.95 ** 10), m_rht_seed=SEED_WGRAD, m_sr_seed=SEED_WGRAD + 1,
                                   v_seed=SEED_QADAMW, v_use_signs=True)
    ws_step = torch.empty(max(nv.qadamw_step_workspace_bytes(FFN, HIDDEN), 16), dtype=torch.uint8,
                          device=dev)
    z = nv.QTensor(torch.zeros((FFN, HIDDEN // 2), dtype=torch.uint8, device=dev),
                   torch.zeros((FFN, HIDDEN // 16), dtype=torch.uint8, device=dev),
                   torch.ones((1,), device=dev))
    zmu = torch.zeros((FFN // 16, HIDDEN // 16), dtype=torch.int16, device=dev)
    # one step from the zero state gives the (non-trivial) states every timed step reads
    st_m, st_mu, st_v = nv.qadamw_step(w_master, g_up, z, zmu, z, p_step, workspace=ws_step)
    st_m2, st_mu2, st_v2 = (nv.QTensor.empty(FFN, HIDDEN, dev), torch.empty_like(zmu),
                            nv.QTensor.empty(FFN, HIDDEN, dev))

    # name -> (kind, algorithmic bytes, flops)
    work = {
        "quant_X_row+colRHT": ("quant", 2 * TOKENS * HIDDEN + 2 * qbytes(TOKENS, HIDDEN), 0),
        "quant_Wup_2d": ("quant", 2 * FFN * HIDDEN + 2 * qbytes(FFN, HIDDEN), 0),
        "gemm_ffn_up": ("gemm", qbytes(TOKENS, HIDDEN) + qbytes(FFN, HIDDEN) + 2 * TOKENS * FFN
                        + 4 * (TOKENS // 256) * (FFN // 256), 2 * TOKENS * FFN * HIDDEN),
        "quant_H_row": ("quant", 2 * TOKENS * FFN + qbytes(TOKENS, FFN), 0),
        "quant_Wdown_2d": ("quant", 2 * HIDDEN * FFN + qbytes(HIDDEN, FFN), 0),
        "gemm_ffn_down": ("gemm", qbytes(TOKENS, FFN) + qbytes(HIDDEN, FFN) + 4 * TOKENS * HIDDEN,
                          2 * TOKENS * HIDDEN * FFN),
        "quant_dY_rowSR+colRHTSR": ("quant", 2 * TOKENS * FFN + 2 * qbytes(TOKENS, FFN), 0),
        "gemm_dgrad": ("gemm", qbytes(TOKENS, FFN) + qbytes(HIDDEN, FFN) + 4 * TOKENS * HIDDEN,
                       2 * TOKENS * HIDDEN * FFN),
        "gemm_wgrad": ("gemm", qbytes(FFN, TOKENS) + qbytes(HIDDEN, TOKENS) + 4 * FFN * HIDDEN,
                       2 * FFN * HIDDEN * TOKENS),
        "qadamw_encode": ("quant", 4 * FFN * HIDDEN + qbytes(FFN, HIDDEN) + FFN * HIDDEN // 128, 0),
        "qadamw_decode": ("quant", qbytes(FFN, HIDDEN) + FFN * HIDDEN // 128 + 4 * FFN * HIDDEN, 0),
        # g bf16 in, w f32 in and out, both states in and out
        "qadamw_step_Wup": ("quant", 2 * FFN * HIDDEN + 8 * FFN * HIDDEN
                            + 2 * (2 * qbytes(FFN, HIDDEN) + FFN * HIDDEN // 128), 0),
        "dequant_Wup": ("quant", qbytes(FFN, HIDDEN) + 4 * FFN * HIDDEN, 0),
    }

    def calls():
        yield "quant_X_row+colRHT", lambda: nv.nvfp4_quantize(X, p_x, qx[0], qx[1], qx[2])
        yield "quant_Wup_2d", lambda: nv.nvfp4_quantize(W_up, p_w, qw[0], qw[1], qw[2])
        yield "gemm_ffn_up", lambda: nv.nvfp4_gemm_bf16(qx[0], qw[0], out=H, tile_amax=T_up)
        yield "quant_H_row", lambda: nv.nvfp4_quantize(H, p_h, qh[0], None, amax_parts=T_up)
        yield "quant_Wdown_2d", lambda: nv.nvfp4_quantize(W_down, p_wd, qwd[0], None, qwd[2])
        yield "gemm_ffn_down", lambda: nv.nvfp4_gemm(qh[0], qwd[0], out=Y_down)
        yield "quant_dY_rowSR+colRHTSR", lambda: nv.nvfp4_quantize(dY, p_dy, qdy[0], qdy[1], qdy[2])
        yield "gemm_dgrad", lambda: nv.nvfp4_gemm(qdy[0], qw[1], out=dX)
        yield "gemm_wgrad", lambda: nv.nvfp4_gemm(qdy[1], qx[1], out=dW)
        yield "qadamw_encode", lambda: nv.qadamw_v_encode(v, SEED_QADAMW, True, mu, qv, ws_v)
        yield "qadamw_decode", lambda: nv.qadamw_v_decode(mu, qv, SEED_QADAMW, True, out=v_out)
        yield "qadamw_step_Wup", lambda: nv.qadamw_step(w_master, g_up, st_m, st_mu, st_v, p_step,
                                                        st_m2, st_mu2, st_v2, ws_step)
        yield "dequant_Wup", lambda: nv.nvfp4_dequantize(qw[0], out=w_dec)

    stream = torch.cuda.current_stream(dev)

    def step(record):
        for name, fn in calls():
            if record is None:
                fn()
            else:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record(stream)
                fn()
                e.record(stream)
                record.append((name, s, e))

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    # per-call times: K eager steps with HIP events between the calls
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_eager = (t1 - t0) * 1e3 / args.steps
    # the step time: the same step captured once as a HIP graph, W replays, then K timed
    # replays (eager launches with --eager, or if the capture is refused)
    timing = {"mode": "eager", "eager_ms_per_step": round(ms_eager, 4)}
    ms_per_step = ms_eager
    if not args.eager:
        try:
            ms_graph = graph_step(torch, step, args.steps, args.warmup)
            timing = {"mode": "hip_graph", "eager_ms_per_step": round(ms_eager, 4),
                      "graph_ms_per_step": round(ms_graph, 4)}
            ms_per_step = ms_graph
        except RuntimeError as exc:
            timing["graph_error"] = str(exc)[:200]

    per = {}
    for name, s, e in events:
        per.setdefault(name, []).append(s.elapsed_time(e))
    kernels = {}
    for name, (kind, nbytes, flops) in work.items():
        ms = sum(per[name]) / len(per[name])
        d = {"ms": round(ms, 5)}
        if kind == "gemm":
            d["TFLOP/s"] = round(flops / ms / 1e9, 1)
            d["frac_f16_peak"] = round(flops / ms / 1e9 / PEAK_F16_TFLOPS, 4)
            d["frac_fp4_peak"] = round(flops / ms / 1e9 / PEAK_FP4_TFLOPS, 4)
        d["GB/s"] = round(nbytes / ms / 1e6, 1)
        if kind == "quant":
            d["frac_hbm_peak"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4)
        kernels[name] = d

    gemm_flops = sum(f for k, b, f in work.values())
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12
    q_names = [n for n, (k, b, f) in work.items() if k == "quant"]
    q_bytes = sum(work[n][1] for n in q_names)
    q_ms = sum(kernels[n]["ms"] for n in q_names)
    up = kernels["gemm_ffn_up"]
    up_flops = work["gemm_ffn_up"][2]
    roofline = {"bound": "mfma", "kernel": "k_gemm_dma<EpiBf16> + k_gemm_half (FFN-up 8192x9216x3072, "
                                                 "bf16 out: 4 whole rounds of 256x256 tiles, then "
                                                 "the last 128 tiles as 256 half-width tiles)",
                "achieved": up["TFLOP/s"], "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(up["TFLOP/s"] / PEAK_F16_TFLOPS, 4),
                "traffic": counters_for("gemm_ffn_up", "gemm")}
    xq = kernels["quant_X_row+colRHT"]
    roofline_quant = {"bound": "hbm", "kernel": "k_amax+k_encode (X 8192x3072 bf16, row + col RHT)",
                      "achieved": xq["GB/s"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(xq["GB/s"] / PEAK_HBM_GBPS, 4),
                      "traffic": counters_for("quant_X_row+colRHT", "quant")}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "3B FFN linear hot path: 8192 tokens, hidden 3072, FFN 9216; "
                               "fwd up (bf16 H with tile maxima) + down, "
                               "bwd up (dgrad, wgrad with RHT16+SR), "
                               "Q-AdamW v 9216x3072 encode+decode, W_up dequantize",
                   "tokens": TOKENS, "hidden": HIDDEN, "ffn": FFN,
                   "gemm_shapes_MxNxK": ["8192x9216x3072", "8192x3072x9216", "8192x3072x9216",
                                         "9216x3072x8192"],
                   "parallelism": "single GPU"},
        "headline": {"gemm_ffn_up_TFLOP/s": up["TFLOP/s"],
                     "quantize_X_GB/s": xq["GB/s"],
                     "quantize_all_GB/s": round(q_bytes / q_ms / 1e6, 1)},
        "roofline": roofline,
        "roofline_quantize": roofline_quant,
        "kernels": kernels,
    }

    out["step_timing"] = timing
    out["qadamw_v_error"] = qadamw_error(nv, torch, v, v_out)
    out["kernels_isolated"] = isolated(torch, dev, calls, work, stream)
    out["extras"] = extras(nv, synthetic, torch, dev, X, dY, p_x, p_dy, qx, qdy, qw, stream)
    # each memory-bound kernel's rate also as a fraction of what a plain device copy reaches
    copy_gbps = out["extras"]["hbm_copy_256MiB"]["GB/s"]
    out["copy_rate_GB/s"] = copy_gbps
    for name, (kind, nbytes, flops) in work.items():
        if kind != "gemm":
            kernels[name]["frac_copy_rate"] = round(kernels[name]["GB/s"] / copy_gbps, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, synthetic, ffn)
    print(json.dumps(out))


def graph_step(torch, step, steps, warmup):
    """ms per step of the step captured once into a HIP graph (every call is allocation-,
    memset- and synchronisation-free) and replayed: W untimed replays, then K timed ones
    bracketed by device synchronisations."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(None)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(None)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def qadamw_error(nv, torch, v, v_hat):
    """Reconstruction error of the Q-AdamW second moment (v 9216 x 3072, the step's GPU
    encode and decode) beside direct NVFP4 1x16 RNE quantization of the same v (GPU
    quantize and dequantize): Rel. MSE = MSE(v - v_hat) / mean(v^2) (Full-Stack FP4 sec. 3.2's
    definition), the median, 99th percentile and mean of |v_hat - v| / v, the fraction of
    elements decoded as 0, and the Rel. MSE of sqrt(v), the quantity the update divides by.
    Measurement only (binary64 on the device), outside the timed region."""
    q, _ = nv.nvfp4_quantize(v, nv.quant_params(rowwise=True))
    v_direct = nv.nvfp4_dequantize(q)
    v64 = v.double().flatten()
    n = v64.numel()

    def metrics(vh):
        vh = vh.double().flatten()
        e = vh - v64
        rel = (e.abs() / v64).sort().values
        se = vh.clamp(min=0).sqrt() - v64.sqrt()
        return {"rel_mse": float((e * e).mean() / (v64 * v64).mean()),
                "median_rel_err": float(rel[n // 2]),
                "p99_rel_err": float(rel[min(n - 1, (99 * n) // 100)]),
                "mean_rel_err": float(rel.mean()),
                "zero_fraction": float((vh == 0).double().mean()),
                "rel_mse_sqrt_v": float((se * se).mean() / v64.mean())}

    return {"workload": "v fp32 9216x3072 log-normal exp(-18 + 3 N(0,1))",
            "pipeline": metrics(v_hat), "direct_nvfp4": metrics(v_direct)}


def isolated(torch, dev, calls, work, stream, reps=10):
    """Each call of the step on its own, median of `reps` HIP-event timings: cold (512 MiB
    of scratch written before every call, so the 256 MB last-level cache holds none of its
    inputs) and warm (the call repeated back to back, inputs left in the caches)."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    res = {}
    for name, fn in calls():
        kind, nbytes, flops = work[name]
        times = {}
        for mode in ("cold", "warm"):
            ev = []
            fn()
            for i in range(reps):
                if mode == "cold":
                    scratch.fill_(i & 0xFF)
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record(stream)
                fn()
                e.record(stream)
                ev.append((s, e))
            torch.cuda.synchronize()
            t = sorted(s.elapsed_time(e) for s, e in ev)
            times[mode] = t[len(t) // 2]
        d = {"cold_ms": round(times["cold"], 5), "warm_ms": round(times["warm"], 5)}
        if kind == "gemm":
            d["cold_TFLOP/s"] = round(flops / times["cold"] / 1e9, 1)
            d["warm_TFLOP/s"] = round(flops / times["warm"] / 1e9, 1)
        else:
            d["cold_GB/s"] = round(nbytes / times["cold"] / 1e6, 1)
            d["warm_GB/s"] = round(nbytes / times["warm"] / 1e6, 1)
        res[name] = d
    return res


def extras(nv, synthetic, torch, dev, X, dY, p_x, p_dy, qx, qdy, qw, stream, iters=20):
    """Measurements outside the step, same method (HIP events on the launch stream):
    the X and dY quantizes with 4/6 adaptive block scaling; eq. (2)'s Wgrad operand of X
    requantized from the rowwise copy; one NVFP4 Newton-Schulz iteration (3072 x 9216); the
    LoRA-SVD branch at rank 64
    (X quantize with the L1 down-projection fused, FFN-up GEMM with the L2 up-projection
    fused, and for dX the dY quantize with L2^T and the dgrad GEMM with L1^T); the
    QKV-projection GEMM of the 3B model; a plain device copy for the device's achievable HBM
    bandwidth; and, as context only, the platform's dense f16 GEMM on the FFN-up shape."""
    qkv = synthetic.qkv()
    Xq, Wqkv = qkv["X"].to(dev), qkv["W"].to(dev)
    p46x = nv.quant_params(rowwise=True, colwise=True, rht_col=True, seed=SEED_WGRAD, scale46=True)
    p46dy = nv.quant_params(rowwise=True, colwise=True, round_row=nv.NVFP4_SR,
                            round_col=nv.NVFP4_SR, rht_col=True, seed=SEED_WGRAD, scale46=True)
    pq = nv.quant_params(rowwise=True)
    qa, _ = nv.nvfp4_quantize(Xq, pq)
    qb, _ = nv.nvfp4_quantize(Wqkv, pq)
    C = torch.empty((Xq.shape[0], Wqkv.shape[0]), dtype=torch.float32, device=dev)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    M, K = Xq.shape
    N = Wqkv.shape[0]
    lo = synthetic.lora()
    R = lo["L1"].shape[0]
    L1 = lo["L1"].to(dev)                                # [r][hidden]
    L2 = lo["L2"].to(dev)                                # [ffn][r]
    L1T = lo["L1"].t().contiguous().to(dev)              # [hidden][r]
    L2T = lo["L2"].t().contiguous().to(dev)              # [r][ffn]
    tx = torch.empty((TOKENS, R), dtype=torch.bfloat16, device=dev)
    tdy = torch.empty((TOKENS, R), dtype=torch.bfloat16, device=dev)
    wsx = torch.empty(nv.load_library().nvfp4_quantize_lora_workspace_bytes(TOKENS, HIDDEN, R),
                      dtype=torch.uint8, device=dev)
    wsdy = torch.empty(nv.load_library().nvfp4_quantize_lora_workspace_bytes(TOKENS, FFN, R),
                       dtype=torch.uint8, device=dev)
    nv.nvfp4_quantize_lora(X, p_x, L1, lo["beta"], qx[0], qx[1], tx, wsx)
    nv.nvfp4_quantize_lora(dY, p_dy, L2T, lo["beta"], qdy[0], qdy[1], tdy, wsdy)
    p_req = nv.quant_params(rowwise=False, colwise=True, rht_col=True, round_col=nv.NVFP4_SR,
                            seed=SEED_WGRAD)
    qreq = nv.QTensor.empty(HIDDEN, TOKENS, dev)
    wsreq = torch.empty(max(nv.load_library().nvfp4_requantize_cols_workspace_bytes(TOKENS, HIDDEN), 16),
                        dtype=torch.uint8, device=dev)
    Xns = synthetic.normal((HIDDEN, FFN), SEED_QADAMW + 7, 1.0 / (HIDDEN ** 0.5 + FFN ** 0.5)).to(dev)
    wsns = torch.empty(nv.load_library().nvfp4_ns_step_workspace_bytes(HIDDEN, FFN), dtype=torch.uint8,
                       device=dev)
    Yl = torch.empty((TOKENS, FFN), dtype=torch.float32, device=dev)
    g16 = torch.Generator(device=dev).manual_seed(SEED_QADAMW + 9)
    a16 = torch.randn((TOKENS, HIDDEN), generator=g16, device=dev, dtype=torch.float16)
    b16 = torch.randn((HIDDEN, FFN), generator=g16, device=dev, dtype=torch.float16)   # K-major, contiguous
    c16 = torch.empty((TOKENS, FFN), dtype=torch.float16, device=dev)
    dXl = torch.empty((TOKENS, HIDDEN), dtype=torch.float32, device=dev)
    H16 = torch.empty((TOKENS, FFN), dtype=torch.bfloat16, device=dev)
    T16 = torch.empty((nv.load_library().nvfp4_gemm_tiles(TOKENS, FFN),), dtype=torch.float32,
                      device=dev)
    cases = {
        "quant_X_row+colRHT_4/6": (lambda: nv.nvfp4_quantize(X, p46x, qx[0], qx[1], qx[2]),
                                   2 * TOKENS * HIDDEN + 2 * qbytes(TOKENS, HIDDEN), 0),
        "quant_dY_rowSR+colRHTSR_4/6": (lambda: nv.nvfp4_quantize(dY, p46dy, qdy[0], qdy[1], qdy[2]),
                                        2 * TOKENS * FFN + 2 * qbytes(TOKENS, FFN), 0),
        "quant_X_row+colRHT_lora_r64": (
            lambda: nv.nvfp4_quantize_lora(X, p_x, L1, lo["beta"], qx[0], qx[1], tx, wsx),
            2 * TOKENS * HIDDEN + 2 * qbytes(TOKENS, HIDDEN) + 2 * TOKENS * R + 2 * R * HIDDEN,
            2 * TOKENS * HIDDEN * R),
        "gemm_ffn_up_lora_r64": (lambda: nv.nvfp4_gemm_lora(qx[0], qw[0], tx, L2, out=Yl),
                                 qbytes(TOKENS, HIDDEN) + qbytes(FFN, HIDDEN) + 4 * TOKENS * FFN
                                 + 2 * TOKENS * R + 2 * FFN * R,
                                 2 * TOKENS * FFN * HIDDEN + 2 * TOKENS * FFN * R),
        "quant_dY_rowSR+colRHTSR_lora_r64": (
            lambda: nv.nvfp4_quantize_lora(dY, p_dy, L2T, lo["beta"], qdy[0], qdy[1], tdy, wsdy),
            2 * TOKENS * FFN + 2 * qbytes(TOKENS, FFN) + 2 * TOKENS * R + 2 * R * FFN,
            2 * TOKENS * FFN * R),
        "gemm_dgrad_lora_r64": (lambda: nv.nvfp4_gemm_lora(qdy[0], qw[1], tdy, L1T, out=dXl),
                                qbytes(TOKENS, FFN) + qbytes(HIDDEN, FFN) + 4 * TOKENS * HIDDEN
                                + 2 * TOKENS * R + 2 * HIDDEN * R,
                                2 * TOKENS * HIDDEN * FFN + 2 * TOKENS * HIDDEN * R),
        # eq. (2): the Wgrad operand of X from its rowwise copy (column RHT, SR)
        "requant_X_cols_from_rowcopy": (
            lambda: nv.nvfp4_requantize_cols(qx[0], p_req, qreq, wsreq),
            2 * qbytes(TOKENS, HIDDEN), 0),
        # NVFP4 Root: one quantized Newton-Schulz iteration on W_up's 3072 x 9216 orientation
        # (three quantizes, A = qX qX^T, B = b A + c qA qA', X = a X + qB qX')
        "ns_step_3072x9216": (lambda: nv.nvfp4_ns_step(Xns, 1.5, -0.5, 0.0, SEED_WGRAD, True, wsns),
                              0, 2 * HIDDEN * HIDDEN * (2 * FFN + HIDDEN)),
        "gemm_qkv_8192x6144x3072": (lambda: nv.nvfp4_gemm(qa, qb, out=C),
                                    qbytes(M, K) + qbytes(N, K) + 4 * M * N, 2 * M * N * K),
        "hbm_copy_256MiB": (lambda: dst.copy_(src), 2 * (256 << 20), 0),
        # the FFN-up GEMM timed like the next line (back to back), for a like-for-like view:
        # FP32 output (balanced schedule) and bf16 output with tile maxima (the step's)
        "gemm_ffn_up_back_to_back": (lambda: nv.nvfp4_gemm(qx[0], qw[0], out=Yl), 0,
                                     2 * TOKENS * FFN * HIDDEN),
        "gemm_ffn_up_bf16_back_to_back": (lambda: nv.nvfp4_gemm_bf16(qx[0], qw[0], out=H16, tile_amax=T16),
                                          0, 2 * TOKENS * FFN * HIDDEN),
        # context, not part of the path: the platform library's dense f16 GEMM (torch.matmul,
        # hipBLASLt) on the FFN-up shape with contiguous operands, the practical ceiling of
        # the f16 datapath on this part
        "context_f16_matmul_8192x9216x3072": (lambda: torch.matmul(a16, b16, out=c16), 0,
                                              2 * TOKENS * FFN * HIDDEN),
    }
    res = {}
    for name, (fn, nbytes, flops) in cases.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(iters):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / iters
        d = {"ms": round(ms, 5), "GB/s": round(nbytes / ms / 1e6, 1)}
        if flops and name.startswith("quant"):
            d["frac_hbm_peak"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4)
        elif flops:
            d["TFLOP/s"] = round(flops / ms / 1e9, 1)
            d["frac_f16_peak"] = round(flops / ms / 1e9 / PEAK_F16_TFLOPS, 4)
            d["frac_fp4_peak"] = round(flops / ms / 1e9 / PEAK_FP4_TFLOPS, 4)
        else:
            d["frac_hbm_peak"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4)
        res[name] = d
    return res


def cpu_baseline(args, synthetic, ffn):
    """The oracle, as it stands, on a bounded sample of the same workload: quantize the
    first rows of X and all of W_up, then the binary64 GEMM of those rows against W_up."""
    import numpy as np
    import oracle
    rows = args.cpu_sample_rows
    x = ffn["X"][:rows].float().numpy()
    w = ffn["W_up"].float().numpy()
    t0 = time.perf_counter()
    qa, _ = oracle.quantize(x)
    qb, _ = oracle.quantize(w, block2d=True)
    t1 = time.perf_counter()
    oracle.gemm_f64(qa, qb)
    t2 = time.perf_counter()
    flops = 2.0 * rows * FFN * HIDDEN
    qbytes_ = 2 * (rows + FFN) * HIDDEN + qbytes(rows, HIDDEN) + qbytes(FFN, HIDDEN)
    # the same at one thread, on 1/16 of the rows and W_up (the GEMM scales with both)
    threads = oracle.num_threads()
    r1, n1 = max(rows // 16, 16), FFN // 16
    oracle.set_num_threads(1)
    t3 = time.perf_counter()
    qa1, _ = oracle.quantize(x[:r1])
    qb1, _ = oracle.quantize(w[:n1], block2d=True)
    oracle.gemm_f64(qa1, qb1)
    t4 = time.perf_counter()
    oracle.set_num_threads(threads)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(flops / (t2 - t0) / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle", "cpu_model": model, "nproc": os.cpu_count(),
            "one_thread": {"TFLOP/s": round(2.0 * r1 * n1 * HIDDEN / (t4 - t3) / 1e12, 6),
                           "sample": f"X[:{r1}] and W_up[:{n1}], quantize + binary64 GEMM",
                           "seconds": round(t4 - t3, 2)},
            "sample": f"FFN-up: quantize X[:{rows}] (1x16) and W_up 9216x3072 (16x16), then the "
                      f"binary64 GEMM {rows}x9216x3072; TFLOP/s counts the GEMM flops over the "
                      f"quantize+GEMM time",
            "quantize_GB/s": round(qbytes_ / (t1 - t0) / 1e9, 3),
            "gemm_TFLOP/s": round(flops / (t2 - t1) / 1e12, 6),
            "seconds": round(t2 - t0, 2)}


if __name__ == "__main__":
    main()
