"""Benchmark of the 4-bit MoE layer on one MI355X.

One step = the whole layer on one batch: moe_route -> moe_sort ->
qswitch_gate_up_geglu -> qswitch_down_combine, on the 256-token decoder
canvas (H = 2816, 128 experts, top-8, moe_intermediate 704, int4 group 64).
Inputs are resident in HBM before timing starts.  Three independent weight
sets (1.28 GB) are rotated between steps so the 256 MB Infinity Cache cannot
serve a layer's weights from the previous step.

Prints ONE JSON line (rank 0):
  value      tokens/s of the whole layer: wall clock over K steps, bracketed
             by device synchronisation, the four calls issued from Python
             with its garbage collector paused (no events inside).  The same
             K steps replayed from HIP graphs (one per weight set) are
             reported under "graph".
  roofline   the dominant kernel (qswitch_gate_up_geglu, one kernel per call):
             algorithmic bytes per launch / its mean launch time, from HIP
             events recorded between the calls on the launch stream in a
             second pass of K steps (events between kernels add a few
             microseconds of idle time per call, so they stay out of `value`)
  layer_roofline  the whole layer against HBM: algorithmic bytes per step
             (touched experts' weights, router weight, x in, y out) over the
             wall-clock step time -- the figure the 60 % target is set on
  cpu_baseline  the CPU oracle timed on this host: the canvas layer with the
             BLAS pool as it comes (value, cores) and with one thread, plus one
             full-size run each of the dense qlinear, the prefill and the
             skewed canvas
  qlinear_c1 the dense 4-bit linear at 2520 x 1152 -> 1152 on its own (mean
             launch time from HIP events, TFLOP/s against the bf16 peak)
  decode_unsorted  diagnostic, not the metric: the small-batch arm (route +
             the two unsorted calls) at 1 and 7 tokens on the same weights
  lm_head    diagnostic, not the metric: the tied LM head with its softcap,
             256 rows x 2816 -> 262,144 (fp32 logits), and the self-conditioning
             signal on the same table (softmax to bf16, untransposed product)
  vision_qlinears  diagnostic, not the metric: the vision tower's 4-bit
             linears, 27 blocks at 2520 x 1152
  other_workloads  diagnostic, not the metric: the same layer on the 4096-token
             prefill and on the Zipf-skewed 256-token canvas
  ff_block   diagnostic, not the metric: the decoder's feed-forward block
             around the same MoE layer (pre-norms, dense GeGLU branch, the
             layer, post-norms and residual) on the same tokens

Two helper modes serve the committed profiles (see profiles/):
  --copy-probe        one plain 256 MiB device copy, five times (the known-size
                      kernel that calibrates rocprofv3's FETCH_SIZE/WRITE_SIZE)
  --summarize DIR     turns the rocprofv3 output under DIR (kt*/, <workload>_{kt,
                      fetch,write,sq}/, copy_fetch/, copy_write/) into the
                      summaries under profiles/
roofline.traffic is read from profiles/qswitch_gate_up_canvas_traffic.txt and
is null when the kernel sources no longer match the hash recorded there.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["bit_quantized_moe_diffrouter_amd/csrc/qswitch.hip", "bit_quantized_moe_diffrouter_amd/csrc/common.h",
                  "bit_quantized_moe_diffrouter_amd/csrc/launch.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qswitch_gate_up_canvas_traffic.txt")
GATE_UP_KERNEL = "qmm_kernel<0,"   # rocprofv3 name of the gate_up switch kernel
COPY_BYTES = 256 << 20
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s + % HBM roofline, H=2816 128-expert top-8 int4, 256 tok"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="moe_canvas_256tok_h2816_e128_top8",
                    help="diagnostic override; the reported line is defined on the canvas workload")
    ap.add_argument("--weight-sets", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ff-block", action="store_true", help="skip the feed-forward block diagnostic")
    ap.add_argument("--no-decode", action="store_true", help="skip the small-batch (unsorted arm) diagnostic")
    ap.add_argument("--no-head", action="store_true", help="skip the LM-head diagnostic")
    ap.add_argument("--no-other", action="store_true", help="skip the prefill and skewed-canvas diagnostic")
    ap.add_argument("--no-vision", action="store_true", help="skip the vision-tower linears diagnostic")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    return ap.parse_args()


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per gate_up launch from the committed counter summary, or None
    when the kernel sources changed since the counters were taken."""
    try:
        kv = dict(line.strip().split("=", 1) for line in open(TRAFFIC_FILE)
                  if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def copy_probe():
    import torch
    src = torch.full((COPY_BYTES // 4,), 7, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def _pmc_per_dispatch(d, counter, match):
    """Mean over matching dispatches of one counter (rocprofv3 csv), and the count."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    v = list(vals.values())
    return (sum(v) / len(v) if v else float("nan")), len(v)


def _kt_table(d, title, cmd, notes):
    import csv
    import glob
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    lines = [f"# {title}", "", "Command (from the repository root, TMPDIR=/tmp):", "", "    " + cmd, ""] + notes + [
        "", "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in sorted(csv.DictReader(open(stats[0])), key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    return lines


SIMD_NUM = 1024  # 256 compute units x 4 SIMDs
PROFILE_RUNS = {
    # tag: (workload, bench arguments, title)
    "canvas": ("moe_canvas_256tok_h2816_e128_top8",
               "--steps 20 --warmup 5 --no-cpu-baseline --no-ff-block --no-decode --no-other --no-head --no-vision",
               "canvas workload (256 tokens, H 2816, 128 experts, top-8, I 704) and the dense qlinear at "
               "2520 x 1152 -> 1152"),
    "prefill": ("moe_prefill_4096tok_h2816_e128_top8", "--workload moe_prefill_4096tok_h2816_e128_top8 "
                "--steps 10 --warmup 2 --no-cpu-baseline",
                "prefill workload (4096 tokens, H 2816, 128 experts, top-8, I 704)"),
    "skew": ("moe_canvas_skew_256tok_zipf1.1", "--workload moe_canvas_skew_256tok_zipf1.1 --steps 20 --warmup 5 "
             "--no-cpu-baseline", "Zipf-skewed canvas (256 tokens, per-expert logit offset 0.1 ln p, p ~ rank^-1.1)"),
}
SQ_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
               "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
KERNEL_ROLES = [("route_logits_kernel", "moe_route: logits (partial sums)"),
                ("route_topk_kernel", "moe_route: sum, norm, top-k, softmax"),
                ("sort_hist_kernel", "moe_sort: slice histograms"),
                ("sort_kernel", "moe_sort"),
                ("qmm_kernel<0,", "qswitch_gate_up_geglu"),
                ("qmm_tall_kernel<0,", "qswitch_gate_up_geglu (tall-tile)"),
                ("qmm_ws_kernel<4,", "qlinear_softcap (weight-stationary)"),
                ("qmm_kernel<1,", "qswitch_down_combine: down"),
                ("combine_kernel", "qswitch_down_combine: weighted sum over k"),
                ("qmm_kernel<2,", "qlinear (2520 x 1152 -> 1152)"),
                ("qmm_tall_kernel<2,", "qlinear (2520 x 1152 -> 1152, tall-tile kernel)")]


def _per_dispatch(d, counters):
    """{kernel name: {counter: [per-dispatch values]}} from a rocprofv3 counter csv
    (the rows of one dispatch and counter are summed)."""
    import csv
    import glob
    acc = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] in counters:
                key = (r["Kernel_Name"], r["Dispatch_Id"], r["Counter_Name"])
                acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (k, _, c), v in acc.items():
        out.setdefault(k, {}).setdefault(c, []).append(v)
    return out


def _kt_means(d):
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    return {r["Name"]: (float(r["AverageNs"]) / 1e3, int(r["Calls"])) for r in csv.DictReader(open(f[0]))} if f else {}


def _counter_summary(d, tag, kf, kw):
    """profiles/layer_kernels_<tag>_counters.md from DIR/<tag>_{kt,fetch,write,sq}."""
    wl, args, title = PROFILE_RUNS[tag]
    kt = _kt_means(os.path.join(d, f"{tag}_kt"))
    fe = _per_dispatch(os.path.join(d, f"{tag}_fetch"), {"FETCH_SIZE"})
    wr = _per_dispatch(os.path.join(d, f"{tag}_write"), {"WRITE_SIZE"})
    sq = _per_dispatch(os.path.join(d, f"{tag}_sq"), set(SQ_COUNTERS))
    mean = lambda m, k, c: float(np.mean(m[k][c])) if k in m and c in m[k] else float("nan")
    cmd = "rocprofv3 {o} -d DIR/{t} -o p --output-format csv -- python3 bench.py " + args
    lines = [f"# Per-kernel counters, {title}", "",
             "Commands (from the repository root, TMPDIR=/tmp), one rocprofv3 run each:", "",
             "    " + cmd.format(o="--kernel-trace --stats", t=f"{tag}_kt"),
             "    " + cmd.format(o="--pmc FETCH_SIZE", t=f"{tag}_fetch"),
             "    " + cmd.format(o="--pmc WRITE_SIZE", t=f"{tag}_write"),
             "    " + cmd.format(o="--pmc " + " ".join(SQ_COUNTERS), t=f"{tag}_sq"),
             "    rocprofv3 --pmc FETCH_SIZE -d DIR/copy_fetch -o p --output-format csv -- python3 bench.py --copy-probe",
             "    rocprofv3 --pmc WRITE_SIZE -d DIR/copy_write -o p --output-format csv -- python3 bench.py --copy-probe",
             "    python3 bench.py --summarize DIR", "",
             f"HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) times {kf:.4f} and {kw:.4f}, what the same",
             "counters read for a plain 256 MiB device copy.  Time: the kernel-trace mean of the same workload.",
             "MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs), the rocprofv3 MfmaUtil",
             "expression; bf16 TFLOP/s: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / time (the bias-term fp32 MFMAs",
             "are not counted); VALU and MFMA: instructions issued per dispatch (wave instructions).", "",
             "| kernel | role | dispatches | mean us | HBM read MB | HBM write MB | HBM GB/s | VALU instr | MFMA instr "
             "| bf16 TFLOP/s | MFMA busy |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    names = sorted(set(kt) | set(fe) | set(sq), key=lambda n: -kt.get(n, (0, 0))[0] * kt.get(n, (0, 0))[1])
    for n in names:
        role = next((r for pat, r in KERNEL_ROLES if pat in n), None)
        if role is None:
            continue
        us, calls = kt.get(n, (float("nan"), 0))
        rd = mean(fe, n, "FETCH_SIZE") * 1024 * kf
        wb = mean(wr, n, "WRITE_SIZE") * 1024 * kw
        gbs = (rd + wb) / (us * 1e-6) / 1e9
        tf = mean(sq, n, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / (us * 1e-6) / 1e12
        busy = 100.0 * mean(sq, n, "SQ_VALU_MFMA_BUSY_CYCLES") / (mean(sq, n, "GRBM_GUI_ACTIVE") * SIMD_NUM)
        short = n.replace("void ", "").replace("qmoe::", "").split("(")[0]
        lines.append(f"| `{short}` | {role} | {calls} | {us:.2f} | {rd / 1e6:.2f} | {wb / 1e6:.2f} | {gbs:.0f} | "
                     f"{mean(sq, n, 'SQ_INSTS_VALU'):.3g} | {mean(sq, n, 'SQ_INSTS_MFMA'):.3g} | {tf:.1f} | {busy:.1f}% |")
    out = os.path.join(ROOT, "profiles", f"layer_kernels_{tag}_counters.md")
    open(out, "w").write("\n".join(lines) + "\n")
    return lines


def summarize(d):
    import glob
    kt = "rocprofv3 --kernel-trace --stats -d DIR/{d} -o kt --output-format csv -- python3 bench.py {a}"
    lines = _kt_table(os.path.join(d, "kt"),
                      "Kernel durations, canvas workload (256 tokens, H 2816, 128 experts, top-8, I 704)",
                      kt.format(d="kt", a="--steps 60 --warmup 10 --no-cpu-baseline --no-ff-block --no-decode --no-other"),
                      ["rocprofv3 kernel-trace statistics; every dispatch of the run (warm-up, the timed",
                       "pass and the event pass).  qmm_kernel<0,...> is qswitch_gate_up_geglu,",
                       "qmm_kernel<1,...> the down switch linear of qswitch_down_combine."])
    out_kt = os.path.join(ROOT, "profiles", "switch_kernels_canvas_kernel_trace.md")
    open(out_kt, "w").write("\n".join(lines) + "\n")
    if glob.glob(os.path.join(d, "kt_ff", "**", "*kernel_stats.csv"), recursive=True):
        ff = _kt_table(os.path.join(d, "kt_ff"),
                       "Kernel durations, feed-forward block around the canvas MoE layer (256 tokens, "
                       "H 2816, dense GeGLU width 2112)",
                       kt.format(d="kt_ff", a="--steps 60 --warmup 10 --no-cpu-baseline --no-decode --no-other"),
                       ["The same run as the canvas line plus the feed-forward block diagnostic, so the",
                        "MoE kernels appear twice as often.  qmm_kernel<3,...> is qlinear_geglu (dense",
                        "gate|up + GeGLU), qmm_kernel<2,...> qlinear (the dense down projection);",
                        "ff_prenorm_kernel and ff_combine_kernel are the five RMSNorms, the residual",
                        "and the layer scalar."])
        open(os.path.join(ROOT, "profiles", "ff_block_canvas_kernel_trace.md"), "w").write("\n".join(ff) + "\n")
    if glob.glob(os.path.join(d, "kt_dec", "**", "*kernel_stats.csv"), recursive=True):
        dec = _kt_table(os.path.join(d, "kt_dec"),
                        "Kernel durations, small-batch arm at 1 and 7 tokens (canvas weights: H 2816, "
                        "128 experts, top-8, I 704)",
                        kt.format(d="kt_dec", a="--steps 60 --warmup 10 --no-cpu-baseline --no-ff-block --no-other"),
                        ["The same run as the canvas line plus the decode diagnostic (moe_route and the",
                         "two unsorted calls, 60 + 10 + 48 layers at each of 1 and 7 tokens), so the",
                         "router kernels also count the decode layers.  qswitch_unsorted_kernel<0,...> is",
                         "the gate_up pass and unsorted_geglu_kernel its part sum + GeGLU;",
                         "qswitch_unsorted_kernel<1,...> the down pass and unsorted_combine_kernel its",
                         "part sum + weighted sum over k.  Both token counts are pooled in one row per",
                         "kernel; the bench line's decode_unsorted object has them apart."])
        open(os.path.join(ROOT, "profiles", "unsorted_decode_kernel_trace.md"), "w").write("\n".join(dec) + "\n")

    for name, wl, title in (
            ("kt_prefill", "moe_prefill_4096tok_h2816_e128_top8",
             "Kernel durations, prefill workload (4096 tokens, H 2816, 128 experts, top-8, I 704)"),
            ("kt_skew", "moe_canvas_skew_256tok_zipf1.1",
             "Kernel durations, Zipf-skewed canvas (256 tokens, per-expert logit offset 0.1 ln p, p ~ rank^-1.1)")):
        if glob.glob(os.path.join(d, name, "**", "*kernel_stats.csv"), recursive=True):
            steps = "--steps 20 --warmup 3" if "prefill" in wl else "--steps 60 --warmup 10"
            tab = _kt_table(os.path.join(d, name), title,
                            kt.format(d=name, a=f"--workload {wl} {steps} --no-cpu-baseline"),
                            ["The four layer calls only (the diagnostics run on the canvas workload alone).",
                             "qmm_kernel<0,...> is qswitch_gate_up_geglu, qmm_kernel<1,...> the down switch",
                             "linear of qswitch_down_combine."])
            out_name = "switch_kernels_" + ("prefill" if "prefill" in wl else "skew") + "_kernel_trace.md"
            open(os.path.join(ROOT, "profiles", out_name), "w").write("\n".join(tab) + "\n")

    fetch, nf = _pmc_per_dispatch(os.path.join(d, "canvas_fetch"), "FETCH_SIZE", lambda n: "qmm_kernel<0" in n)
    write, nw = _pmc_per_dispatch(os.path.join(d, "canvas_write"), "WRITE_SIZE", lambda n: "qmm_kernel<0" in n)
    # the copy: the dispatches of the largest kernel in the probe run
    cf, ncf = _pmc_per_dispatch(os.path.join(d, "copy_fetch"), "FETCH_SIZE", lambda n: "opy" in n)
    cw, ncw = _pmc_per_dispatch(os.path.join(d, "copy_write"), "WRITE_SIZE", lambda n: "opy" in n)
    kf = COPY_BYTES / (cf * 1024.0)   # true bytes per reported byte, reads
    kw = COPY_BYTES / (cw * 1024.0)   # and writes
    traffic = fetch * 1024.0 * kf + write * 1024.0 * kw
    cmd = ("rocprofv3 --pmc {c} -d DIR/{d} -o p --output-format csv -- python3 bench.py {a}")
    txt = ["# HBM traffic of qswitch_gate_up_geglu (qmm_kernel<0,...>), canvas workload",
           "# Commands (from the repository root, TMPDIR=/tmp), one counter per run:",
           "#   " + cmd.format(c="FETCH_SIZE", d="canvas_fetch", a=PROFILE_RUNS["canvas"][1]),
           "#   " + cmd.format(c="WRITE_SIZE", d="canvas_write", a=PROFILE_RUNS["canvas"][1]),
           "#   " + cmd.format(c="FETCH_SIZE", d="copy_fetch", a="--copy-probe"),
           "#   " + cmd.format(c="WRITE_SIZE", d="copy_write", a="--copy-probe"),
           "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the same",
           "# counter reads for a plain device copy of copy_bytes (read and written once).",
           f"source_sha256={kernel_source_hash()}",
           f"fetch_kib_per_dispatch={fetch:.1f}", f"fetch_dispatches={nf}",
           f"write_kib_per_dispatch={write:.1f}", f"write_dispatches={nw}",
           f"copy_bytes={COPY_BYTES}", f"copy_fetch_kib={cf:.1f}", f"copy_write_kib={cw:.1f}",
           f"fetch_scale={kf:.4f}", f"write_scale={kw:.4f}",
           f"traffic_bytes_per_launch={traffic:.0f}"]
    open(TRAFFIC_FILE, "w").write("\n".join(txt) + "\n")
    print("\n".join(lines[-12:]))
    for tag in PROFILE_RUNS:
        if os.path.isdir(os.path.join(d, f"{tag}_sq")):
            print("\n".join(_counter_summary(d, tag, kf, kw)[-10:]))
    print("\n".join(txt[-11:]))


def expert_bytes(cfg):
    """Algorithmic bytes of one touched expert: packed codes + bf16 scales + biases."""
    gu = 2 * cfg.I * (cfg.H // 2 + 2 * 2 * (cfg.H // 64))
    dn = cfg.H * (cfg.I // 2 + 2 * 2 * (cfg.I // 64))
    return gu, dn


def router_bytes(cfg):
    return cfg.E * (cfg.H // 2 + 4 * (cfg.H // 64)) + 2 * cfg.H + 2 * cfg.E


def _timed_runs(fn, seconds, max_runs=5):
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= seconds or len(times) >= max_runs:
            return float(np.median(times)), len(times)


def cpu_baseline(cfg, inp, seconds, synth):
    """The oracle as it stands, on this host's cores: the canvas layer with the
    BLAS thread pool as it comes (the reported value) and with one thread, and
    one run each of the dense qlinear (C1 geometry), the 4096-token prefill and
    the skewed canvas, all full size (about 20-30 s of CPU work in all)."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or len(os.sched_getaffinity(0))
    wt = inp.weights
    layer = lambda c, i: (lambda: O.moe_layer(i.x, i.weights, c.k, c.I, c.eps, grouped=True))
    t, n = _timed_runs(layer(cfg, inp), seconds)
    with threadpool_limits(1):
        t1, n1 = _timed_runs(layer(cfg, inp), 0.0, 1)
    others = {}
    c1 = synth.make_qlinear_inputs(synth.QLINEAR_VISION)
    tq, nq = _timed_runs(lambda: O.qlinear(c1.x, c1.W.w, c1.W.scales, c1.W.biases), 1.0)
    others[synth.QLINEAR_VISION.name] = {"value": c1.cfg.M / tq, "unit": "rows/s", "seconds": tq, "runs": nq,
                                         "what": "fp64 dequantize + matmul, full size"}
    for oc in (synth.PREFILL, synth.SKEW):
        w = wt if oc.zipf_tau is None else synth.MoEWeights(
            wt.norm_scale, wt.router, wt.per_expert_scale, wt.gate_up, wt.down,
            synth.zipf_logit_bias(oc.E, oc.zipf_tau, oc.zipf_perm_seed))
        oi = synth.make_moe_inputs(oc, w)
        to, no = _timed_runs(layer(oc, oi), 0.0, 1)
        others[oc.name] = {"value": oc.T / to, "unit": "tokens/s", "seconds": to, "runs": no,
                           "what": "full layer (route + grouped fp32 experts)"}
    return {"value": cfg.T / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full {cfg.T}-token layer (route + grouped fp32 experts), {n} run(s), "
                      f"median {t:.2f} s, BLAS pool of {threads} threads; host has {os.cpu_count()} logical CPUs",
            "single_thread": {"value": cfg.T / t1, "unit": "tokens/s", "cores": 1, "seconds": t1, "runs": n1},
            "other_configs": others}


LAYER_CALLS = ["moe_route", "moe_sort", "qswitch_gate_up_geglu", "qswitch_down_combine"]


def make_layer_step(q, torch, cfg, x):
    """The layer's four calls on preallocated outputs and workspaces (the
    library allocates nothing); step(p, ev) records ev[0..4] around the calls."""
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    dev = x.device
    buf = dict(idx=torch.empty((T, k), dtype=torch.int32, device=dev),
               wts=torch.empty((T, k), dtype=torch.float32, device=dev),
               off=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sa=torch.empty(T * k, dtype=torch.int32, device=dev),
               mid=torch.empty(q.qswitch_mid_bytes(T, k, I, E), dtype=torch.uint8, device=dev),
               y=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
               ws_r=torch.empty(max(1, q.moe_route_workspace(T, H, E)), dtype=torch.uint8, device=dev),
               ws_s=torch.empty(max(1, q.moe_sort_workspace(T, k, E)), dtype=torch.uint8, device=dev),
               ws_d=torch.empty(max(1, q.qswitch_down_combine_workspace(T, k, H, 1)), dtype=torch.uint8, device=dev))
    idx, wts, off, sa, mid, y = (buf[n] for n in ("idx", "wts", "off", "sa", "mid", "y"))

    def step(p, ev=None):
        if ev is not None:
            ev[0].record()
        q.moe_route(x, p.norm_scale, cfg.eps, p.router, p.per_expert_scale, k, p.logit_bias,
                    indices=idx, weights=wts, workspace=buf["ws_r"])
        if ev is not None:
            ev[1].record()
        q.moe_sort(idx, E, off, sa, workspace=buf["ws_s"])
        if ev is not None:
            ev[2].record()
        q.qswitch_gate_up_geglu(x, p.gate_up, I, k, off, sa, mid=mid)
        if ev is not None:
            ev[3].record()
        q.qswitch_down_combine(mid, T, k, p.down, wts, off, sa, y=y, workspace=buf["ws_d"], deterministic=1)
        if ev is not None:
            ev[4].record()

    return step, buf


class _no_gc:
    """Python's cyclic garbage collector off inside a timed loop: a full
    collection over the interpreter's (torch-sized) heap stalls the host for
    milliseconds, long enough to drain the launch queue and idle the GPU."""

    def __enter__(self):
        import gc
        gc.collect()
        gc.freeze()
        gc.disable()

    def __exit__(self, *exc):
        import gc
        gc.enable()
        gc.unfreeze()


def time_layer_graph(torch, step, sets, K, warmup):
    """The same K steps, each layer replayed from a HIP graph (one graph per
    weight set, captured once): no host work between the kernels.  Returns
    wall seconds."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for p in sets:
            step(p)
    torch.cuda.current_stream().wait_stream(side)
    graphs = []
    for p in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(p)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    with _no_gc():
        t0 = time.perf_counter()
        for i in range(K):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    del graphs
    return wall


def time_layer(torch, step, sets, K, warmup, off):
    """Wall time of K steps (weight sets rotated, no events inside), then the
    per-call mean times (us) from a second pass of K steps with HIP events
    between the calls on the launch stream.  Returns (wall_s, mean_us,
    experts touched per set)."""
    touched = []
    for p in sets:
        step(p)
        torch.cuda.synchronize()
        touched.append(int((torch.diff(off.cpu()) > 0).sum()))
    for i in range(warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    with _no_gc():
        t0 = time.perf_counter()
        for i in range(K):
            step(sets[i % len(sets)])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    per = {n: [] for n in LAYER_CALLS}
    for ev in evs:
        for j, n in enumerate(LAYER_CALLS):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
    return wall, {n: float(np.mean(v)) for n, v in per.items()}, touched


def other_workloads_timing(q, torch, synth, sets, K, warmup, t):
    """Diagnostic: the same four calls on the 4096-token prefill and on the
    Zipf-skewed 256-token canvas, with the canvas's weight sets (same shapes;
    the skewed canvas adds its per-expert logit offset to each set).  Prefill
    is priced against the bf16 MFMA peak (its contraction, not its bytes,
    bounds it); the skewed canvas against HBM like the canvas."""
    import dataclasses
    res = {}
    for cfg in (synth.PREFILL, synth.SKEW):
        T, k, H, I = cfg.T, cfg.k, cfg.H, cfg.I
        A = T * k
        x = t(synth.make_activations(T, H, cfg.seed_x))
        run_sets = sets
        if cfg.zipf_tau:
            bias = t(synth.zipf_logit_bias(cfg.E, cfg.zipf_tau, cfg.zipf_perm_seed))
            run_sets = [dataclasses.replace(p, logit_bias=bias) for p in sets]
        step, buf = make_layer_step(q, torch, cfg, x)
        n = max(10, K // 10) if T > 1024 else K
        wall, mean_us, touched = time_layer(torch, step, run_sets, n, max(3, warmup // 10), buf["off"])
        gu_b, dn_b = expert_bytes(cfg)
        n_touch = float(np.mean(touched))
        gu_us = mean_us["qswitch_gate_up_geglu"]
        gu_flops = 2.0 * A * 2 * I * H
        gu_bytes = n_touch * gu_b + T * H * 2 + A * I * 2
        layer_flops = 2.0 * A * (2 * I * H + H * I) + 2.0 * T * cfg.E * H
        layer_bytes = n_touch * (gu_b + dn_b) + router_bytes(cfg) + 2 * T * H * 2
        ms = wall / n * 1e3
        res[cfg.name] = {
            "steps": n, "tokens_per_s": T * n / wall, "ms_per_layer": ms, "experts_touched": n_touch,
            "call_mean_us": mean_us,
            "gate_up": {"TFLOPs": gu_flops / (gu_us * 1e-6) / 1e12,
                        "mfma_frac": gu_flops / (gu_us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                        "GBs": gu_bytes / (gu_us * 1e-6) / 1e9,
                        "hbm_frac": gu_bytes / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "layer": {"mfma_frac": layer_flops / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                      "hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        }
        del step, buf, x
    return res



def ff_block_timing(q, torch, synth, ffc, h, sets, K, warmup, t, buf):
    """Diagnostic: the decoder's whole feed-forward block around the MoE
    (ff_prenorm, qlinear_geglu, qlinear, the four MoE calls, ff_combine) on the
    same tokens, K blocks with HIP events between the calls.  The dense
    branch's weights are cloned to 32 distinct buffers (about 290 MB) and
    rotated with the MoE weight sets, so neither is served from the Infinity
    Cache of the previous block."""
    import dataclasses
    cfg, Id = ffc.moe, ffc.I_dense
    T, H, k, E, I = cfg.T, cfg.H, cfg.k, cfg.E, cfg.I
    fw = synth.make_ff_weights(ffc)
    qw = lambda m: q.QuantWeight(t(m.w), t(m.scales), t(m.biases))
    base = q.FFParams.from_rows(t(fw.pre_ff), t(fw.pre_ff2), t(fw.post_ff1), t(fw.post_ff2), t(fw.post_ff),
                                qw(fw.gate), qw(fw.up), qw(fw.down), fw.layer_scalar)
    reps = [dataclasses.replace(base, gate_up=dataclasses.replace(base.gate_up, buf=base.gate_up.buf.clone()),
                                down=dataclasses.replace(base.down, buf=base.down.buf.clone()))
            for _ in range(32)]
    dev = h.device
    xa = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    xb = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    gmid = torch.empty((T, Id), dtype=torch.bfloat16, device=dev)
    dense = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    b = buf

    def block(i, ev=None):
        p, f = sets[i % len(sets)], reps[i % len(reps)]
        mark = (lambda j: ev[j].record()) if ev is not None else (lambda j: None)
        mark(0)
        q.ff_prenorm(h, f.pre_ff, f.pre_ff2, cfg.eps, xa, xb)
        mark(1)
        q.qlinear_geglu(xa, f.gate_up, gmid)
        mark(2)
        q.qlinear(gmid, f.down, dense)
        mark(3)
        q.moe_route(h, p.norm_scale, cfg.eps, p.router, p.per_expert_scale, k, p.logit_bias,
                    indices=b["idx"], weights=b["wts"], workspace=b["ws_r"])
        q.moe_sort(b["idx"], E, b["off"], b["sa"], workspace=b["ws_s"])
        q.qswitch_gate_up_geglu(xb, p.gate_up, I, k, b["off"], b["sa"], mid=b["mid"])
        q.qswitch_down_combine(b["mid"], T, k, p.down, b["wts"], b["off"], b["sa"], y=b["y"],
                               workspace=b["ws_d"], deterministic=1)
        mark(4)
        q.ff_combine(h, dense, b["y"], f.post_ff1, f.post_ff2, f.post_ff, cfg.eps, f.layer_scalar, out)
        mark(5)

    for i in range(warmup):
        block(i)
    torch.cuda.synchronize()
    with _no_gc():
        t0 = time.perf_counter()
        for i in range(K):
            block(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for i in range(K):
        block(i, evs[i])
    torch.cuda.synchronize()
    names = ["ff_prenorm", "qlinear_geglu", "qlinear_down", "moe_layer", "ff_combine"]
    mean_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) * 1e3 for ev in evs])) for j, n in enumerate(names)}
    wgu = 2 * Id * (H // 2 + 4 * (H // 64))
    wdn = H * (Id // 2 + 4 * (Id // 64))
    geglu_alg = wgu + T * H * 2 + T * Id * 2
    down_alg = wdn + T * Id * 2 + T * H * 2
    return {"workload": ffc.name, "dense_intermediate": Id, "blocks": K,
            "us_per_block": wall / K * 1e6, "tokens_per_s": T * K / wall, "call_mean_us": mean_us,
            "qlinear_geglu_GBs": geglu_alg / (mean_us["qlinear_geglu"] * 1e-6) / 1e9,
            "qlinear_down_GBs": down_alg / (mean_us["qlinear_down"] * 1e-6) / 1e9,
            "dense_weight_bytes": wgu + wdn}


def decode_timing(q, torch, synth, sets, K, warmup, tokens=(1, 7)):
    """Diagnostic: the small-batch arm (moe_route + the two unsorted calls) at
    decode batch sizes on the canvas weights: K layers launched one by one
    (wall clock, then with HIP events between the calls), and 48 layers
    captured in one HIP graph and replayed.  Sixteen token sets and the three
    weight sets rotate, so most experts' weights come from HBM."""
    cfg = synth.CANVAS
    k, E, H, I = cfg.k, cfg.E, cfg.H, cfg.I
    dev = torch.device("cuda:0")
    gu_b, dn_b = expert_bytes(cfg)
    out = {}
    for T in tokens:
        xs = [torch.from_numpy(synth.make_activations(T, H, 1000 + j)).to(dev) for j in range(16)]
        ws = q.unsorted_workspace(T, k, H, I)
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, k), dtype=torch.float32, device=dev)
        ws_r = torch.empty(max(1, q.moe_route_workspace(T, H, E)), dtype=torch.uint8, device=dev)
        mid = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        touched = []

        def layer(i, ev=None):
            x, p = xs[i % 16], sets[i % len(sets)]
            mark = (lambda j: ev[j].record()) if ev is not None else (lambda j: None)
            mark(0)
            q.moe_route(x, p.norm_scale, cfg.eps, p.router, p.per_expert_scale, k, p.logit_bias,
                        indices=idx, weights=wts, workspace=ws_r)
            mark(1)
            q.qswitch_gate_up_geglu_unsorted(x, p.gate_up, I, idx, ws, mid)
            mark(2)
            q.qswitch_down_combine_unsorted(mid, T, k, p.down, idx, wts, ws, y)
            mark(3)

        for i in range(48):
            layer(i)
            if i < 16 * len(sets):
                torch.cuda.synchronize()
                touched.append(len(set(idx.cpu().numpy().reshape(-1).tolist())))
        for i in range(warmup):
            layer(i)
        torch.cuda.synchronize()
        with _no_gc():
            t0 = time.perf_counter()
            for i in range(K):
                layer(i)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for i in range(K):
            layer(i, evs[i])
        torch.cuda.synchronize()
        names = ["moe_route", "qswitch_gate_up_geglu_unsorted", "qswitch_down_combine_unsorted"]
        mean_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) * 1e3 for ev in evs])) for j, n in enumerate(names)}
        # the same layers captured in one HIP graph (48 layers, all token and
        # weight sets), replayed: the host's per-call launch cost leaves the loop
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer(0)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(48):
                layer(i)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, K // 48)
        with _no_gc():
            t0 = time.perf_counter()
            for _ in range(reps):
                graph.replay()
            torch.cuda.synchronize()
            us_graph = (time.perf_counter() - t0) / (reps * 48) * 1e6
        n_touch = float(np.mean(touched))
        alg = n_touch * (gu_b + dn_b) + router_bytes(cfg) + 2 * T * H * 2
        us = wall / K * 1e6
        out[f"T{T}"] = {"tokens": T, "us_per_layer_graph": us_graph, "tokens_per_s_graph": T / (us_graph * 1e-6),
                        "achieved_GBs_graph": alg / (us_graph * 1e-6) / 1e9,
                        "us_per_layer_eager": us, "experts_touched": n_touch, "alg_bytes": alg,
                        "call_mean_us_eager": mean_us}
    return out


def lm_head_timing(q, torch, synth, K, warmup, vocab=262144, rows=256, hidden=2816, cap=30.0):
    """Diagnostic: the tied LM head with its softcap (qlinear_softcap) on the
    canvas rows, vocabulary 262,144 (its 4-bit weight, 415 MB, exceeds the
    Infinity Cache, so every call streams it from HBM)."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(31)
    W = synth.random_qtensor(rng, (vocab,), hidden)
    Wq = q.QuantWeight(torch.from_numpy(W.w).to(dev), torch.from_numpy(W.scales).to(dev),
                       torch.from_numpy(W.biases).to(dev))
    Wt = Wq.tiled(0)
    WtT = Wq.tiled_t()  # the same table for the untransposed self-conditioning product
    del W, Wq
    x = torch.from_numpy(synth.make_activations(rows, hidden, 32)).to(dev)
    y = torch.empty((rows, vocab), dtype=torch.float32, device=dev)
    n = max(4, K // 10)
    for _ in range(max(2, warmup // 10)):
        q.qlinear_softcap(x, Wt, cap, y)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        q.qlinear_softcap(x, Wt, cap, y)
        b.record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs]))
    flops = 2.0 * rows * vocab * hidden
    wbytes = vocab * (hidden // 2 + 4 * (hidden // 64))
    hbm = wbytes + rows * hidden * 2 + rows * vocab * 4
    head = {"rows": rows, "vocab": vocab, "hidden": hidden, "calls": n, "mean_launch_us": us,
            "tflops": flops / (us * 1e-6) / 1e12, "mfma_frac": flops / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "hbm_bytes": hbm, "achieved_GBs": hbm / (us * 1e-6) / 1e9, "hbm_frac": hbm / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    # the self-conditioning signal on the same table: softmax of fp32 logits
    # [rows, vocab] to bf16, then probabilities times the untransposed table
    z = y  # the head's softcapped logits serve as self-conditioning logits
    probs = torch.empty((rows, vocab), dtype=torch.bfloat16, device=dev)
    se = torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(int(q.lib().embed_matmul_t_workspace(rows, vocab, hidden)), dtype=torch.uint8, device=dev)
    scale = float(np.sqrt(hidden))
    for _ in range(2):
        q.softmax_rows_bf16(z, probs)
        q.embed_matmul_t(probs, WtT, scale, se, ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for e in ev:
        e[0].record()
        q.softmax_rows_bf16(z, probs)
        e[1].record()
        q.embed_matmul_t(probs, WtT, scale, se, ws)
        e[2].record()
    torch.cuda.synchronize()
    us_sm = float(np.mean([e[0].elapsed_time(e[1]) * 1e3 for e in ev]))
    us_mm = float(np.mean([e[1].elapsed_time(e[2]) * 1e3 for e in ev]))
    sm_bytes = rows * vocab * (4 * 2 + 2)  # two passes over the fp32 logits, bf16 out
    head["self_conditioning"] = {
        "softmax_us": us_sm, "softmax_GBs": sm_bytes / (us_sm * 1e-6) / 1e9,
        "product_us": us_mm, "product_tflops": flops / (us_mm * 1e-6) / 1e12,
        "product_mfma_frac": flops / (us_mm * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "product_hbm_GBs": (wbytes + rows * vocab * 2) / (us_mm * 1e-6) / 1e9}
    return head


def qlinear_c1_timing(q, torch, synth, K, warmup):
    """The dense 4-bit linear at the vision tower's geometry on its own: x
    [2520, 1152] bf16 against one 1152 -> 1152 weight, bf16 out, K launches
    each bracketed by HIP events on the launch stream."""
    cfg = synth.QLINEAR_VISION
    dev = torch.device("cuda:0")
    inp = synth.make_qlinear_inputs(cfg)
    x = torch.from_numpy(inp.x).to(dev)
    W = q.QuantWeight(*(torch.from_numpy(a).to(dev) for a in (inp.W.w, inp.W.scales, inp.W.biases))).tiled(0)
    y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        q.qlinear(x, W, y)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record()
        q.qlinear(x, W, y)
        b.record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in ev]))
    flops = 2.0 * cfg.M * cfg.N * cfg.K
    hbm = cfg.M * cfg.K * 2 + cfg.N * (cfg.K // 2 + 4 * (cfg.K // 64)) + cfg.M * cfg.N * 2
    return {"workload": cfg.name, "launches": K, "mean_launch_us": us, "tflops": flops / (us * 1e-6) / 1e12,
            "mfma_frac": flops / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "hbm_GBs": hbm / (us * 1e-6) / 1e9, "alg_bytes": hbm, "flops": flops}


def vision_timing(q, torch, synth, passes=3, blocks=27, rows=2520, hidden=1152, mlp=4304):
    """Diagnostic: the vision tower's 4-bit linears at their geometry, 27
    blocks x (q, k, v, o: 1152 -> 1152; gate|up fused with GeGLU: 1152 ->
    4304) on 2520 patch rows, each block with its own weights (231 MB in all).
    Attention and the bf16 down projection are not part of this library."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(51)
    qw = lambda n: q.QuantWeight(*(torch.from_numpy(a).to(dev) for a in
                                   (lambda t: (t.w, t.scales, t.biases))(synth.random_qtensor(rng, (n,), hidden))))
    weights = []
    for _ in range(blocks):
        proj = [qw(hidden).tiled(0) for _ in range(4)]
        g, u = qw(mlp), qw(mlp)
        gu = q.QuantWeight(torch.cat([g.w, u.w]), torch.cat([g.scales, u.scales]),
                           torch.cat([g.biases, u.biases])).tiled(mlp)
        weights.append((proj, gu))
    x = torch.from_numpy(synth.make_activations(rows, hidden, 52)).to(dev)
    outs = [torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    mid = torch.empty((rows, mlp), dtype=torch.bfloat16, device=dev)

    def tower():
        for proj, gu in weights:
            for W, y in zip(proj, outs):
                q.qlinear(x, W, y)
            q.qlinear_geglu(x, gu, mid)

    tower()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(passes + 1)]
    ev[0].record()
    for i in range(passes):
        tower()
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = float(np.mean([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(passes)]))
    flops = 2.0 * rows * hidden * (4 * hidden + 2 * mlp) * blocks
    wbytes = (4 * hidden + 2 * mlp) * (hidden // 2 + 4 * (hidden // 64)) * blocks
    return {"blocks": blocks, "rows": rows, "hidden": hidden, "mlp": mlp, "us_per_tower": us,
            "tflops": flops / (us * 1e-6) / 1e12, "mfma_frac": flops / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "weight_bytes": wbytes}


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the layer runs on one GPU only (how it would split across GPUs is "
              "described, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return

    import torch

    import bit_quantized_moe_diffrouter_amd as q
    import synth

    cfg = synth.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- inputs resident in HBM: x and three independent weight sets
    seeds = [cfg.seed_w + 10 * i for i in range(args.weight_sets)]
    sets, host_first = [], None
    for s in seeds:
        w = synth.make_moe_weights(cfg, seed=s)
        if host_first is None:
            host_first = w
        sets.append(q.MoEParams.from_rows(
            t(w.norm_scale), q.QuantWeight(t(w.router.w), t(w.router.scales), t(w.router.biases)),
            t(w.per_expert_scale), q.QuantWeight(t(w.gate_up.w), t(w.gate_up.scales), t(w.gate_up.biases)),
            q.QuantWeight(t(w.down.w), t(w.down.scales), t(w.down.biases)),
            None if w.logit_bias is None else t(w.logit_bias)))
    x_host = synth.make_activations(cfg.T, cfg.H, cfg.seed_x)
    x = t(x_host)
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    A = T * k
    step, buf = make_layer_step(q, torch, cfg, x)
    wall, mean_us, touched = time_layer(torch, step, sets, args.steps, args.warmup, buf["off"])
    wall_graph = time_layer_graph(torch, step, sets, args.steps, args.warmup)
    K = args.steps

    gu_b, dn_b = expert_bytes(cfg)
    n_touch = float(np.mean(touched))
    x_bytes, y_bytes = T * H * 2, T * H * 2
    gate_up_alg = n_touch * gu_b + x_bytes + A * I * 2  # weights + rows in + mid out
    layer_alg = n_touch * (gu_b + dn_b) + router_bytes(cfg) + x_bytes + y_bytes
    flops = 2.0 * A * (2 * I * H + H * I) + 2.0 * T * E * H
    ms = wall / K * 1e3
    gbs_gu = gate_up_alg / (mean_us["qswitch_gate_up_geglu"] * 1e-6) / 1e9
    layer_gbs = layer_alg / (ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": T * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "experts": E, "top_k": k,
                   "moe_intermediate": I, "group": 64, "bits": 4, "weight_sets": len(sets),
                   "experts_touched": n_touch, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "qswitch_gate_up_geglu", "achieved": gbs_gu,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs_gu / HBM_PEAK_GBS,
                     "traffic": read_traffic(), "alg_bytes_per_launch": gate_up_alg,
                     "mean_launch_us": mean_us["qswitch_gate_up_geglu"]},
        "layer_roofline": {"bound": "hbm", "achieved": layer_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": layer_gbs / HBM_PEAK_GBS, "alg_bytes_per_step": layer_alg,
                           "what": "the whole layer: algorithmic bytes per step / wall-clock step time"},
        "layer": {"alg_bytes": layer_alg, "achieved_GBs": layer_gbs, "hbm_frac": layer_gbs / HBM_PEAK_GBS,
                  "flops": flops, "mfma_frac": flops / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                  "call_mean_us": mean_us,
                  "call_sum_us": float(sum(mean_us.values()))},
        "cpu_baseline": None,
        "graph": {"tokens_per_s": T * K / wall_graph, "ms_per_step": wall_graph / K * 1e3,
                  "what": "the same K steps, each layer replayed from a HIP graph (one per weight set)"},
    }
    if cfg.name == synth.CANVAS.name:
        out["qlinear_c1"] = qlinear_c1_timing(q, torch, synth, K, args.warmup)
    if cfg.name == synth.CANVAS.name and not args.no_decode:
        out["decode_unsorted"] = decode_timing(q, torch, synth, sets, K, args.warmup)
    if cfg.name == synth.CANVAS.name and not args.no_other:
        out["other_workloads"] = other_workloads_timing(q, torch, synth, sets, K, args.warmup, t)
    if cfg.name == synth.CANVAS.name and not args.no_head:
        out["lm_head"] = lm_head_timing(q, torch, synth, K, args.warmup)
    if cfg.name == synth.CANVAS.name and not args.no_vision:
        out["vision_qlinears"] = vision_timing(q, torch, synth)
    ffc = next((f for f in synth.FF_CONFIGS.values() if f.moe.name == cfg.name), None)
    if ffc is not None and not args.no_ff_block:
        out["ff_block"] = ff_block_timing(q, torch, synth, ffc, x, sets, K, args.warmup, t,
                                          buf)
    if not args.no_cpu_baseline:
        inp = synth.MoEInputs(cfg, x_host, host_first)
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds, synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
