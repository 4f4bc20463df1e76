"""Benchmark of the FP4 quantization path on one MI355X.

Default workload (one step = the whole path over one batch): a random-init
Qwen2.5-14B-shaped stack, 48 layers x {q 5120x5120, k and v 1024x5120, o
5120x5120, gate and up 13824x5120, down 5120x13824}, bf16 N(0, 0.02) seeded
per tensor (13.2e9 parameters, 26.4 GB resident in HBM before timing).  Every
tensor is quantized twice per step: MXFP4 (block 32, E8M0) and NVFP4 (block
16, UE4M3 under the dynamic FP32 per-tensor scale, whose tensor maximum the
MXFP4 pass takes on the way), each with packed codes, scale bytes, the relative
per-block MSE and the three-term error split.  Every five consecutive tensors
of the stack go in one fp4_quantize_mx_nv_batch call (one launch per format;
--batch N for N per call, --no-batch for one fp4_quantize_mx_nv call per
tensor, --separate for the two single-format calls, NVFP4 with its own amax
pass).  The step spreads its calls over two HIP streams (one workspace each;
--streams 1 runs them back to back): while one call's VALU-heavy NVFP4 pass
runs, the other stream's MXFP4 pass overlaps it.

Prints one JSON line:
  value         GB/s of input quantized+packed+MSE'd over the whole step (every
                kernel of every call; K steps between HIP events), with the
                per-step median and minimum beside the mean.
  roofline      the step's own quantize launches: one step's calls replayed back
                to back on one stream, each kernel launch bracketed by HIP
                events on that stream (fp4q_profile_events); achieved = their
                algorithmic bytes (read 2 B/element, codes 0.5, scale bytes 1/b,
                per-block MSE 4/b) over their summed durations, against 8 TB/s.
                The per-tensor amax pass (read 2 B/element) is reported beside it
                as s0_amax_pass.  `traffic` is the counter-measured HBM bytes per
                launch from profiles/ when taken on the current kernel source.
  copy_ceiling  a plain device copy of the largest tensor (read + write), the
                bandwidth this access pattern reaches on the box.
  cpu_baseline  the oracle on a bounded sample of the same workload, on all host
                threads (row slices) and on one, with the CPU model.

Workloads (--workload):
  qwen14model  the default above (--layers L runs only the first L layers)
  qwen7        six bf16 Qwen2.5-7B MLP tensors, 18944x3584 and 3584x18944 with
               N(0, sigma), sigma in {0.01, 0.02, 0.04}: NVFP4 under the dynamic
               per-tensor scale, per-block MSE and the three-term split
  qwen05       fp32 4864 x 896 (Qwen2.5-0.5B up-projection), MXFP4 with per-block
               MSE: launch-bound, reported in GB/s only
  llama8       four bf16 14336 x 4096 tensors (Llama-3.1-8B MLP), narrow Normal
               sigma in {0.002, 0.005, 0.01, 0.05}, UE4M3 and UE5M3 scales without
               a per-tensor scale at block sizes 256 ... 8, MSE and split, with the
               three-term model's prediction beside the measured terms
  qwen14rot    bf16 13824 x 5120 Student-t(4) with 1 % outlier columns x20:
               MXFP4 and dynamic NVFP4, each without and with block rotation
  act5120      activation matrices of 1, 16, 128, 2048 and 8192 tokens x 5120:
               NVFP4 + rotation with per-token scales, NVFP4 with the per-tensor
               dynamic scale, MXFP4 + rotation; time per call for each
  qwen7search  the six qwen7 tensors, MXFP4 and dynamic NVFP4 with the per-block
               scale search (radius 1)
  gemm         a W4A4 Qwen2.5-7B MLP forward over 8192 tokens on MXFP4 operands:
               quantize the activations X (8192 x 3584) and H (8192 x 18944) to
               MXFP4, then the gate and up products (8192 x 18944 x 3584) and the
               down product (8192 x 3584 x 18944) against MXFP4 weights quantized
               beforehand, bf16 outputs.  Reported in TFLOP/s of the three products
               over the whole step; `roofline` is one up-projection call (scale
               packing + product) against the dense FP4 matrix-core peak.
"""
import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s of bf16 input quantized+packed+MSE'd (MXFP4/NVFP4); % of HBM peak"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "microscaling_fp4_quantization_amd", "csrc")
# Per workload: the roofline kernel's source file and its committed traffic record.
TRAFFIC = {
    "qwen14model": (os.path.join(CSRC, "fp4q_kernels.hip"),
                    os.path.join(ROOT, "profiles", "quantize_qwen14_model_traffic.json")),
    "qwen7": (os.path.join(CSRC, "fp4q_kernels.hip"),
              os.path.join(ROOT, "profiles", "quantize_nvfp4_qwen7_traffic.json")),
    "gemm": (os.path.join(CSRC, "fp4q_gemm.hip"),
             os.path.join(ROOT, "profiles", "gemm_mxfp4_qwen7_traffic.json")),
}


def kernel_source_hash(workload="qwen7") -> str:
    return hashlib.sha256(open(TRAFFIC[workload][0], "rb").read()).hexdigest()[:16]


def read_traffic(workload="qwen7"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC[workload][1]))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(workload):
        return None
    return t.get("hbm_bytes_per_launch")


# What one roofline "launch" is in each workload's counter runs: the kernels
# of one call (name fragment, grid size in work items or None for any), the
# bytes of the calibration copy, and the call's algorithmic bytes.
QWEN14_BATCH = 5    # tensors per batched call in the 48-layer step
COUNTER_LAYERS = 5  # layers the counter runs of that step cover (seven calls)


def _traffic_plan(workload):
    if workload == "qwen14model":
        import fp4_workloads as wl
        # The counter runs cover the first COUNTER_LAYERS layers in the default
        # grouping (QWEN14_BATCH consecutive tensors per call): the mean
        # algorithmic bytes and elements of one batched quantize launch there
        # (MXFP4 b32 and NVFP4 b16, relative per-block MSE).
        ns = [r * c for _, (r, c) in wl.QWEN14_PROJ] * COUNTER_LAYERS
        groups = -(-len(ns) // QWEN14_BATCH)
        alg = sum(n * (2 + 0.5 + 1 / 32 + 4 / 32) + n * (2 + 0.5 + 1 / 16 + 4 / 16) for n in ns) / (2 * groups)
        return {"parts": [("k_quantize", None)],
                "label": f"k_quantize_mx_batch (MXFP4 b32) and k_quantize_nv_batch (NVFP4 b16 under the "
                         f"per-tensor g), the step's launches, each over {QWEN14_BATCH} consecutive tensors "
                         "of the stack, with relative per-block MSE and the three-term split: mean per "
                         f"launch over the first {COUNTER_LAYERS} layers",
                "calib_bytes": 5120 * 5120 * 2, "alg_bytes": int(alg),
                "elems_per_batch_launch": sum(ns) / groups,
                "run": f"python -u bench.py --layers {COUNTER_LAYERS} --steps 1 --warmup 0 --no-cpu-baseline "
                       "--calibration-copy"}
    if workload == "qwen7":
        n = 18944 * 3584
        return {"parts": [("k_quantize<0, 1, 16, 0, true, false, false>", None)],
                "label": "k_quantize<bf16, UE, 16, no rotation, err, no sumsq> (one launch)",
                "calib_bytes": n * 2, "alg_bytes": int(n * (2 + 0.5 + 1 / 16 + 4 / 16)),
                "run": "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --calibration-copy"}
    if workload == "gemm":
        T, H, I = GEMM_TOKENS, 3584, 18944
        tiles = -(-T // 256) * -(-I // 256)
        return {"parts": [("k_gemm_mxfp4", tiles * 512), ("k_pack_scales", (-(-T // 32) + -(-I // 32)) * 256)],
                "label": "fp4_gemm_mxfp4 up projection 8192x18944x3584: k_pack_scales + k_gemm_mxfp4",
                "calib_bytes": I * H // 2,
                "alg_bytes": T * H // 2 + T * H // 32 + I * H // 2 + I * H // 32 + T * I * 2,
                "run": "python -u bench.py --workload gemm --steps 2 --warmup 1 --no-cpu-baseline "
                       "--calibration-copy"}
    raise SystemExit(f"no traffic plan for workload {workload}")


def write_traffic(workload, fetch_dir, write_dir, out_json=None):
    """Turn two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE; csv output, -o
    run) into the workload's traffic record and summary under profiles/.
    The counters read KiB per dispatch; each is scaled by what it reads for
    the calibration copy (the last `copyBuffer` dispatch) of known size."""
    import csv
    plan = _traffic_plan(workload)

    def load(d, counter):
        out = []
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                            float(r["Counter_Value"])))
        return out

    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = load(d, counter)
        copies = [r for r in rows if "copyBuffer" in r[1]]
        if not copies:
            raise SystemExit(f"{d}: no calibration copy dispatch")
        calib_kib = max(copies)[3]
        parts = []
        for frag, grid in plan["parts"]:
            vals = [r[3] for r in rows if frag in r[1] and (grid is None or r[2] == grid)]
            if not vals:
                raise SystemExit(f"{d}: no dispatch of {frag} (grid {grid})")
            parts.append((frag, grid, len(vals), sum(vals) / len(vals)))
        res[counter] = (calib_kib, parts)
    f_cal, f_parts = res["FETCH_SIZE"]
    w_cal, w_parts = res["WRITE_SIZE"]
    f_scale = plan["calib_bytes"] / (f_cal * 1024)
    w_scale = plan["calib_bytes"] / (w_cal * 1024)
    f_kib = sum(p[3] for p in f_parts)
    w_kib = sum(p[3] for p in w_parts)
    hbm = int(round(f_kib * 1024 * f_scale + w_kib * 1024 * w_scale))
    src, default_json = TRAFFIC[workload]
    out_json = out_json or default_json
    rel = lambda d: os.path.relpath(os.path.abspath(d), ROOT)
    cmds = [f"rocprofv3 --pmc {c} --output-format csv -d {rel(d)} -o run -- " + plan["run"]
            for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))]
    rec = {"kernel": plan["label"], "kernel_source_sha256_16": kernel_source_hash(workload),
           "fetch_kib_per_launch": round(f_kib, 1), "write_kib_per_launch": round(w_kib, 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": plan["alg_bytes"],
           "commands": cmds}
    json.dump(rec, open(out_json, "w"), indent=1)
    lines = [f"# HBM traffic per launch: bench.py workload `{workload}`", "",
             "Commands (from the repository root on the MI355X box), one counter per run, then",
             f"`python bench.py --workload {workload} --write-traffic {rel(fetch_dir)} {rel(write_dir)}`"
             " to write this file:", "", "```",
             *cmds, "```", "",
             f"The calibration copy moves {plan['calib_bytes']:,} bytes each way; the counters read "
             f"{f_cal:,.1f} KiB (fetch) and {w_cal:,.1f} KiB (write) for it, so the scales are "
             f"x{f_scale:.4f} (fetch) and x{w_scale:.4f} (write).", "",
             "| kernel | grid (work items) | dispatches | FETCH_SIZE KiB (mean) | WRITE_SIZE KiB (mean) |",
             "|---|---|---|---|---|"]
    for fp, wp in zip(f_parts, w_parts):
        lines.append(f"| `{fp[0]}` | {fp[1] if fp[1] else 'any'} | {fp[2]} | {fp[3]:,.1f} | {wp[3]:,.1f} |")
    lines += ["", f"Per launch ({plan['label']}): {f_kib * 1024 * f_scale / 1e6:.2f} MB read and "
                  f"{w_kib * 1024 * w_scale / 1e6:.2f} MB written, {hbm / 1e6:.2f} MB in all, against "
                  f"{plan['alg_bytes'] / 1e6:.2f} MB algorithmic (ratio {hbm / plan['alg_bytes']:.4f}).  "
                  f"Taken on kernel source sha256[:16] = {rec['kernel_source_sha256_16']} "
                  f"({os.path.relpath(src, ROOT)}); bench.py reports this traffic only while the "
                  "source is unchanged."]
    open(out_json[:-5] + ".md", "w").write("\n".join(lines) + "\n")
    print(json.dumps(rec))


COUNTER_CLOCK_GHZ = 2.4  # MI355X peak engine clock; the clock under load is lower


def write_counters(workload, out_md, bench_line, dirs):
    """Summarise rocprofv3 counter runs (csv output, -o run, of the workload's
    counter command) per kernel instantiation: instructions per 512-element
    chunk, and the derived busy figures rocprofv3 computes.  `bench_line` is
    an untraced bench.py JSON line of the same workload; its per-format
    launch times give the VALU issue share (VALU wave-instructions over
    256 CUs x the launch time x the peak clock, one wave-instruction per CU
    per cycle; a lower bound, since the clock under load is lower)."""
    import csv
    import fp4_workloads as wl
    if workload != "qwen14model":
        raise SystemExit("--write-counters covers the qwen14model workload")
    plan = _traffic_plan(workload)
    line = json.loads(open(bench_line).read().strip().splitlines()[-1])
    spec_us = {k: v["us_per_launch"] for k, v in line["roofline"]["per_spec"].items()}
    amax_us = line["roofline"].get("s0_amax_pass", {}).get("us_per_launch")
    layer_elems = sum(r * c for _, (r, c) in wl.QWEN14_PROJ)
    mean_elems = layer_elems / len(wl.QWEN14_PROJ)
    batch_elems = plan["elems_per_batch_launch"]
    chunks = mean_elems / 512
    kinds = {"k_quantize_mx_batch<0": ("MXFP4 b32 quantize of a batch of tensors in one launch "
                                       "(relative MSE, three-term split, tensor maxima)", spec_us.get("mx32")),
             "k_quantize_nv_batch<0, 16": ("NVFP4 b16 quantize of a batch of tensors in one launch "
                                           "(given per-tensor g, relative MSE, three-term split)",
                                           spec_us.get("nv16_dyn")),
             "k_quantize_amax<0": ("MXFP4 b32 quantize (relative MSE, three-term split, tensor maximum)",
                                   spec_us.get("mx32")),
             "k_quantize<0, 0, 32": ("MXFP4 b32 quantize (relative MSE, three-term split)", spec_us.get("mx32")),
             "k_quantize<0, 1, 16": ("NVFP4 b16 quantize (dynamic g, relative MSE, three-term split)",
                                     spec_us.get("nv16_dyn")),
             "k_amax": ("amax pre-pass of dynamic NVFP4 (also sums x^2)", amax_us)}
    acc = {}
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            kn = r["Kernel_Name"]
            key = next((k for k in kinds if k in kn), None)
            if key is None:
                continue
            a = acc.setdefault(key, {})
            a.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    rel = lambda d: os.path.relpath(os.path.abspath(d), ROOT)
    lines = [f"# Instruction and busy counters per launch: bench.py workload `{workload}`", "",
             "Counter runs (from the repository root on the MI355X box), one counter set per run, "
             "csv output under the directories named:", "", "```"]
    sets = []
    for d in dirs:
        names = []
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] not in names:
                names.append(r["Counter_Name"])
        sets.append(" ".join(names))
    lines += [f"rocprofv3 --pmc {c} --output-format csv -d {rel(d)} -o run -- {plan['run']}"
              for c, d in zip(sets, dirs)]
    lines += ["```", "", f"then `python bench.py --workload {workload} --write-counters {out_md} "
              f"{rel(bench_line)} {' '.join(rel(d) for d in dirs)}`.  Launch times come from the untraced "
              f"bench line ({rel(bench_line)}: per-format mean over the step's launches).", "",
              f"A chunk is 512 elements; a batched launch of the counter runs covers {batch_elems / 1e6:.2f} M "
              f"elements on average ({batch_elems / 512:,.0f} chunks), a single-tensor launch "
              f"{mean_elems / 1e6:.2f} M ({chunks:,.0f} chunks).  VALU issue share = VALU wave-instructions / "
              f"(256 CUs x launch time x {COUNTER_CLOCK_GHZ} GHz), one wave-instruction per CU per cycle; "
              "the clock under load is lower than the peak, so the true share is higher.  VALUBusy, "
              "SALUBusy and MemUnitStalled are rocprofv3's derived metrics (percent of the counter "
              "window, which also covers the dispatch's start and drain).", ""]
    hdr = None
    for key, (label, us) in kinds.items():
        if key not in acc:
            continue
        a = acc[key]
        per_launch_chunks = batch_elems / 512 if "_batch<" in key else chunks
        mean = {c: sum(v) / len(v) for c, v in a.items() if not c.startswith("_")}
        n_disp = max(len(v) for c, v in a.items() if not c.startswith("_"))
        lines += [f"## `{key}...>`: {label}", "",
                  f"{n_disp} dispatches per counter; launch time {us} us (untraced, mean over the "
                  "format's launches in the bench line).", "", "| counter | mean per launch | per chunk |",
                  "|---|---|---|"]
        for c in sorted(mean):
            per = f"{mean[c] / per_launch_chunks:.2f}" if c.startswith("SQ_INSTS") else ""
            lines.append(f"| {c} | {mean[c]:,.2f} | {per} |")
        if "SQ_INSTS_VALU" in mean and us:
            share = mean["SQ_INSTS_VALU"] / (256 * us * 1e-6 * COUNTER_CLOCK_GHZ * 1e9)
            lines += ["", f"VALU issue share (lower bound): {share:.3f}"]
        lines.append("")
    open(out_md, "w").write("\n".join(lines))
    print("\n".join(lines))


def _short_kernel(name):
    name = name.replace("fp4q::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0] if "<" in name.split("(")[0] else name


def write_trace(workload, out_md, bench_line, trace_dir, command, untraced_line=None):
    """Summarise a `rocprofv3 --kernel-trace --stats` run of bench.py (csv
    output, -o bench) into OUT_MD: every kernel's statistics, and the launches
    of the roofline leg (the step replayed on one stream after the warm-up
    and timed steps and one warm replay) set against the leg's own HIP-event
    timing in the bench line the same run printed, and, when given, in an
    untraced run of the same command (the tracer adds work around every
    dispatch, which the traced run's event pairs include)."""
    import csv
    line = json.loads(open(bench_line).read().strip().splitlines()[-1])
    r = line["roofline"]
    per_step_q = r["launches"]
    specs = list(r["per_spec"])
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_stats.csv"))))
    trace = sorted(csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_trace.csv"))),
                   key=lambda t: int(t["Dispatch_Id"]))
    import re
    quant = [t for t in trace if re.search(r"k_quantize(_amax|_mx_batch|_nv_batch)?<", t["Kernel_Name"])]
    start = (line["warmup"] + line["steps"] + 1) * per_step_q
    leg = quant[start:start + per_step_q]
    if len(leg) != per_step_q:
        raise SystemExit(f"trace holds {len(quant)} quantize launches; the leg needs {start + per_step_q}")
    dur = lambda t: (int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) / 1e3
    rel = lambda d: os.path.relpath(os.path.abspath(d), ROOT)
    un = json.loads(open(untraced_line).read().strip().splitlines()[-1]) if untraced_line else None
    lines = [f"# Kernel trace: bench.py workload `{workload}`", "",
             "Command (from the repository root on the MI355X box), then "
             f"`python bench.py --workload {workload} --write-trace {out_md} {rel(bench_line)} "
             f"{rel(trace_dir)} \"<command>\"" + (f" {rel(untraced_line)}" if un else "") +
             "` to write this file:", "", "```", command, "```", "",
             "| kernel | calls | total us | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for s in stats:
        lines.append(f"| `{_short_kernel(s['Name'])[:100]}` | {s['Calls']} | "
                     f"{int(s['TotalDurationNs']) / 1e3:.1f} | {float(s['AverageNs']) / 1e3:.3f} | "
                     f"{int(s['MinNs']) / 1e3:.3f} | {int(s['MaxNs']) / 1e3:.3f} |")
    lines += ["", f"The timed steps run their calls on {line['config'].get('streams', 1)} streams, so "
              "their launches overlap and the statistics above mix overlapped and lone launches.  "
              f"The roofline leg is quantize launches {start} to {start + per_step_q - 1} in launch "
              f"order ({line['warmup']} warm-up and {line['steps']} timed steps, then one warm replay "
              "come before it): one step's calls replayed on one stream.", "",
              "| roofline leg, per format | launches | trace avg us | events, traced run | difference |"
              + (" events, untraced run | difference |" if un else ""),
              "|---|---|---|---|---|" + ("---|---|" if un else "")]

    def row(tag, n, tr, ev, ev_un):
        cells = f"| {tag} | {n} | {tr:.3f} | {ev:.3f} | {100 * (ev - tr) / tr:+.2f} % |"
        if ev_un is not None:
            cells += f" {ev_un:.3f} | {100 * (ev_un - tr) / tr:+.2f} % |"
        return cells
    for si, tag in enumerate(specs):
        sel = [dur(t) for i, t in enumerate(leg) if i % len(specs) == si]
        lines.append(row(tag, len(sel), sum(sel) / len(sel), r["per_spec"][tag]["us_per_launch"],
                         un["roofline"]["per_spec"][tag]["us_per_launch"] if un else None))
    lines.append(row("all", len(leg), sum(dur(t) for t in leg) / len(leg), r["us_per_launch"],
                     un["roofline"]["us_per_launch"] if un else None))
    lines += ["", f"Bench line of the traced run: value {line['value']} GB/s, "
              f"{line['ms_per_step']} ms per step, roofline frac {r['frac']}."]
    if un:
        lines += ["", f"Untraced bench.py run (the same workload and GPU legs; it also ran the CPU baseline leg) in the same session on the same box: value {un['value']} GB/s, "
                  f"{un['ms_per_step']} ms per step, roofline frac {un['roofline']['frac']}.  Under "
                  "the tracer every dispatch carries the tracer's own completion work, which the "
                  "traced run's event pairs (recorded around each launch) include and the kernels' "
                  "own start and end timestamps do not; the untraced run's events measure the "
                  "launches without it."]
    lines.append("")
    open(out_md, "w").write("\n".join(lines))
    print("\n".join(lines))


# ------------------------------------------------------------------ workloads
class Spec:
    """One quantization call applied to every tensor of a workload.  fmt "pair"
    is one fp4_quantize_mx_nv call: MXFP4 and dynamic NVFP4 (block `block`)
    of the tensor, the NVFP4 per-tensor scale taken from the MXFP4 pass."""

    def __init__(self, tag, fmt, block, scale_fmt=1, gmode=0, rotate=0, mse_kind=0,
                 block_mse=True, stats=True, radius=None):
        self.tag, self.fmt, self.block, self.scale_fmt = tag, fmt, block, scale_fmt
        self.gmode, self.rotate, self.mse_kind = gmode, rotate, mse_kind
        self.block_mse, self.stats = block_mse, stats
        self.radius = radius  # per-block scale search radius, None for the plain call
        self.parts = []
        if fmt == "pair":
            self.parts = [Spec("mx32", "mx", 32, mse_kind=mse_kind, block_mse=block_mse, stats=stats),
                          Spec(f"nv{block}_dyn", "nv", block, 1, 1, mse_kind=mse_kind,
                               block_mse=block_mse, stats=stats)]

    @property
    def formats(self):
        """Quantizations of each tensor one call performs."""
        return len(self.parts) if self.parts else 1

    def algorithmic_bytes(self, n, in_bytes):
        """Bytes every kernel of the call must move: the amax pre-pass read (dynamic
        NVFP4 alone), the quantize read, codes, scale bytes and per-block MSE."""
        if self.parts:
            return sum(p.quantize_bytes(n, in_bytes) for p in self.parts)
        b = self.quantize_bytes(n, in_bytes)
        if self.fmt == "nv" and self.gmode == 1:
            b += n * in_bytes
        return b

    def launches(self):
        """The kernels one call launches, in order, each with the format it serves."""
        if self.parts:  # the MXFP4 pass's reduction also forms g
            return [(k, p.tag) for p in self.parts for k in ("quantize", "finalize")]
        seq = ["amax"] if (self.fmt == "nv" and self.gmode == 1) else []
        seq.append("quantize")
        if self.stats:
            seq.append("finalize")
        return [(k, self.tag) for k in seq]

    def part(self, tag):
        return next(p for p in self.parts if p.tag == tag) if self.parts else self

    def quantize_bytes(self, n, in_bytes):
        """Algorithmic bytes of the quantize kernel alone: its read, the codes,
        scale bytes and per-block MSE."""
        return n * (in_bytes + 0.5 + 1.0 / self.block + (4.0 / self.block if self.block_mse else 0))

    def describe(self):
        if self.parts:
            return " + ".join(p.describe() for p in self.parts) + " (one call, g from the MXFP4 pass)"
        if self.fmt == "mx":
            s = "MXFP4 b32"
        else:
            s = f"{'UE4M3' if self.scale_fmt == 1 else 'UE5M3'} b{self.block}"
            s += {0: "", 1: " dynamic g", 2: " given g", 3: " per-row g"}[self.gmode]
        if self.rotate:
            s += f" rot{self.rotate}"
        if self.radius is not None:
            s += f" scale search radius {self.radius}"
        return s


class Workload:
    """`sample` = (description, number of tensors, spec indices) of the oracle's
    bounded CPU sample.  `per_call` asks for a time per (tensor, spec) pair in
    the breakdown (latency-bound workloads)."""

    def __init__(self, name, config, make_tensors, specs, steps, warmup, sample, per_call=False,
                 batch=0):
        self.name, self.config, self.make_tensors = name, config, make_tensors
        self.specs, self.steps, self.warmup, self.sample = specs, steps, warmup, sample
        self.per_call = per_call
        # batch > 0: a "pair" spec is issued as fp4_quantize_mx_nv_batch calls over
        # consecutive groups of `batch` tensors (one layer of the stack).
        self.batch = batch


def _qwen7_tensors():
    import fp4_workloads as wl
    return [wl.qwen7_mlp(si, gi) for si in range(2) for gi in range(3)]


def _qwen05_tensors():
    import torch
    import fp4_workloads as wl
    return [torch.from_numpy(wl.qwen05_up())]


def _llama8_tensors():
    import fp4_workloads as wl
    return [wl.llama8_sweep(i) for i in range(len(wl.LLAMA8_SIGMAS))]


def _qwen14rot_tensors():
    import fp4_workloads as wl
    return [wl.qwen14_outliers()]


def _act5120_tensors():
    import fp4_workloads as wl
    return [wl.activations_5120(m) for m in wl.ACT_TOKENS]


QWEN14_LAYERS_RUN = None  # --layers: leading layers of the stack to run (counter runs)


def _qwen14model_tensors():
    """Generated on host threads (one PCG64 stream per tensor, as the recipe says)
    and moved to the device one by one; yields host tensors lazily."""
    import fp4_workloads as wl
    layers = QWEN14_LAYERS_RUN or wl.QWEN14_LAYERS
    keys = [(layer, p) for layer in range(layers) for p in range(len(wl.QWEN14_PROJ))]
    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        for t in ex.map(lambda k: wl.qwen14_layer_tensor(*k), keys):
            yield t


WORKLOADS = {
    "qwen7": Workload(
        "qwen2.5-7b-mlp-nvfp4",
        {"tensors": "6 bf16: 18944x3584 and 3584x18944, sigma 0.01/0.02/0.04",
         "format": "NVFP4: block 16, UE4M3 scales, dynamic FP32 per-tensor scale",
         "outputs": "codes + scales + per-block MSE + three-term error split"},
        _qwen7_tensors, [Spec("nv16_dyn", "nv", 16, 1, 1)], 50, 5,
        ("4 of the 6 tensors (the three 18944x3584 ones and 3584x18944 with sigma 0.01), whole",
         4, [0])),
    "qwen05": Workload(
        "qwen2.5-0.5b-up-mxfp4-fp32",
        {"tensors": "1 fp32 4864x896, N(0, 0.02), seed 0",
         "format": "MXFP4: block 32, E8M0 scales", "outputs": "codes + scales + per-block MSE"},
        _qwen05_tensors, [Spec("mx32", "mx", 32, stats=False)], 400, 20,
        ("the tensor, whole", 1, [0])),
    "llama8": Workload(
        "llama3.1-8b-mlp-ue4m3-block-sweep",
        {"tensors": "4 bf16 14336x4096, sigma 0.002/0.005/0.01/0.05",
         "format": "UE4M3 and UE5M3 scales, no per-tensor scale, blocks 256/128/64/32/16/8",
         "outputs": "codes + scales + per-block MSE + three-term error split"},
        _llama8_tensors,
        [Spec(f"ue4m3_b{b}", "nv", b, 1, 0) for b in (256, 128, 64, 32, 16, 8)] +
        [Spec(f"ue5m3_b{b}", "nv", b, 2, 0) for b in (256, 128, 64, 32, 16, 8)],
        20, 2, ("2 of the 4 tensors (sigma 0.002 and 0.005), whole, at block 16", 2, [4, 10])),
    "qwen14rot": Workload(
        "qwen2.5-14b-mlp-outliers-rotation",
        {"tensors": "1 bf16 13824x5120, Student-t(4) sd 0.02, 51 outlier columns x20",
         "format": "MXFP4 b32 and NVFP4 b16 dynamic g, each without and with block Hadamard",
         "outputs": "codes + scales + per-block MSE + three-term error split"},
        _qwen14rot_tensors,
        [Spec("mx32", "mx", 32), Spec("mx32_rot", "mx", 32, rotate=32),
         Spec("nv16_dyn", "nv", 16, 1, 1), Spec("nv16_dyn_rot", "nv", 16, 1, 1, rotate=16)],
        50, 5, ("the tensor, whole", 1, [0, 3])),
    "qwen7search": Workload(
        "qwen2.5-7b-mlp-scale-search",
        {"tensors": "6 bf16: 18944x3584 and 3584x18944, sigma 0.01/0.02/0.04",
         "format": "MXFP4 b32 and NVFP4 b16 dynamic g, per-block scale search over the "
                   "max-based code and its neighbours (radius 1)",
         "outputs": "codes + scales + per-block MSE + three-term error split"},
        _qwen7_tensors,
        [Spec("mx32_search1", "mx", 32, radius=1), Spec("nv16_dyn_search1", "nv", 16, 1, 1, radius=1)],
        20, 2, ("1 of the 6 tensors (18944x3584, sigma 0.01), whole", 1, [0])),
    "act5120": Workload(
        "activations-5120-token-shapes",
        {"tensors": "5 bf16 activation matrices M x 5120, M = 1, 16, 128, 2048, 8192",
         "format": "NVFP4 b16 + rotation 16 with one dynamic scale per token, NVFP4 b16 with "
                   "the per-tensor dynamic scale, MXFP4 b32 + rotation 32",
         "outputs": "codes + scales (the inference use: no MSE)"},
        _act5120_tensors,
        [Spec("nv16_rot_rowg", "nv", 16, 1, 3, rotate=16, block_mse=False, stats=False),
         Spec("nv16_tensor_g", "nv", 16, 1, 1, block_mse=False, stats=False),
         Spec("mx32_rot", "mx", 32, rotate=32, block_mse=False, stats=False)],
        50, 5, ("all five matrices, whole", 5, [0, 1, 2]),
        per_call=True),
    "qwen14model": Workload(
        "qwen2.5-14b-shaped-model-sweep",
        {"tensors": "336 bf16 (48 layers x q,k,v,o,gate,up,down), N(0, 0.02), 13.2e9 params",
         "format": "MXFP4 b32 and NVFP4 b16 dynamic g",
         "outputs": "codes + scales + relative per-block MSE + per-tensor split"},
        _qwen14model_tensors,
        [Spec("mx32+nv16_dyn", "pair", 16, mse_kind=1)],
        20, 3, ("layer 0's seven projections (q, k, v, o, gate, up, down), whole", 7, [0]),
        batch=QWEN14_BATCH),
}


# ------------------------------------------------------------------ GEMM workload
GEMM_TOKENS = 8192
GEMM_METRIC = ("TFLOP/s of MXFP4 x MXFP4 products (W4A4 Qwen2.5-7B MLP, 8192 tokens, "
               "activation quantization included); % of dense FP4 matrix-core peak")
MFMA_FP4_PEAK_TFLOPS = 10100.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
GEMM_SAMPLE_ROWS = 12


def gemm_main(args, steps, warmup):
    import numpy as np
    import torch
    import microscaling_fp4_quantization_amd as fq
    import fp4_workloads as wl

    dev = torch.device("cuda:0")
    hidden, inter = wl.QWEN7_SHAPES[1]
    T = GEMM_TOKENS
    x_host = wl.activations_f32(T, hidden, [7, T, hidden])
    acts = {"x": wl.to_bf16(x_host).to(dev),
            "h": wl.to_bf16(wl.activations_f32(T, inter, [7, T, inter])).to(dev)}
    w_host = {"gate": wl.qwen7_mlp(0, 0), "up": wl.qwen7_mlp(0, 1), "down": wl.qwen7_mlp(1, 2)}
    weights = {}
    for name, w in w_host.items():
        q = fq.mxfp4_quantize(w.to(dev), 0, block_mse=False, stats=False)
        weights[name] = (q.codes, q.scales)
    qa = {k: fq.mxfp4_quantize(v, 0, block_mse=False, stats=False) for k, v in acts.items()}
    prods = [("gate", "x"), ("up", "x"), ("down", "h")]
    outs = {n: torch.empty((T, weights[n][0].shape[0]), dtype=torch.bfloat16, device=dev)
            for n, _ in prods}
    # Decode-sized products (a few tokens against the same weights) for the
    # breakdown: the first rows of the quantized activations.
    decode = [(tok, n, a) for tok in (1, 16) for n, a in (("up", "x"), ("down", "h"))]
    need = max([fq.lib().fp4_gemm_workspace_bytes(T, weights[n][0].shape[0], acts[a].shape[1])
                for n, a in prods] +
               [fq.lib().fp4_gemm_nvfp4_workspace_bytes(T, weights["up"][0].shape[0], hidden)] +
               [fq.lib().fp4_gemm_workspace_bytes(tok, weights[n][0].shape[0], acts[a].shape[1])
                for tok, n, a in decode])
    ws = fq.gemm_workspace(dev, need)
    flops = {n: 2.0 * T * weights[n][0].shape[0] * acts[a].shape[1] for n, a in prods}

    def quantize(a):
        fq.mxfp4_quantize(acts[a], 0, codes=qa[a].codes, scales=qa[a].scales, block_mse=False,
                          stats=False)

    def gemm(n, a):
        fq.fp4_gemm_mxfp4(qa[a].codes, qa[a].scales, weights[n][0], weights[n][1],
                          torch.bfloat16, out=outs[n], ws=ws)

    def step():
        quantize("x")
        gemm("gate", "x")
        gemm("up", "x")
        quantize("h")
        gemm("down", "h")

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    t_wall = time.perf_counter()
    ms_step = time_region(torch, stream, step, steps)
    t_wall = time.perf_counter() - t_wall
    total_flops = sum(flops.values())
    value = total_flops / (ms_step * 1e-3) / 1e12

    reps = max(10, steps)
    breakdown = {}
    for n, a in prods:
        ms = time_region(torch, stream, lambda n=n, a=a: gemm(n, a), reps)
        breakdown[f"gemm_{n}"] = {"shape_MxNxK": f"{T}x{weights[n][0].shape[0]}x{acts[a].shape[1]}",
                                  "us_per_call": round(ms * 1e3, 2),
                                  "TFLOPs": round(flops[n] / (ms * 1e-3) / 1e12, 1)}
    for tok, n, a in decode:
        wc, wsc = weights[n]
        cd = torch.empty((tok, wc.shape[0]), dtype=torch.bfloat16, device=dev)
        fn = lambda tok=tok, n=n, a=a, cd=cd: fq.fp4_gemm_mxfp4(
            qa[a].codes[:tok], qa[a].scales[:tok], weights[n][0], weights[n][1], torch.bfloat16,
            out=cd, ws=ws)
        fn()
        ms = time_region(torch, stream, fn, max(50, steps))
        wbytes = wc.numel() + wsc.numel()
        breakdown[f"decode_{n}_{tok}tok"] = {
            "shape_MxNxK": f"{tok}x{wc.shape[0]}x{acts[a].shape[1]}",
            "us_per_call": round(ms * 1e3, 2),
            "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1)}
    # The same up projection in NVFP4 (block 16, UE4M3, dynamic g; bf16 matrix
    # cores, so its peak is the dense bf16 one).
    nw = fq.nvfp4_quantize(w_host["up"].to(dev), 16, fq.FMT_UE4M3, fq.G_DYNAMIC, block_mse=False,
                           stats=False)
    nx = fq.nvfp4_quantize(acts["x"], 16, fq.FMT_UE4M3, fq.G_DYNAMIC, block_mse=False, stats=False)
    cn = torch.empty_like(outs["up"])
    nv_fn = lambda: fq.fp4_gemm_nvfp4(nx.codes, nx.scales, nx.g, nw.codes, nw.scales, nw.g,
                                      torch.bfloat16, out=cn, ws=ws)
    nv_fn()
    ms = time_region(torch, stream, nv_fn, reps)
    breakdown["nvfp4_gemm_up"] = {"shape_MxNxK": breakdown["gemm_up"]["shape_MxNxK"],
                                  "us_per_call": round(ms * 1e3, 2),
                                  "TFLOPs": round(flops["up"] / (ms * 1e-3) / 1e12, 1),
                                  "frac_of_bf16_dense_peak": round(flops["up"] / (ms * 1e-3) / 1e12
                                                                   / MFMA_BF16_PEAK_TFLOPS, 4)}
    del nw
    for a in ("x", "h"):
        ms = time_region(torch, stream, lambda a=a: quantize(a), reps)
        breakdown[f"quantize_{a}"] = {"shape": "x".join(map(str, acts[a].shape)),
                                      "us_per_call": round(ms * 1e3, 2),
                                      "input_GBps": round(acts[a].numel() * 2 / (ms * 1e-3) / 1e9, 1)}
    up = breakdown["gemm_up"]
    achieved = flops["up"] / (up["us_per_call"] * 1e-6) / 1e12
    if args.calibration_copy:
        src = weights["up"][0]
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP4_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP4_PEAK_TFLOPS, 4),
                "traffic": read_traffic("gemm"),
                "kernel": "fp4_gemm_mxfp4 up projection (k_pack_scales + k_gemm_mxfp4)",
                "us_per_launch": up["us_per_call"], "algorithmic_flops_per_launch": flops["up"]}
    line = {
        "metric": GEMM_METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4-e2m1 x fp4-e2m1, f32 accumulate",
        "data": "synthetic (seeded numpy PCG64, rounded to bf16, then MXFP4)",
        "config": {"workload": "qwen2.5-7b-mlp-w4a4-gemm", "tokens": T, "hidden": hidden,
                   "intermediate": inter, "format": "MXFP4 operands (E2M1, E8M0 per 32), bf16 C",
                   "flops_per_step": total_flops},
        "roofline": roofline,
        "step_breakdown": {"wall_s_timed_region": round(t_wall, 3), **breakdown},
    }
    if not args.no_cpu_baseline:
        import oracle
        r = GEMM_SAMPLE_ROWS
        qx = oracle.quantize(np.ascontiguousarray(x_host[:r]), oracle.FMT_MXFP4, 32)
        qw = oracle.quantize(w_host["up"].float().numpy(), oracle.FMT_MXFP4, 32)
        t = time.perf_counter()
        oracle.gemm_mxfp4(qx["codes"], qx["scales"], qw["codes"], qw["scales"], r, inter, hidden)
        el = time.perf_counter() - t
        line["cpu_baseline"] = {
            "value": round(2.0 * r * inter * hidden / el / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the up projection for the first {r} tokens ({r}x{inter}x{hidden}), "
                      "single-threaded C oracle in binary64",
            "seconds": round(el, 2)}
    print(json.dumps(line), flush=True)


# ------------------------------------------------------------------ running
class Runner:
    """Device buffers and calls for every (tensor, spec) pair of a workload.

    The step issues its calls round-robin over `n_streams` HIP streams (default
    priority, one workspace each), so that independent calls overlap: one
    tensor's memory-bound amax pass runs beside another's quantize pass.  The
    streams join the caller's stream at the start and end of every step."""

    def __init__(self, fq, torch, dev, xs, specs, n_streams=1, batch=0):
        self.fq, self.torch, self.dev, self.xs, self.specs = fq, torch, dev, xs, specs
        # With batch > 0 (a single "pair" spec), a call covers `batch` consecutive
        # tensors; calls alternate over the streams.
        self.batch = batch if (batch and len(specs) == 1 and specs[0].parts) else 0
        self.groups = ([list(range(i, min(i + self.batch, len(xs)))) for i in range(0, len(xs), self.batch)]
                       if self.batch else None)
        self.streams = [torch.cuda.current_stream(dev)] + [torch.cuda.Stream(dev)
                                                           for _ in range(n_streams - 1)]
        ws_bytes = fq.workspace_bytes()
        self.wss = [fq.workspace(dev)] + [torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
                                          for _ in range(n_streams - 1)]
        self.ws = self.wss[0]
        self.out = {}
        # Outputs are shared by the calls of one stream on tensors of one shape
        # (each call overwrites them); g and stats are per call so the given-g
        # replay can reuse the step's g.
        shared = {}
        k = 0
        def outputs(r, c, block, stream, slot=0):
            key = (r, c, block, stream, slot)
            if key not in shared:
                shared[key] = dict(
                    codes=torch.empty((r, c // 2), dtype=torch.uint8, device=dev),
                    scales=torch.empty((r, c // block), dtype=torch.uint8, device=dev),
                    block_mse=torch.empty((r, c // block), dtype=torch.float32, device=dev))
            o = dict(shared[key])
            o["stats"] = fq.new_stats(dev)
            return o

        for ti, x in enumerate(xs):
            r, c = x.shape
            for si, s in enumerate(specs):
                stream = k % n_streams
                slot = 0
                if self.batch:  # distinct outputs within a call, one stream per call
                    stream, slot = (ti // self.batch) % n_streams, ti % self.batch
                k += 1
                if s.parts:
                    o = {p.tag: outputs(r, c, p.block, stream, slot) for p in s.parts}
                else:
                    o = outputs(r, c, s.block, stream)
                o["g"] = torch.ones(r if s.gmode == 3 else 1, dtype=torch.float32, device=dev)
                o["stream"] = stream
                self.out[(ti, si)] = o

    def call(self, ti, si, given=False, ws=None):
        fq, x, s, o = self.fq, self.xs[ti], self.specs[si], self.out[(ti, si)]
        ws = self.ws if ws is None else ws
        if s.parts:
            mx, nv = ({"codes": o[p.tag]["codes"], "scales": o[p.tag]["scales"],
                       "block_mse": o[p.tag]["block_mse"] if s.block_mse else False,
                       "stats": o[p.tag]["stats"] if (s.stats and not given) else False}
                      for p in s.parts)
            fq.fp4_quantize_mx_nv(x, s.block, mse_kind=s.mse_kind, mx=mx, nv=nv, g=o["g"], ws=ws)
            return
        bm = o["block_mse"] if s.block_mse else False
        if s.radius is not None:
            fmt = fq.FMT_MXFP4 if s.fmt == "mx" else s.scale_fmt
            gmode = fq.G_GIVEN if (given and s.gmode == 1) else s.gmode
            st = o["stats"] if (s.stats and not given) else False
            fq.fp4_quantize_search(x, fmt, s.block, gmode, o["g"] if s.fmt == "nv" else None,
                                   s.rotate, s.radius, codes=o["codes"], scales=o["scales"],
                                   block_mse=bm, mse_kind=s.mse_kind, stats=st, ws=ws)
        elif s.fmt == "mx":
            st = o["stats"] if (s.stats and not given) else False
            fq.mxfp4_quantize(x, s.rotate, codes=o["codes"], scales=o["scales"], block_mse=bm,
                              mse_kind=s.mse_kind, stats=st, ws=ws)
        else:
            gmode = fq.G_GIVEN if (given and s.gmode == 1) else s.gmode
            st = o["stats"] if (s.stats and not given) else False
            fq.nvfp4_quantize(x, s.block, s.scale_fmt, gmode, o["g"], s.rotate, codes=o["codes"],
                              scales=o["scales"], block_mse=bm, mse_kind=s.mse_kind, stats=st,
                              ws=ws)

    def call_batch(self, gi, ws=None):
        """One fp4_quantize_mx_nv_batch call over tensor group gi."""
        fq, s = self.fq, self.specs[0]
        ws = self.ws if ws is None else ws
        outs = []
        for ti in self.groups[gi]:
            o = self.out[(ti, 0)]
            mx, nv = ({"codes": o[p.tag]["codes"], "scales": o[p.tag]["scales"],
                       "block_mse": o[p.tag]["block_mse"] if s.block_mse else False,
                       "stats": o[p.tag]["stats"] if s.stats else False} for p in s.parts)
            outs.append((mx, nv, o["g"]))
        fq.fp4_quantize_mx_nv_batch([self.xs[ti] for ti in self.groups[gi]], s.block,
                                    mse_kind=s.mse_kind, outs=outs, ws=ws)

    def step(self, given=False, one_stream=False):
        """All calls of one step; with one_stream (or given, which also passes the
        dynamic per-tensor scale as given) they run back to back on the caller's
        stream."""
        if self.batch:
            one = one_stream or len(self.streams) == 1
            main = self.streams[0]
            if not one:
                for st in self.streams[1:]:
                    st.wait_stream(main)
            for gi in range(len(self.groups)):
                k = 0 if one else self.out[(self.groups[gi][0], 0)]["stream"]
                with self.torch.cuda.stream(self.streams[k]):
                    self.call_batch(gi, self.wss[k])
            if not one:
                for st in self.streams[1:]:
                    main.wait_stream(st)
            return
        if given or one_stream or len(self.streams) == 1:
            for ti in range(len(self.xs)):
                for si in range(len(self.specs)):
                    self.call(ti, si, given)
            return
        main = self.streams[0]
        for st in self.streams[1:]:
            st.wait_stream(main)
        for ti in range(len(self.xs)):
            for si in range(len(self.specs)):
                k = self.out[(ti, si)]["stream"]
                with self.torch.cuda.stream(self.streams[k]):
                    self.call(ti, si, False, self.wss[k])
        for st in self.streams[1:]:
            main.wait_stream(st)


def search_gain(fq, torch, run, si):
    """For a scale-search spec: total SSE over the workload with the search and
    with the max-based scales (radius 0), and their ratio."""
    s = run.specs[si]
    if s.radius is None or not s.stats:
        return {}
    tot = {}
    for radius in (s.radius, 0):
        acc = 0.0
        for ti, x in enumerate(run.xs):
            o = run.out[(ti, si)]
            fmt = fq.FMT_MXFP4 if s.fmt == "mx" else s.scale_fmt
            st = fq.new_stats(x.device)
            fq.fp4_quantize_search(x, fmt, s.block, s.gmode, o["g"] if s.fmt == "nv" else None,
                                   s.rotate, radius, codes=o["codes"], scales=o["scales"],
                                   block_mse=False, stats=st, ws=run.ws)
            d = fq.stats_dict(st)
            acc += d["sse_nonmax"] + d["sse_max"] + d["sse_zero"]
        tot[radius] = acc
    return {"sse_with_search": tot[s.radius], "sse_max_based": tot[0],
            "sse_ratio": round(tot[s.radius] / tot[0], 6)}


def time_graph(torch, fn, calls=20, replays=10):
    """us per call of fn, captured `calls` times into one HIP graph and replayed:
    the GPU time per call without the host's launch overhead."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (calls * replays)


def time_region(torch, stream, fn, reps):
    """ms per rep of fn, bracketed by HIP events on `stream`."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_call(oracle, xf, s, threads, pool):
    """One call of spec s on float32 array xf through the oracle, on row slices
    over `threads` threads (the per-tensor dynamic scale from the slices' amax)."""
    if s.parts:
        for p in s.parts:
            _oracle_call(oracle, xf, p, threads, pool)
        return
    fmt = oracle.FMT_MXFP4 if s.fmt == "mx" else s.scale_fmt
    rows = xf.shape[0]
    n = max(1, min(rows, 2 * threads))
    cuts = [rows * i // n for i in range(n + 1)]
    slices = [xf[cuts[i]:cuts[i + 1]] for i in range(n)]
    run = (lambda f, it: list(pool.map(f, it))) if pool else (lambda f, it: [f(v) for v in it])
    g, gmode = None, oracle.GMODE_NONE
    if s.fmt == "nv" and s.gmode == 1:
        g = oracle.dynamic_g(max(run(lambda a: oracle.tensor_amax(a, s.rotate), slices)))
        gmode = oracle.GMODE_GIVEN
    elif s.fmt == "nv" and s.gmode == 3:
        gmode = oracle.GMODE_ROW
    if s.radius is not None:
        run(lambda a: oracle.quantize_search(a, fmt, s.block, gmode, g, s.rotate, s.radius,
                                             s.mse_kind), slices)
    else:
        run(lambda a: oracle.quantize(a, fmt, s.block, gmode, g, s.rotate, s.mse_kind), slices)


def cpu_baseline(w, xs_host_sample):
    """The oracle as it stands, on a bounded sample of the workload: every spec
    of the step (or the sample's subset) on the sample tensors, on all host
    threads (row slices), and on one thread for the first sample tensor."""
    import numpy as np
    import oracle
    desc, n_tensors, spec_idx = w.sample
    specs = [w.specs[i] for i in spec_idx]
    threads = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                         else (os.cpu_count() or 1)))
    host = []
    for x in xs_host_sample[:n_tensors]:
        in_bytes = 4 if (hasattr(x, "dtype") and str(x.dtype) == "torch.float32") else 2
        host.append((x.float().numpy() if hasattr(x, "float") else np.asarray(x, np.float32), in_bytes))

    def timed(tensors, pool, nthreads):
        t = time.perf_counter()
        nbytes = 0
        for xf, in_bytes in tensors:
            for s in specs:
                _oracle_call(oracle, xf, s, nthreads, pool)
                nbytes += xf.size * in_bytes * s.formats
        return nbytes, time.perf_counter() - t

    with ThreadPoolExecutor(threads) as pool:
        nb, el = timed(host, pool, threads)
    nb1, el1 = timed(host[:1], None, 1)
    what = ", ".join(s.describe() for s in specs)
    return {"value": round(nb / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{desc}; {what}; C oracle on {threads} host threads (row slices)",
            "seconds": round(el, 2), "cpu_model": _cpu_model(),
            "single_thread": {"value": round(nb1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"the first of those tensors; {what}",
                              "seconds": round(el1, 2)}}


def three_term_table(fq, run, sigmas):
    """Per-element non-max, max-element and zero-rounding terms the GPU measured
    (each call's tensor stats) beside the three-term model's prediction for
    N(0, sigma) (stored by tests/golden/make_mse_model.py), and the small-block
    inversion (total MSE at block 8 above that at block 16)."""
    try:
        model = json.load(open(os.path.join(ROOT, "tests", "golden", "mse_model_llama8.json")))["terms"]
    except (OSError, ValueError):
        model = {}
    fmt_name = {1: "ue4m3", 2: "ue5m3"}
    table, totals = {}, {}
    for ti, x in enumerate(run.xs):
        sigma = sigmas[ti]
        n = x.numel()
        for si, s in enumerate(run.specs):
            st = fq.stats_dict(run.out[(ti, si)]["stats"])
            meas = [st["sse_nonmax"] / n, st["sse_max"] / n, st["sse_zero"] / n]
            name = fmt_name[s.scale_fmt]
            key = f"{name}/{sigma}/{s.block}"
            m = model.get(key)
            entry = {"measured_N_M_Z": [float(f"{v:.5g}") for v in meas],
                     "measured_total": float(f"{sum(meas):.5g}")}
            if m:
                entry["model_N_M_Z"] = [float(f"{m[k]:.5g}") for k in ("nonmax", "max", "zero")]
                entry["model_total"] = float(f"{m['total']:.5g}")
                entry["measured_over_model"] = round(sum(meas) / m["total"], 4)
            table.setdefault(name, {}).setdefault(str(sigma), {})[str(s.block)] = entry
            totals[(name, sigma, s.block)] = sum(meas)
    inversion = {}
    for name in ("ue4m3", "ue5m3"):
        for sigma in sigmas:
            if (name, sigma, 8) in totals and (name, sigma, 16) in totals:
                inversion[f"{name}/{sigma}"] = totals[(name, sigma, 8)] > totals[(name, sigma, 16)]
    return {"per_element_terms": table, "mse_b8_above_b16": inversion}


def launch_times(fq, torch, run):
    """Every call of one step replayed back to back on one stream, each kernel
    launch timed with HIP events on that stream (fp4q_profile_events).  Returns
    {kind: [(us, algorithmic bytes, format tag, tensor shape)]} for kinds amax,
    quantize and finalize."""
    seq = []
    if run.batch:  # one launch per pass covers a group of tensors
        s = run.specs[0]
        for grp in run.groups:
            n_el = sum(run.xs[ti].numel() for ti in grp)
            in_bytes = run.xs[grp[0]].element_size()
            label = f"batch of {len(grp)}"
            for kind, tag in s.launches():
                nb = s.part(tag).quantize_bytes(n_el, in_bytes) if kind == "quantize" else 0
                seq.append((label, tag, kind, nb))
    for ti, x in enumerate(run.xs if not run.batch else []):
        for si, s in enumerate(run.specs):
            in_bytes = x.element_size()
            for kind, tag in s.launches():
                nb = {"amax": x.numel() * in_bytes,
                      "quantize": s.part(tag).quantize_bytes(x.numel(), in_bytes), "finalize": 0}[kind]
                seq.append(("x".join(map(str, x.shape)), tag, kind, nb))
    run.step(given=False, one_stream=True)  # warm
    torch.cuda.synchronize()
    with fq.LaunchTimer(len(seq)) as t:
        run.step(given=False, one_stream=True)
    us = t.durations_us()
    if len(us) != len(seq):
        raise RuntimeError(f"recorded {len(us)} launches, expected {len(seq)}")
    out = {}
    for (label, tag, kind, nb), u in zip(seq, us):
        out.setdefault(kind, []).append((u, nb, tag, label))
    return out


def copy_ceiling(torch, xs):
    """A plain device copy of the largest tensor (cycling over up to three of
    that size, so the 256 MB last-level cache does not hold them): read + write
    bytes over time, the bandwidth this access pattern reaches."""
    big = max(x.numel() for x in xs)
    shape = next(x.shape for x in xs if x.numel() == big)
    src = [x.view(-1) for x in xs if x.numel() == big][:3]
    dst = torch.empty_like(src[0])
    stream = torch.cuda.current_stream()
    for i in range(3):
        dst.copy_(src[i % len(src)])
    reps = 30
    ms = time_region(torch, stream, lambda: [dst.copy_(src[i % len(src)]) for i in range(len(src))], reps)
    per = ms / len(src)
    nbytes = src[0].numel() * src[0].element_size()
    gbs = 2 * nbytes / (per * 1e-3) / 1e9
    return {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "us_per_copy": round(per * 1e3, 2),
            "what": f"device copy of a {'x'.join(map(str, shape))} {str(src[0].dtype)[6:]} tensor "
                    f"(read + write), {len(src)} distinct tensors cycled"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="qwen14model", choices=sorted(WORKLOADS) + ["gemm"])
    ap.add_argument("--layers", type=int, default=None,
                    help="qwen14model: run only the first LAYERS layers (short counter runs)")
    ap.add_argument("--separate", action="store_true",
                    help="issue a combined MXFP4 + NVFP4 call as its two separate calls "
                         "(NVFP4 with its own amax pass)")
    ap.add_argument("--no-batch", action="store_true",
                    help="issue the combined call tensor by tensor instead of one batched call "
                         "per layer")
    ap.add_argument("--batch", type=int, default=None,
                    help="tensors per batched call (default: the workload's; 5 for the 48-layer stack)")
    ap.add_argument("--streams", type=int, default=None,
                    help="HIP streams the step's independent calls are spread over (default 2, "
                         "or 1 when a step is a single call: the cross-stream joins would cost "
                         "more than a lone call takes)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain device copy of the first tensor (a kernel of "
                         "known traffic, for scaling rocprofv3 byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the workload's traffic record under profiles/ from two "
                         "rocprofv3 counter runs, then exit (no GPU needed)")
    ap.add_argument("--write-counters", nargs="+", metavar="ARG",
                    help="OUT_MD BENCH_LINE DIR...: summarise rocprofv3 instruction/busy counter "
                         "runs of the workload into OUT_MD, then exit (no GPU needed)")
    ap.add_argument("--write-trace", nargs="+", metavar="ARG",
                    help="OUT_MD BENCH_LINE TRACE_DIR COMMAND [UNTRACED_LINE]: summarise a rocprofv3 "
                         "--kernel-trace --stats run of bench.py into OUT_MD, then exit (no GPU needed)")
    args = ap.parse_args()
    if args.write_trace:
        if len(args.write_trace) not in (4, 5):
            ap.error("--write-trace needs OUT_MD BENCH_LINE TRACE_DIR COMMAND [UNTRACED_LINE]")
        write_trace(args.workload, *args.write_trace)
        return
    if args.write_traffic:
        write_traffic(args.workload, *args.write_traffic)
        return
    if args.write_counters:
        if len(args.write_counters) < 3:
            ap.error("--write-counters needs OUT_MD BENCH_LINE and at least one DIR")
        write_counters(args.workload, args.write_counters[0], args.write_counters[1],
                       args.write_counters[2:])
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by rows, with one max- and one sum-all-reduce)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "gemm":
        gemm_main(args, args.steps if args.steps is not None else 20,
                  args.warmup if args.warmup is not None else 3)
        return
    global QWEN14_LAYERS_RUN
    QWEN14_LAYERS_RUN = args.layers
    w = WORKLOADS[args.workload]
    if args.separate:
        specs = [p for s in w.specs for p in (s.parts or [s])]
        w = Workload(w.name, w.config, w.make_tensors, specs, w.steps, w.warmup,
                     (w.sample[0], w.sample[1], list(range(len(specs)))), w.per_call)
    steps = args.steps if args.steps is not None else w.steps
    warmup = args.warmup if args.warmup is not None else w.warmup

    import torch
    import microscaling_fp4_quantization_amd as fq

    dev = torch.device("cuda:0")
    xs, sample_host = [], []
    n_sample = w.sample[1]
    for x in w.make_tensors():
        if len(sample_host) < n_sample:
            sample_host.append(x)
        xs.append(x.to(dev))
        del x
    in_bytes = xs[0].element_size()
    n_calls = len(xs) * len(w.specs)
    streams = args.streams if args.streams is not None else (1 if n_calls == 1 else 2)
    batch = 0 if args.no_batch else (args.batch if args.batch is not None else w.batch)
    run = Runner(fq, torch, dev, xs, w.specs, max(1, streams), batch)
    n_elem_calls = sum(x.numel() for x in xs) * sum(s.formats for s in w.specs)
    alg_bytes = sum(s.algorithmic_bytes(x.numel(), in_bytes) for x in xs for s in w.specs)

    for _ in range(warmup):
        run.step()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        run.step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    ms_step = ev[0].elapsed_time(ev[steps]) / steps
    value = n_elem_calls * in_bytes / (ms_step * 1e-3) / 1e9

    # Dominant kernel: the step's own quantize launches (every call of a step,
    # replayed on one stream, each launch timed with events on that stream).
    lt = launch_times(fq, torch, run)
    q = lt["quantize"]
    q_us, q_bytes = sum(e[0] for e in q), sum(e[1] for e in q)
    achieved = q_bytes / (q_us * 1e-6) / 1e9
    per_spec = {}
    for tag in dict.fromkeys(e[2] for e in q):
        sel = [e for e in q if e[2] == tag]
        su, sb = sum(e[0] for e in sel), sum(e[1] for e in sel)
        by_shape = {}
        for e in sel:
            by_shape.setdefault(e[3], []).append(e)
        per_spec[tag] = {"launches": len(sel), "us_per_launch": round(su / len(sel), 3),
                           "GBps": round(sb / (su * 1e-6) / 1e9, 1),
                           "frac": round(sb / (su * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if len(by_shape) > 1:
            per_spec[tag]["by_shape"] = {
                shp: {"launches": len(v), "us_per_launch": round(sum(e[0] for e in v) / len(v), 3),
                      "frac": round(sum(e[1] for e in v) / (sum(e[0] for e in v) * 1e-6) / 1e9
                                    / HBM_PEAK_GBS, 4)}
                for shp, v in by_shape.items()}
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(args.workload) if args.workload in TRAFFIC else None,
                "kernel": "k_quantize: every quantize launch of one step (the step's calls replayed "
                          "on one stream, HIP events around each launch)",
                "us_per_launch": round(q_us / len(q), 3),
                "algorithmic_bytes_per_launch": int(q_bytes / len(q)),
                "launches": len(q), "per_spec": per_spec}
    if "amax" in lt:
        a = lt["amax"]
        a_us, a_bytes = sum(e[0] for e in a), sum(e[1] for e in a)
        roofline["s0_amax_pass"] = {
            "kernel": "k_amax (per-tensor amax for the dynamic scale: reads the input once)",
            "launches": len(a), "us_per_launch": round(a_us / len(a), 3),
            "GBps": round(a_bytes / (a_us * 1e-6) / 1e9, 1),
            "frac": round(a_bytes / (a_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    elif any(s.parts for s in w.specs):
        roofline["s0_amax_pass"] = {
            "kernel": "none: the MXFP4 quantize launch of each fp4_quantize_mx_nv call also takes "
                      "the tensor maximum (per-workgroup maxima, reduced to g by its stats reduction), "
                      "so the NVFP4 pass needs no amax read"}
    if "finalize" in lt:
        f = lt["finalize"]
        roofline["stats_reduction_us_per_launch"] = round(sum(e[0] for e in f) / len(f), 3)

    # Per-spec breakdown: one timed pass of each call type over all tensors.
    breakdown = {}
    if w.per_call:
        # Latency-bound calls: timed from a captured HIP graph (GPU time per call),
        # and back to back from Python (host launch cost included).
        for ti, x in enumerate(xs):
            for si, s in enumerate(w.specs):
                fn = lambda ti=ti, si=si: run.call(ti, si)
                us = time_graph(torch, fn)
                us_eager = time_region(torch, stream, fn, 200) * 1e3
                breakdown[f"{s.tag}_M{x.shape[0]}"] = {
                    "us_per_call_graph": round(us, 2),
                    "us_per_call_eager": round(us_eager, 2),
                    "algorithmic_GBps": round(s.algorithmic_bytes(x.numel(), in_bytes)
                                              / (us * 1e-6) / 1e9, 1)}
    elif len(w.specs) > 1:
        for si, s in enumerate(w.specs):
            fn = lambda si=si: [run.call(ti, si) for ti in range(len(xs))]
            ms = time_region(torch, stream, fn, max(1, min(steps, 10)))
            nb = sum(s.algorithmic_bytes(x.numel(), in_bytes) for x in xs)
            breakdown[s.tag] = {"us_per_call": round(ms * 1e3 / len(xs), 2),
                                **search_gain(fq, torch, run, si),
                                "input_GBps": round(sum(x.numel() for x in xs) * in_bytes
                                                    / (ms * 1e-3) / 1e9, 1),
                                "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1)}

    ceiling = copy_ceiling(torch, xs) if not w.per_call else None
    if args.calibration_copy:
        dst = torch.empty_like(xs[0])
        dst.copy_(xs[0])
        torch.cuda.synchronize()

    config = {"workload": w.name, **w.config, "elements_per_step": n_elem_calls,
              "calls": "; ".join(s.describe() for s in w.specs),
              "streams": max(1, streams),
              "arithmetic": "binary32 scales and codes, binary64 error sums, binary32 block sums of exact squares of x"}
    if args.workload == "qwen14model":
        config["layers"] = QWEN14_LAYERS_RUN or 48
    if run.batch:
        config["tensors_per_call"] = run.batch
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4),
        "ms_per_step_min": round(per_step[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if in_bytes == 4 else "bf16",
        "data": "synthetic (seeded numpy PCG64, " +
                ("fp32" if in_bytes == 4 else "rounded to bf16") + ")",
        "config": config,
        "roofline": roofline,
        "step_breakdown": {"algorithmic_GBps_all_kernels":
                           round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
                           "frac_all_kernels": round(alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "wall_s_timed_region": round(t_wall, 3), **breakdown},
    }
    if ceiling:
        line["copy_ceiling"] = ceiling
    if args.workload == "llama8":
        import fp4_workloads as wl
        line["three_term_model"] = three_term_table(fq, run, wl.LLAMA8_SIGMAS)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, sample_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
