"""Benchmark of the FP4 quantization path on one MI355X.

Default workload (one step = the whole path over one batch):
  six bf16 Qwen2.5-7B MLP tensors, 18944 x 3584 and 3584 x 18944 with
  N(0, sigma), sigma in {0.01, 0.02, 0.04} (seeded), each quantized to NVFP4:
  the per-tensor amax pass, then block-16 UE4M3 scales under the dynamic FP32
  per-tensor scale, E2M1 codes packed two per byte, dequantization, per-block
  MSE and the three-term error split.  Inputs are resident in HBM before timing.
  The step spreads its independent per-tensor calls over two HIP streams (one
  workspace each; --streams 1 runs them back to back on one stream).

Prints one JSON line.  `value` is GB/s of input quantized+packed+MSE'd over
the whole step (all kernels of all tensors).  For the default workload
`roofline` is the quantize kernel alone (the step's own k_quantize
instantiation, launched once per tensor with the step's per-tensor scale
given), timed with HIP events on the stream it runs on; algorithmic bytes per
element = 2 (read) + 0.5 (codes) + 1/16 (scales) + 4/16 (per-block MSE).  For
the other workloads it is the whole step's algorithmic bytes (every kernel,
the amax pre-pass read included) over the step time.  `cpu_baseline` times the
oracle (single thread) on a bounded sample of the same workload.

Workloads (--workload):
  qwen7        the default above
  qwen05       fp32 4864 x 896 (Qwen2.5-0.5B up-projection), MXFP4 with per-block
               MSE: launch-bound, reported in GB/s only
  llama8       four bf16 14336 x 4096 tensors (Llama-3.1-8B MLP), narrow Normal
               sigma in {0.002, 0.005, 0.01, 0.05}, UE4M3 without a per-tensor
               scale at block sizes 256, 128, 64, 32, 16 and 8, MSE and split
  qwen14rot    bf16 13824 x 5120 Student-t(4) with 1 % outlier columns x20:
               MXFP4 and dynamic NVFP4, each without and with block rotation
  act5120      activation matrices of 1, 16, 128, 2048 and 8192 tokens x 5120:
               NVFP4 + rotation with per-token scales, NVFP4 with the per-tensor
               dynamic scale, MXFP4 + rotation; time per call for each
  qwen7search  the six default tensors, MXFP4 and dynamic NVFP4 with the per-block
               scale search (radius 1)
  qwen14model  a random-init Qwen2.5-14B-shaped stack (48 layers x 7 projections,
               13.2e9 bf16 parameters, 26.4 GB) quantized whole to MXFP4 and to
               dynamic NVFP4, relative per-block MSE and per-tensor split
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
def _traffic_plan(workload):
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


# ------------------------------------------------------------------ workloads
class Spec:
    """One quantization call applied to every tensor of a workload."""

    def __init__(self, tag, fmt, block, scale_fmt=1, gmode=0, rotate=0, mse_kind=0,
                 block_mse=True, stats=True, radius=None):
        self.tag, self.fmt, self.block, self.scale_fmt = tag, fmt, block, scale_fmt
        self.gmode, self.rotate, self.mse_kind = gmode, rotate, mse_kind
        self.block_mse, self.stats = block_mse, stats
        self.radius = radius  # per-block scale search radius, None for the plain call

    def algorithmic_bytes(self, n, in_bytes):
        """Bytes every kernel of the call must move: the amax pre-pass read (dynamic
        NVFP4), the quantize read, codes, scale bytes and per-block MSE."""
        b = n * (in_bytes + 0.5 + 1.0 / self.block + (4.0 / self.block if self.block_mse else 0))
        if self.fmt == "nv" and self.gmode == 1:
            b += n * in_bytes
        return b

    def describe(self):
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
    """`sample` = (description, tensors, repeats, spec index) of the oracle's
    bounded CPU sample.  `per_call` asks for a time per (tensor, spec) pair in
    the breakdown (latency-bound workloads)."""

    def __init__(self, name, config, make_tensors, specs, steps, warmup, sample, per_call=False):
        self.name, self.config, self.make_tensors = name, config, make_tensors
        self.specs, self.steps, self.warmup, self.sample = specs, steps, warmup, sample
        self.per_call = per_call


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


def _qwen14model_tensors():
    """Generated on host threads (one PCG64 stream per tensor, as the recipe says)
    and moved to the device one by one; yields host tensors lazily."""
    import fp4_workloads as wl
    keys = [(layer, p) for layer in range(wl.QWEN14_LAYERS) for p in range(len(wl.QWEN14_PROJ))]
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
         4, 1, 0)),
    "qwen05": Workload(
        "qwen2.5-0.5b-up-mxfp4-fp32",
        {"tensors": "1 fp32 4864x896, N(0, 0.02), seed 0",
         "format": "MXFP4: block 32, E8M0 scales", "outputs": "codes + scales + per-block MSE"},
        _qwen05_tensors, [Spec("mx32", "mx", 32, stats=False)], 400, 20,
        ("the tensor, whole, 40 times", 1, 40, 0)),
    "llama8": Workload(
        "llama3.1-8b-mlp-ue4m3-block-sweep",
        {"tensors": "4 bf16 14336x4096, sigma 0.002/0.005/0.01/0.05",
         "format": "UE4M3 scales, no per-tensor scale, blocks 256/128/64/32/16/8",
         "outputs": "codes + scales + per-block MSE + three-term error split"},
        _llama8_tensors, [Spec(f"ue4m3_b{b}", "nv", b, 1, 0) for b in (256, 128, 64, 32, 16, 8)],
        20, 2, ("2 of the 4 tensors (sigma 0.002 and 0.005), whole", 2, 1, 4)),
    "qwen14rot": Workload(
        "qwen2.5-14b-mlp-outliers-rotation",
        {"tensors": "1 bf16 13824x5120, Student-t(4) sd 0.02, 51 outlier columns x20",
         "format": "MXFP4 b32 and NVFP4 b16 dynamic g, each without and with block Hadamard",
         "outputs": "codes + scales + per-block MSE + three-term error split"},
        _qwen14rot_tensors,
        [Spec("mx32", "mx", 32), Spec("mx32_rot", "mx", 32, rotate=32),
         Spec("nv16_dyn", "nv", 16, 1, 1), Spec("nv16_dyn_rot", "nv", 16, 1, 1, rotate=16)],
        50, 5, ("the tensor, whole, 3 times", 1, 3, 2)),
    "qwen7search": Workload(
        "qwen2.5-7b-mlp-scale-search",
        {"tensors": "6 bf16: 18944x3584 and 3584x18944, sigma 0.01/0.02/0.04",
         "format": "MXFP4 b32 and NVFP4 b16 dynamic g, per-block scale search over the "
                   "max-based code and its neighbours (radius 1)",
         "outputs": "codes + scales + per-block MSE + three-term error split"},
        _qwen7_tensors,
        [Spec("mx32_search1", "mx", 32, radius=1), Spec("nv16_dyn_search1", "nv", 16, 1, 1, radius=1)],
        20, 2, ("1 of the 6 tensors (18944x3584, sigma 0.01), whole", 1, 1, 1)),
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
        50, 5, ("all five matrices, whole, 8 times", 5, 8, 0),
        per_call=True),
    "qwen14model": Workload(
        "qwen2.5-14b-shaped-model-sweep",
        {"tensors": "336 bf16 (48 layers x q,k,v,o,gate,up,down), N(0, 0.02), 13.2e9 params",
         "format": "MXFP4 b32 and NVFP4 b16 dynamic g",
         "outputs": "codes + scales + relative per-block MSE + per-tensor split"},
        _qwen14model_tensors,
        [Spec("mx32", "mx", 32, mse_kind=1), Spec("nv16_dyn", "nv", 16, 1, 1, mse_kind=1)],
        5, 1, ("layer 0's q, k, v, o, gate and up projections, whole", 6, 1, 1)),
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

    def __init__(self, fq, torch, dev, xs, specs, n_streams=1):
        self.fq, self.torch, self.dev, self.xs, self.specs = fq, torch, dev, xs, specs
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
        for ti, x in enumerate(xs):
            r, c = x.shape
            for si, s in enumerate(specs):
                key = (r, c, s.block, k % n_streams)
                k += 1
                if key not in shared:
                    shared[key] = dict(
                        codes=torch.empty((r, c // 2), dtype=torch.uint8, device=dev),
                        scales=torch.empty((r, c // s.block), dtype=torch.uint8, device=dev),
                        block_mse=torch.empty((r, c // s.block), dtype=torch.float32, device=dev))
                o = dict(shared[key])
                o["stats"] = fq.new_stats(dev)
                o["g"] = torch.ones(r if s.gmode == 3 else 1, dtype=torch.float32, device=dev)
                o["stream"] = key[3]
                self.out[(ti, si)] = o

    def call(self, ti, si, given=False, ws=None):
        fq, x, s, o = self.fq, self.xs[ti], self.specs[si], self.out[(ti, si)]
        ws = self.ws if ws is None else ws
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

    def step(self, given=False):
        """All calls of one step; with given=True each runs alone on the caller's
        stream (the roofline leg)."""
        if given or len(self.streams) == 1:
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


def cpu_baseline(w, xs_host_sample):
    """The oracle as it stands (one thread) on a bounded sample of the workload."""
    import numpy as np
    import oracle
    desc, n_tensors, repeat, spec_idx = w.sample
    s = w.specs[spec_idx]
    fmt = oracle.FMT_MXFP4 if s.fmt == "mx" else s.scale_fmt
    gmode = {0: oracle.GMODE_NONE, 1: oracle.GMODE_DYNAMIC, 2: oracle.GMODE_GIVEN,
             3: oracle.GMODE_ROW}[s.gmode]
    n, el, in_bytes = 0, 0.0, 2
    for x in xs_host_sample[:n_tensors]:
        xf = x.float().numpy() if hasattr(x, "float") else np.asarray(x, np.float32)
        in_bytes = 4 if (hasattr(x, "dtype") and str(x.dtype) == "torch.float32") else 2
        for _ in range(repeat):
            t = time.perf_counter()
            if s.radius is not None:
                oracle.quantize_search(xf, fmt, s.block, gmode, None, s.rotate, s.radius,
                                       s.mse_kind)
            else:
                oracle.quantize(xf, fmt, s.block, gmode, None, s.rotate, s.mse_kind)
            el += time.perf_counter() - t
            n += xf.size
    return {"value": round(n * in_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{desc}, {s.describe()}, single-threaded C oracle",
            "seconds": round(el, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="qwen7", choices=sorted(WORKLOADS) + ["gemm"])
    ap.add_argument("--streams", type=int, default=2,
                    help="HIP streams the step's independent calls are spread over")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain device copy of the first tensor (a kernel of "
                         "known traffic, for scaling rocprofv3 byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the workload's traffic record under profiles/ from two "
                         "rocprofv3 counter runs, then exit (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.workload, *args.write_traffic)
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
    w = WORKLOADS[args.workload]
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
    run = Runner(fq, torch, dev, xs, w.specs, max(1, args.streams))
    n_elem_calls = sum(x.numel() for x in xs) * len(w.specs)
    alg_bytes = sum(s.algorithmic_bytes(x.numel(), in_bytes) for x in xs for s in w.specs)

    for _ in range(warmup):
        run.step()
    stream = torch.cuda.current_stream(dev)
    t_wall = time.perf_counter()
    ms_step = time_region(torch, stream, run.step, steps)
    t_wall = time.perf_counter() - t_wall
    value = n_elem_calls * in_bytes / (ms_step * 1e-3) / 1e9

    if args.workload == "qwen7":
        # Dominant kernel alone.  With the per-tensor scale given (the g each step
        # computed), per-block MSE and no stats, a call launches exactly one
        # kernel: the same k_quantize instantiation the step runs (in the dynamic
        # mode the amax pass supplies sum x^2, so the step's quantize kernel omits
        # it too).  The step's launches also form the tensor terms and reduce the
        # amax partials, so they run on the one-round grid; these run on
        # short-lived workgroups, and skip the tensor-term arithmetic.
        reps = max(10, steps)
        run.step(given=True)
        us_launch = time_region(torch, stream, lambda: run.step(given=True), reps) * 1e3 / len(xs)
        bytes_launch = xs[0].numel() * (2 + 0.5 + 1 / 16 + 4 / 16)
        achieved = bytes_launch / (us_launch * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": read_traffic(),
                    "kernel": "k_quantize<bf16, UE, 16, no rotation, err, no sumsq>",
                    "us_per_launch": round(us_launch, 3),
                    "algorithmic_bytes_per_launch": int(bytes_launch)}
    else:
        achieved = alg_bytes / (ms_step * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": "whole step (every kernel of every call)",
                    "algorithmic_bytes_per_step": int(alg_bytes)}

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

    if args.calibration_copy:
        dst = torch.empty_like(xs[0])
        dst.copy_(xs[0])
        torch.cuda.synchronize()

    config = {"workload": w.name, **w.config, "elements_per_step": n_elem_calls,
              "streams": max(1, args.streams)}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64, " +
                ("fp32" if in_bytes == 4 else "rounded to bf16") + ")",
        "config": config,
        "roofline": roofline,
        "step_breakdown": {"algorithmic_GBps_all_kernels":
                           round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
                           "wall_s_timed_region": round(t_wall, 3), **breakdown},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, sample_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
