"""Benchmark of the FP4 quantization path on one MI355X.

Default workload (one step = the whole path over one batch):
  six bf16 Qwen2.5-7B MLP tensors, 18944 x 3584 and 3584 x 18944 with
  N(0, sigma), sigma in {0.01, 0.02, 0.04} (seeded), each quantized to NVFP4:
  the per-tensor amax pass, then block-16 UE4M3 scales under the dynamic FP32
  per-tensor scale, E2M1 codes packed two per byte, dequantization, per-block
  MSE and the three-term error split.  Inputs are resident in HBM before timing.

Prints one JSON line.  `value` is GB/s of bf16 input quantized+packed+MSE'd
over the whole step (all kernels of all six tensors).  `roofline` is the
quantize kernel alone (the step's own k_quantize instantiation, launched once
per tensor with the step's per-tensor scale given), timed with HIP events on
the stream it runs on; algorithmic bytes per element = 2 (read) + 0.5 (codes)
+ 1/16 (scales) + 4/16 (per-block MSE).  `cpu_baseline` times the oracle
(single thread) on two of the six tensors.

Other workloads for reference numbers: --workload qwen05 | llama8 | qwen14rot | qwen14model.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s of bf16 input quantized+packed+MSE'd (MXFP4/NVFP4); % of HBM peak"
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "microscaling_fp4_quantization_amd", "csrc", "fp4q_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_nvfp4_qwen7_traffic.json")


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def gen_qwen7():
    import fp4_workloads as wl
    xs = []
    for si in range(2):
        for gi in range(3):
            xs.append(wl.qwen7_mlp(si, gi))
    return xs


def cpu_baseline(xs_host):
    """The oracle as it stands (one thread) on two whole tensors of the workload."""
    import oracle
    n, el = 0, 0.0
    for x in xs_host[:2]:
        xf = x.float().numpy()
        t = time.perf_counter()
        oracle.quantize(xf, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC)
        el += time.perf_counter() - t
        n += xf.size
    return {"value": round(n * 2 / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "2 of the 6 tensors (18944x3584, sigma 0.01 and 0.02), whole, NVFP4 with "
                      "dynamic per-tensor scale, single-threaded C oracle",
            "seconds": round(el, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="qwen7")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain device copy of the first tensor (a kernel of "
                         "known traffic, for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by rows with one max- and one sum-all-reduce; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload != "qwen7":
        import bench_workloads
        bench_workloads.run(args)
        return

    import torch
    import microscaling_fp4_quantization_amd as fq

    dev = torch.device("cuda:0")
    xs_host = gen_qwen7()
    xs = [x.to(dev) for x in xs_host]
    outs = []
    for x in xs:
        r, c = x.shape
        outs.append(dict(codes=torch.empty((r, c // 2), dtype=torch.uint8, device=dev),
                         scales=torch.empty((r, c // 16), dtype=torch.uint8, device=dev),
                         block_mse=torch.empty((r, c // 16), dtype=torch.float32, device=dev),
                         stats=fq.new_stats(dev),
                         g=torch.empty(1, dtype=torch.float32, device=dev)))
    ws = fq.workspace(dev)
    n_elem = sum(x.numel() for x in xs)

    def step():
        for x, o in zip(xs, outs):
            fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_DYNAMIC, o["g"], 0, codes=o["codes"],
                              scales=o["scales"], block_mse=o["block_mse"], stats=o["stats"],
                              ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    value = n_elem * 2 / (ms_step * 1e-3) / 1e9

    # Dominant kernel alone.  With the per-tensor scale given (the g each step
    # computed), per-block MSE and no stats, a call launches exactly one kernel:
    # the same k_quantize instantiation the step runs (in the dynamic mode the
    # amax pass supplies sum x^2, so the step's quantize kernel omits it too).
    reps = max(10, args.steps)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def quantize_only():
        for x, o in zip(xs, outs):
            fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_GIVEN, o["g"], 0, codes=o["codes"],
                              scales=o["scales"], block_mse=o["block_mse"], stats=False)

    quantize_only()
    torch.cuda.synchronize()
    k0.record(stream)
    for _ in range(reps):
        quantize_only()
    k1.record(stream)
    torch.cuda.synchronize()
    us_launch = k0.elapsed_time(k1) * 1e3 / (reps * len(xs))
    bytes_launch = xs[0].numel() * (2 + 0.5 + 1 / 16 + 4 / 16)
    achieved = bytes_launch / (us_launch * 1e-6) / 1e9

    if args.calibration_copy:
        dst = torch.empty_like(xs[0])
        dst.copy_(xs[0])
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64 normal, rounded to bf16)",
        "config": {"workload": "qwen2.5-7b-mlp-nvfp4",
                   "tensors": "6 bf16: 18944x3584 and 3584x18944, sigma 0.01/0.02/0.04",
                   "format": "NVFP4: block 16, UE4M3 scales, dynamic FP32 per-tensor scale",
                   "outputs": "codes + scales + per-block MSE + three-term error split",
                   "elements_per_step": n_elem},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(),
                     "kernel": "k_quantize<bf16, UE, 16, no rotation, err, no sumsq>",
                     "us_per_launch": round(us_launch, 3),
                     "algorithmic_bytes_per_launch": int(bytes_launch)},
        "step_breakdown": {"algorithmic_GBps_both_passes":
                           round(n_elem * (2 + 2.8125) / (ms_step * 1e-3) / 1e9, 1)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(xs_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
