"""GPU parity at the workloads' full sizes, element by element, in the launch
configuration the benchmark uses.

The library processes each whole tensor; the oracle processes every row of it
too (on row slices in parallel threads, outputs concatenated and tensor terms
summed), and every code byte, scale byte and per-block MSE is compared, along
with the per-tensor scale and the four tensor terms.  The dynamic per-tensor
scale comes from the oracle's amax of the whole tensor.  Nothing is sampled.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fp4_workloads as wl
import oracle
from oracle import mse_model
import microscaling_fp4_quantization_amd as fq
from parity_util import compare_quant, to_oracle_input

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
THREADS = 16  # the host share of one GPU
POOL = ThreadPoolExecutor(THREADS)


def oracle_tensor(xf: np.ndarray, fmt, block, g, rotate, kind) -> dict:
    """oracle.quantize of the whole tensor under per-tensor scale g, computed on
    row slices in parallel."""
    rows = xf.shape[0]
    n = max(1, min(2 * THREADS, rows))
    cuts = np.linspace(0, rows, n + 1).astype(int)
    gm = oracle.GMODE_GIVEN if fmt == oracle.FMT_UE4M3 else oracle.GMODE_NONE

    def run(i):
        return oracle.quantize(xf[cuts[i]:cuts[i + 1]], fmt, block, gm, g, rotate, kind)

    parts = list(POOL.map(run, range(n)))
    return {"codes": np.concatenate([p["codes"] for p in parts]),
            "scales": np.concatenate([p["scales"] for p in parts]),
            "block_mse": np.concatenate([p["block_mse"] for p in parts]),
            "terms": np.sum([p["terms"] for p in parts], axis=0),
            "counts": np.sum([p["counts"] for p in parts], axis=0),
            "g": g}


def check_workload(x: torch.Tensor, fmt, block, gmode, rotate, kind):
    print(f"  case shape={tuple(x.shape)} fmt={fmt} block={block} gmode={gmode} rot={rotate} "
          f"kind={kind}", flush=True)
    if fmt == oracle.FMT_MXFP4:
        q = fq.mxfp4_quantize(x, rotate, mse_kind=kind)
    else:
        q = fq.nvfp4_quantize(x, block, fmt, gmode, None, rotate, mse_kind=kind)
    torch.cuda.synchronize()
    xf = to_oracle_input(x)
    g = 1.0
    if fmt == oracle.FMT_UE4M3 and gmode == oracle.GMODE_DYNAMIC:
        g = oracle.dynamic_g(oracle.tensor_amax(xf, rotate))
    ref = oracle_tensor(xf, fmt, block, g, rotate, kind)
    compare_quant(q, ref)
    return q, ref


def test_qwen05_up_fp32_mxfp4_full():
    """fp32 4864 x 896, N(0, 0.02), seed 0, MXFP4 (block 32, E8M0)."""
    xf = wl.qwen05_up()
    x = torch.from_numpy(xf).to(DEV)
    q = fq.mxfp4_quantize(x)
    ref = oracle.quantize(xf, oracle.FMT_MXFP4, 32)
    compare_quant(q, ref)


@pytest.mark.parametrize("shape_idx", [0, 1])
@pytest.mark.parametrize("sigma_idx", [0, 1, 2])
def test_qwen7_mlp_nvfp4_dynamic(shape_idx, sigma_idx):
    """bf16 18944 x 3584 and 3584 x 18944, N(0, sigma): NVFP4 (block 16, UE4M3,
    dynamic per-tensor scale)."""
    x = wl.qwen7_mlp(shape_idx, sigma_idx).to(DEV)
    check_workload(x, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC, 0, oracle.MSE_ABS)


@pytest.mark.parametrize("sigma_idx", [0, 1, 2, 3])
def test_llama8_block_sweep(sigma_idx):
    """bf16 14336 x 4096, narrow Normal: UE4M3 and UE5M3 scales without a
    per-tensor scale at block sizes 256 ... 8, plus UE4M3 under the dynamic
    per-tensor scale at block 16.  Besides parity with the oracle, the GPU's
    per-element total error agrees with the three-term model for N(0, sigma)
    ("Is finer better?", Framework Teorico) within 5 standard errors (from the
    spread of the per-block MSE) plus 3 %: the model takes continuous inputs,
    and the bf16 rounding of these narrow-Normal inputs shifts the UE4M3 totals
    by up to about 2 % (measured with the oracle at full size; UE5M3 and the
    widest sigma agree within 0.1 %, and the model matches fp32 inputs within 5
    standard errors in the oracle's own tests); and at
    sigma = 0.002 the total error at block 8 exceeds that at block 16 under
    UE4M3 but not under UE5M3 (Contributi Chiave item 3, Risultati)."""
    sigma = wl.LLAMA8_SIGMAS[sigma_idx]
    x = wl.llama8_sweep(sigma_idx).to(DEV)
    n = x.numel()
    totals = {}
    for b in wl.LLAMA8_BLOCKS:
        for fmt, name in ((oracle.FMT_UE4M3, "ue4m3"), (oracle.FMT_UE5M3, "ue5m3")):
            q, _ = check_workload(x, fmt, b, oracle.GMODE_NONE, 0, oracle.MSE_ABS)
            st = fq.stats_dict(q.stats)
            total = (st["sse_nonmax"] + st["sse_max"] + st["sse_zero"]) / n
            sse_blocks = q.block_mse.double().cpu().numpy().ravel() * b
            se = sse_blocks.std(ddof=1) / np.sqrt(sse_blocks.size) / b
            pred = mse_model.predict(sigma, b, name)["total"]
            assert abs(total - pred) <= 5 * se + 3e-2 * pred, (name, b, total, pred, se)
            totals[(name, b)] = total
    if sigma_idx == 0:
        assert totals[("ue4m3", 8)] > totals[("ue4m3", 16)]
        assert totals[("ue5m3", 8)] < totals[("ue5m3", 16)]
    check_workload(x, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC, 0, oracle.MSE_ABS)


@pytest.mark.parametrize("fmt,block,gmode", [(0, 32, 0), (1, 16, 1)])
@pytest.mark.parametrize("rotate", [False, True])
def test_qwen14_outliers_rotation(fmt, block, gmode, rotate):
    """bf16 13824 x 5120 Student-t(4) with outlier columns: MXFP4 and dynamic
    NVFP4, without and with the block Hadamard rotation."""
    x = wl.qwen14_outliers().to(DEV)
    check_workload(x, fmt, block, gmode, block if rotate else 0, oracle.MSE_ABS)


@pytest.mark.parametrize("layer", range(wl.QWEN14_LAYERS))
def test_qwen14_model_layer(layer):
    """One layer of the Qwen2.5-14B-shaped stack: all seven projections, each in
    MXFP4 and in dynamic NVFP4 with the relative per-block MSE."""
    hosts = list(POOL.map(lambda p: wl.qwen14_layer_tensor(layer, p), range(len(wl.QWEN14_PROJ))))
    for p_idx, xh in enumerate(hosts):
        print(f" layer {layer} {wl.QWEN14_PROJ[p_idx][0]}", flush=True)
        x = xh.to(DEV)
        check_workload(x, oracle.FMT_MXFP4, 32, oracle.GMODE_NONE, 0, oracle.MSE_REL)
        check_workload(x, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC, 0, oracle.MSE_REL)
        del x
