"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses.  The library processes every whole tensor; the oracle checks a
sample of rows element by element (codes, scale bytes, per-block MSE) and the
tensor-level error terms over the whole tensor (computed on row slices in
parallel threads and summed; the per-tensor scale of the dynamic mode comes
from the oracle's amax of the whole tensor).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fp4_workloads as wl
import oracle
import microscaling_fp4_quantization_amd as fq
from parity_util import assert_stats, compare_quant, to_oracle_input

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
THREADS = 16


def sample_rows(rows: int, seed, k: int = 40) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(rows, size=min(k, rows), replace=False).tolist()) | {0, rows - 1}
    return np.array(sorted(pick))


def oracle_terms(xf: np.ndarray, fmt, block, g, rotate, kind):
    """Tensor terms of the whole tensor from the oracle, on row slices."""
    rows = xf.shape[0]
    cuts = np.linspace(0, rows, THREADS + 1).astype(int)
    gm = oracle.GMODE_GIVEN if fmt == oracle.FMT_UE4M3 else oracle.GMODE_NONE

    def run(i):
        r = oracle.quantize(xf[cuts[i]:cuts[i + 1]], fmt, block, gm, g, rotate, kind)
        return r["terms"], r["counts"]

    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(run, range(THREADS)))
    terms = np.zeros(4)
    counts = np.zeros(2, np.int64)
    for t, c in parts:
        terms += t
        counts += c
    return terms, counts


def check_workload(x: torch.Tensor, fmt, block, gmode, rotate, kind, seed, full_terms=True):
    print(f"  case shape={tuple(x.shape)} fmt={fmt} block={block} gmode={gmode} rot={rotate}",
          flush=True)
    if fmt == oracle.FMT_MXFP4:
        q = fq.mxfp4_quantize(x, rotate, mse_kind=kind)
    else:
        q = fq.nvfp4_quantize(x, block, fmt, gmode, None, rotate, mse_kind=kind)
    torch.cuda.synchronize()
    xf = to_oracle_input(x)
    g = 1.0
    if fmt == oracle.FMT_UE4M3 and gmode == oracle.GMODE_DYNAMIC:
        g = oracle.dynamic_g(oracle.tensor_amax(xf, rotate))
    rows = sample_rows(x.shape[0], seed)
    gm = oracle.GMODE_GIVEN if fmt == oracle.FMT_UE4M3 else oracle.GMODE_NONE
    ref = oracle.quantize(xf[rows], fmt, block, gm, g, rotate, kind)
    ref["g"] = g
    compare_quant(q, ref, rows=rows)
    if full_terms:
        terms, counts = oracle_terms(xf, fmt, block, g, rotate, kind)
        assert_stats(fq.stats_dict(q.stats), terms, counts)
    return q


def test_qwen05_up_fp32_mxfp4_full():
    """fp32 4864 x 896, N(0, 0.02), seed 0, MXFP4: whole tensor element by element."""
    xf = wl.qwen05_up()
    x = torch.from_numpy(xf).to(DEV)
    q = fq.mxfp4_quantize(x)
    ref = oracle.quantize(xf, oracle.FMT_MXFP4, 32)
    compare_quant(q, ref)


@pytest.mark.parametrize("shape_idx", [0, 1])
@pytest.mark.parametrize("sigma_idx", [0, 1, 2])
def test_qwen7_mlp_nvfp4_dynamic(shape_idx, sigma_idx):
    x = wl.qwen7_mlp(shape_idx, sigma_idx).to(DEV)
    check_workload(x, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC, 0, oracle.MSE_ABS,
                   [2, shape_idx, sigma_idx])


@pytest.mark.parametrize("sigma_idx", [0, 1, 2, 3])
def test_llama8_block_sweep(sigma_idx):
    x = wl.llama8_sweep(sigma_idx).to(DEV)
    for b in wl.LLAMA8_BLOCKS:
        check_workload(x, oracle.FMT_UE4M3, b, oracle.GMODE_NONE, 0, oracle.MSE_ABS, [3, b])
    check_workload(x, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC, 0, oracle.MSE_ABS, [3, 99],
                   full_terms=False)


@pytest.mark.parametrize("fmt,block,gmode", [(0, 32, 0), (1, 16, 1)])
@pytest.mark.parametrize("rotate", [False, True])
def test_qwen14_outliers_rotation(fmt, block, gmode, rotate):
    x = wl.qwen14_outliers().to(DEV)
    check_workload(x, fmt, block, gmode, block if rotate else 0, oracle.MSE_ABS, [4, fmt])


@pytest.mark.parametrize("layer", [0, 47])
def test_qwen14_model_layers(layer):
    for p_idx, (name, shape) in enumerate(wl.QWEN14_PROJ):
        x = wl.qwen14_layer_tensor(layer, p_idx).to(DEV)
        check_workload(x, oracle.FMT_MXFP4, 32, oracle.GMODE_NONE, 0, oracle.MSE_REL,
                       [5, layer, p_idx], full_terms=(layer == 0))
        check_workload(x, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC, 0, oracle.MSE_REL,
                       [5, layer, p_idx, 1], full_terms=(layer == 0))
        del x
