"""Dense binary32 sweeps through every rounding decision of the fp32 input path,
GPU against the oracle, bit for bit.

The bf16 path is covered exhaustively elsewhere (every bf16 value); here the
inputs are binary32 values within +-1024 ulps of each decision boundary:
  - E2M1 element codes under MXFP4 block exponents from the subnormal regime
    (E = -127, whose grid midpoints are binary32 subnormals) to E = 125: every
    midpoint t * 2^E, t in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}, both signs.
    ("Diagnosing FP4 inference", technical summary section 2: E2M1 elements
    under a shared exponent; the tie and saturation rules are the library's.)
  - UE4M3 scale bytes: with g = RN32(1/6), D = RN32(6 g) is exactly 1, so the
    scale quotient is the block maximum itself, swept across every midpoint
    between consecutive UE4M3 values and past the top value ("Is finer better?",
    Framework Teorico: unsigned E4M3 block scales).
  - UE5M3 scale bytes (g = 1, D = 6): block maxima RN32(6 s) for s swept across
    every midpoint between consecutive UE5M3 values (Contributi Chiave item 3).
"""
import numpy as np
import pytest
import torch

import oracle
import microscaling_fp4_quantization_amd as fq
from parity_util import compare_quant

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ULPS = 1024
E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def ulp_sweep(center: float, k: int = ULPS) -> np.ndarray:
    """The binary32 values within k ulps of positive `center` (center included)."""
    bits = np.array([center], np.float32).view(np.int32)[0]
    return (bits + np.arange(-k, k + 1, dtype=np.int32)).view(np.float32)


def rows_of_blocks(blocks: np.ndarray, per_row: int) -> np.ndarray:
    """Blocks (n x b) laid out per_row to a row, the last row padded with zeros."""
    n, b = blocks.shape
    pad = (-n) % per_row
    if pad:
        blocks = np.concatenate([blocks, np.zeros((pad, b), np.float32)])
    return np.ascontiguousarray(blocks.reshape(-1, per_row * b))


@pytest.mark.parametrize("E", [-127, -120, -3, 0, 5, 60, 125])
def test_mxfp4_fp32_e2m1_midpoints(E):
    """Every E2M1 midpoint under block exponent E, +-1024 ulps, both signs; each
    block's first element is 7 * 2^E, which fixes the exponent at E."""
    scale = np.float32(2.0) ** E if E > -127 else np.float32(2.0 ** -127)
    vals = np.concatenate([ulp_sweep(float(np.float32(t) * scale)) for t in E2M1_MIDPOINTS])
    vals = np.concatenate([vals, -vals])
    n_blocks = -(-vals.size // 31)
    body = np.zeros(n_blocks * 31, np.float32)
    body[:vals.size] = vals
    pin = np.float32(7.0) * scale
    blocks = np.concatenate([np.full((n_blocks, 1), pin, np.float32), body.reshape(n_blocks, 31)], axis=1)
    x = rows_of_blocks(blocks, 32)
    q = fq.mxfp4_quantize(torch.from_numpy(x).to(DEV))
    ref = oracle.quantize(x, oracle.FMT_MXFP4, 32)
    assert np.all(ref["scales"][:, 0] == E + 127)
    compare_quant(q, ref, xin=x)


def _ue_values(fmt: int) -> np.ndarray:
    if fmt == oracle.FMT_UE4M3:
        return np.array([oracle.ue4m3_value(c) for c in range(0x7F)])
    return np.array([oracle.ue5m3_value(c) for c in range(0xF8)])


def test_ue4m3_fp32_scale_midpoints():
    """Block maxima swept across every UE4M3 midpoint (and past 448) with D = 1."""
    g = np.float32(1.0) / np.float32(6.0)
    assert np.float32(6.0) * g == np.float32(1.0)
    v = _ue_values(oracle.FMT_UE4M3)
    mids = list((v[:-1] + v[1:]) / 2) + [448.0, 464.0, 500.0]
    m = np.concatenate([ulp_sweep(float(t)) for t in mids])
    blocks = np.zeros((m.size, 16), np.float32)
    blocks[:, 0] = m
    blocks[:, 5] = -m * np.float32(0.3)  # a second element, coded under the same scale
    x = rows_of_blocks(blocks, 64)
    gt = torch.tensor([float(g)], dtype=torch.float32, device=DEV)
    q = fq.nvfp4_quantize(torch.from_numpy(x).to(DEV), 16, fq.FMT_UE4M3, fq.G_GIVEN, gt)
    ref = oracle.quantize(x, oracle.FMT_UE4M3, 16, oracle.GMODE_GIVEN, float(g))
    compare_quant(q, ref, xin=x)


def test_ue5m3_fp32_scale_midpoints():
    """Block maxima RN32(6 s) for s swept across every UE5M3 midpoint (g = 1)."""
    v = _ue_values(oracle.FMT_UE5M3)
    mids = list((v[:-1] + v[1:]) / 2) + [61440.0, 63488.0]
    s = np.concatenate([ulp_sweep(float(t), 256) for t in mids])
    m = (np.float32(6.0) * s).astype(np.float32)
    blocks = np.zeros((m.size, 16), np.float32)
    blocks[:, 0] = m
    blocks[:, 9] = m * np.float32(0.55)
    x = rows_of_blocks(blocks, 64)
    q = fq.nvfp4_quantize(torch.from_numpy(x).to(DEV), 16, fq.FMT_UE5M3, fq.G_NONE)
    ref = oracle.quantize(x, oracle.FMT_UE5M3, 16)
    compare_quant(q, ref, xin=x)
