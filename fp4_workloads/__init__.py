"""Seeded synthetic inputs for the FP4 quantization path.

The only module that both the product tests/benchmark and the oracle-side tests
use.  It draws random numbers and converts dtypes; it holds none of the
quantization arithmetic.

Workloads (shapes from the layers the pages study; values synthetic):

* ``qwen05_up``: one fp32 4864 x 896 matrix (Qwen2.5-0.5B MLP up-projection
  shape), N(0, 0.02), numpy PCG64 seed 0.  MXFP4 block 32.
* ``qwen7_mlp``: bf16 18944 x 3584 and 3584 x 18944 (Qwen2.5-7B MLP up/down
  shapes), N(0, sigma) for sigma in {0.01, 0.02, 0.04}: six tensors, seed
  [2, shape index, sigma index].  NVFP4 block 16 with a dynamic per-tensor scale.
* ``llama8_sweep``: bf16 14336 x 4096 (Llama-3.1-8B MLP shape), narrow Normal
  sigma in {0.002, 0.005, 0.01, 0.05}, seed [3, sigma index].  UE4M3 block
  sizes 256 ... 8.
* ``qwen14_outliers``: bf16 13824 x 5120 (Qwen2.5-14B MLP shape), Student-t
  with 4 degrees of freedom scaled to standard deviation 0.02 (the t(4)
  variance is 2), with 51 of the 5120 input columns (1 %, chosen by the seeded
  generator) multiplied by 20.  Seed [4].
* ``activations_5120``: bf16 activation matrices of M tokens x 5120 (the
  Qwen2.5-14B hidden size) for M in {1, 16, 128, 2048, 8192}: Student-t(4)
  times 0.5, each token scaled by 2^k with k uniform in [-8, 8), and 1 % of the
  channels (chosen by the generator) x16.  Seed [6, M].
* ``qwen14_model``: a random-init Qwen2.5-14B-shaped layer stack, 48 layers x
  {q 5120x5120, k 1024x5120, v 1024x5120, o 5120x5120, gate 13824x5120,
  up 13824x5120, down 5120x13824}, bf16 N(0, 0.02), seed [5, layer, proj].

Generation recipe: ``numpy.random.default_rng(seed).standard_normal(shape,
dtype=float32) * float32(sigma)``, then round-to-nearest-even to bfloat16 with
torch (the fp32 workload stays fp32).
"""
from __future__ import annotations

import numpy as np

QWEN05_UP = (4864, 896)
QWEN7_SHAPES = ((18944, 3584), (3584, 18944))
QWEN7_SIGMAS = (0.01, 0.02, 0.04)
LLAMA8_SHAPE = (14336, 4096)
LLAMA8_SIGMAS = (0.002, 0.005, 0.01, 0.05)
LLAMA8_BLOCKS = (256, 128, 64, 32, 16, 8)
QWEN14_SHAPE = (13824, 5120)
QWEN14_OUTLIER_COLS = 51
QWEN14_OUTLIER_GAIN = 20.0
QWEN14_LAYERS = 48
QWEN14_PROJ = (("q", (5120, 5120)), ("k", (1024, 5120)), ("v", (1024, 5120)),
               ("o", (5120, 5120)), ("gate", (13824, 5120)), ("up", (13824, 5120)),
               ("down", (5120, 13824)))


def normal_f32(shape, sigma: float, seed) -> np.ndarray:
    """N(0, sigma) in float32 from a PCG64 stream."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(sigma)
    return a


def student_t_outliers_f32(shape, sigma: float, n_outlier_cols: int, gain: float,
                           seed) -> np.ndarray:
    """Student-t(4) scaled to standard deviation sigma, with a seeded choice of
    input columns (axis 1) multiplied by ``gain``."""
    rng = np.random.default_rng(seed)
    cols = rng.choice(shape[1], size=n_outlier_cols, replace=False)
    a = (rng.standard_t(4, size=shape) * (sigma / np.sqrt(2.0))).astype(np.float32)
    a[:, cols] *= np.float32(gain)
    return a


def to_bf16(a: np.ndarray):
    """Round a float32 array to a torch bfloat16 tensor (nearest, ties to even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)


def bf16_to_f32(t) -> np.ndarray:
    """Exact widening of a torch bfloat16 tensor to a float32 numpy array."""
    import torch
    return t.to(torch.float32).numpy()


# ----------------------------------------------------------------- workloads
def qwen05_up():
    """The fp32 workload: returns a float32 numpy array."""
    return normal_f32(QWEN05_UP, 0.02, 0)


def qwen7_mlp(shape_idx: int, sigma_idx: int, shape=None):
    """One of the six bf16 tensors; ``shape`` overrides the size (parity runs)."""
    shp = QWEN7_SHAPES[shape_idx] if shape is None else shape
    return to_bf16(normal_f32(shp, QWEN7_SIGMAS[sigma_idx], [2, shape_idx, sigma_idx]))


def llama8_sweep(sigma_idx: int, shape=None):
    shp = LLAMA8_SHAPE if shape is None else shape
    return to_bf16(normal_f32(shp, LLAMA8_SIGMAS[sigma_idx], [3, sigma_idx]))


def qwen14_outliers(shape=None):
    shp = QWEN14_SHAPE if shape is None else shape
    n_out = QWEN14_OUTLIER_COLS if shape is None else max(1, round(0.01 * shp[1]))
    return to_bf16(student_t_outliers_f32(shp, 0.02, n_out, QWEN14_OUTLIER_GAIN, [4]))


def qwen14_layer_tensor(layer: int, proj_idx: int, shape=None):
    shp = QWEN14_PROJ[proj_idx][1] if shape is None else shape
    return to_bf16(normal_f32(shp, 0.02, [5, layer, proj_idx]))


ACT_TOKENS = (1, 16, 128, 2048, 8192)
ACT_HIDDEN = 5120


def activations_f32(rows: int, cols: int, seed) -> np.ndarray:
    """Student-t(4) x 0.5 with a per-token power-of-two magnitude and 1 % outlier
    channels x16."""
    rng = np.random.default_rng(seed)
    a = (rng.standard_t(4, (rows, cols)) * 0.5).astype(np.float32)
    a *= (2.0 ** rng.integers(-8, 8, (rows, 1))).astype(np.float32)
    a[:, rng.choice(cols, max(1, cols // 100), replace=False)] *= np.float32(16.0)
    return a


def activations_5120(tokens: int):
    return to_bf16(activations_f32(tokens, ACT_HIDDEN, [6, tokens]))


def qwen14_param_count() -> int:
    return QWEN14_LAYERS * sum(r * c for _, (r, c) in QWEN14_PROJ)
