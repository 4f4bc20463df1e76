"""GPU parity of the per-row dynamic scale mode (FP4Q_G_ROW: one UE4M3 scale
per token row of an activation matrix) against the oracle, element by element:
token counts from 1 up, rows ending in a partial chunk, every block size,
rotation, both dtypes, relative MSE, the tensor terms, the empty cases and the
largest token shape on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import microscaling_fp4_quantization_amd as fq
from parity_util import assert_block_mse, assert_stats, to_oracle_input

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def activations(rows, cols, seed, dtype):
    """Student-t(4) activations with a per-token magnitude spread and a few
    outlier channels (x16), as activation matrices have."""
    rng = np.random.default_rng(seed)
    a = (rng.standard_t(4, (rows, cols)) * 0.5).astype(np.float32)
    a *= (2.0 ** rng.integers(-8, 8, (rows, 1))).astype(np.float32)
    a[:, rng.choice(cols, max(1, cols // 100), replace=False)] *= 16.0
    return torch.from_numpy(a).to(dtype).to(DEV)


def check(q, ref, rows=None):
    codes, scales = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    g = q.g.cpu().numpy()
    if rows is not None:
        codes, scales, g = codes[rows], scales[rows], g[rows]
    np.testing.assert_array_equal(g.view(np.uint32), ref["g"].view(np.uint32), err_msg="g per row")
    np.testing.assert_array_equal(scales, ref["scales"], err_msg="scale bytes")
    np.testing.assert_array_equal(codes, ref["codes"], err_msg="codes")
    if q.block_mse is not None:
        bm = q.block_mse.cpu().numpy()
        assert_block_mse(bm if rows is None else bm[rows], ref["block_mse"])
    if q.stats is not None and rows is None:
        assert_stats(fq.stats_dict(q.stats), ref["terms"], ref["counts"])


@pytest.mark.parametrize("rows,cols", [(1, 5120), (16, 5120), (128, 5120), (7, 896), (33, 2560)])
@pytest.mark.parametrize("block,rotate", [(16, 16), (16, 0), (32, 32)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rows_parity(rows, cols, block, rotate, dtype):
    x = activations(rows, cols, [91, rows, cols, block, rotate], dtype)
    q = fq.nvfp4_quantize(x, block, fq.FMT_UE4M3, fq.G_ROW, None, rotate)
    ref = oracle.quantize(to_oracle_input(x), oracle.FMT_UE4M3, block, oracle.GMODE_ROW, None,
                          rotate)
    check(q, ref)


@pytest.mark.parametrize("block", [8, 64, 128, 256])
def test_rows_other_blocks_relative_mse(block):
    x = activations(24, 2048, [92, block], torch.bfloat16)
    q = fq.nvfp4_quantize(x, block, fq.FMT_UE4M3, fq.G_ROW, None, 0, mse_kind=fq.MSE_REL)
    ref = oracle.quantize(to_oracle_input(x), oracle.FMT_UE4M3, block, oracle.GMODE_ROW, None, 0,
                          oracle.MSE_REL)
    check(q, ref)


def test_rows_codes_only_and_zero_rows():
    x = activations(40, 1024, 93, torch.bfloat16)
    x[5] = 0.0
    x[17] = -0.0
    q = fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_ROW, None, 0, block_mse=False, stats=False)
    ref = oracle.quantize(to_oracle_input(x), oracle.FMT_UE4M3, 16, oracle.GMODE_ROW)
    q.block_mse = None
    check(q, ref)
    assert q.g[5].item() == 1.0 and q.g[17].item() == 1.0


def test_rows_empty():
    g = torch.full((6,), 7.0, device=DEV)
    x = torch.empty((6, 0), dtype=torch.bfloat16, device=DEV)
    q = fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_ROW, g, 0)
    assert torch.all(g == 1.0)
    st = fq.stats_dict(q.stats)
    assert st["n_blocks"] == 0 and st["sse_nonmax"] == 0.0
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_ROW, torch.empty(0, device=DEV), 0)


def test_rows_largest_token_shape_sampled():
    """8192 x 5120 bf16 with rotation 16: sampled rows element by element, the
    tensor terms over every row."""
    x = activations(8192, 5120, 94, torch.bfloat16)
    print("  case rows 8192x5120 rot16", flush=True)
    q = fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_ROW, None, 16)
    xf = to_oracle_input(x)
    rows = np.array(sorted(set(np.random.default_rng(95).choice(8192, 48, replace=False).tolist())
                           | {0, 8191}))
    ref = oracle.quantize(xf[rows], oracle.FMT_UE4M3, 16, oracle.GMODE_ROW, None, 16)
    check(q, ref, rows=rows)
    full = oracle.quantize(xf, oracle.FMT_UE4M3, 16, oracle.GMODE_ROW, None, 16)
    assert_stats(fq.stats_dict(q.stats), full["terms"], full["counts"])
    np.testing.assert_array_equal(q.g.cpu().numpy().view(np.uint32), full["g"].view(np.uint32))
