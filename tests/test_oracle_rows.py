"""Pins for the oracle's per-row dynamic scale (reading R9: each row, one token
of an activation matrix, quantized under its own g_r = RN32(amax_r / 2688)).
The pages leave the granularity of the activation scale open ("Bridging the
Gap Between Promise and Performance for Microscaling FP4 Quantization",
Sommario tecnico section 3 item 4: rotation fused with quantization and scale
computation for activations).

Checked against: the already pinned per-tensor dynamic mode applied to each
row alone, g_r recomputed in numpy binary32, row permutation, power-of-two
scaling of a single row, and an all-zero row.
"""
import numpy as np
import pytest


def tokens(rows, cols, seed):
    rng = np.random.default_rng(seed)
    a = (rng.standard_t(4, (rows, cols)) * 0.5).astype(np.float32)
    a *= (2.0 ** rng.integers(-6, 6, (rows, 1))).astype(np.float32)  # per-token magnitude spread
    return a


@pytest.mark.parametrize("block,rotate", [(16, 0), (16, 16), (32, 32), (64, 0), (8, 0)])
def test_each_row_is_the_dynamic_mode_on_that_row(orc, block, rotate):
    x = tokens(12, 640, [71, block, rotate])
    q = orc.quantize(x, orc.FMT_UE4M3, block, orc.GMODE_ROW, None, rotate, orc.MSE_REL)
    terms = np.zeros(4)
    for r in range(x.shape[0]):
        ref = orc.quantize(x[r:r + 1], orc.FMT_UE4M3, block, orc.GMODE_DYNAMIC, None, rotate,
                           orc.MSE_REL)
        assert np.float32(q["g"][r]) == np.float32(ref["g"]), r
        np.testing.assert_array_equal(q["codes"][r], ref["codes"][0])
        np.testing.assert_array_equal(q["scales"][r], ref["scales"][0])
        np.testing.assert_array_equal(q["block_mse"][r], ref["block_mse"][0])
        terms += ref["terms"]
    np.testing.assert_allclose(q["terms"], terms, rtol=1e-13)
    assert q["counts"][0] == x.size // block


def test_row_scale_in_numpy():
    """g_r = RN32(max|x_r| / 2688) without rotation, 1 for an all-zero row."""
    import oracle as orc
    x = tokens(9, 256, 72)
    x[4] = 0.0
    q = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_ROW)
    want = np.abs(x).max(axis=1).astype(np.float32) / np.float32(2688.0)
    want[4] = 1.0
    np.testing.assert_array_equal(q["g"].view(np.uint32), want.astype(np.float32).view(np.uint32))
    assert np.all(q["scales"][4] == 0) and np.all(q["codes"][4] == 0)


def test_rows_are_independent_under_permutation(orc):
    x = tokens(10, 512, 73)
    perm = np.random.default_rng(74).permutation(10)
    a = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_ROW)
    b = orc.quantize(x[perm], orc.FMT_UE4M3, 16, orc.GMODE_ROW)
    np.testing.assert_array_equal(b["g"], a["g"][perm])
    np.testing.assert_array_equal(b["codes"], a["codes"][perm])
    np.testing.assert_array_equal(b["scales"], a["scales"][perm])
    np.testing.assert_array_equal(b["block_mse"], a["block_mse"][perm])


def test_power_of_two_on_one_row(orc):
    """Scaling row 3 by 2^t multiplies g_3 by 2^t exactly and leaves its codes and
    scale bytes (and every other row) unchanged."""
    x = tokens(6, 512, 75)
    a = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_ROW)
    for t in (-7, 9):
        y = x.copy()
        y[3] *= np.float32(2.0 ** t)
        b = orc.quantize(y, orc.FMT_UE4M3, 16, orc.GMODE_ROW)
        assert b["g"][3] == np.float32(a["g"][3] * 2.0 ** t)
        np.testing.assert_array_equal(b["codes"], a["codes"])
        np.testing.assert_array_equal(b["scales"], a["scales"])
        np.testing.assert_array_equal(np.delete(b["g"], 3), np.delete(a["g"], 3))
