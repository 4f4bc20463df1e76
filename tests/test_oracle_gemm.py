"""Pins for the oracle's MXFP4 GEMM (reading R10: C = A_hat B_hat^T in binary64
from the exactly dequantized operands; "Bridging the Gap Between Promise and
Performance for Microscaling FP4 Quantization", Sommario tecnico section 3 item
4 and section 4, the FP4 GEMM consuming the packed codes and scales).

Checked against: numpy's matmul of the operands dequantized by the (pinned)
oracle dequantizer on inputs whose products and sums are exact in binary64,
a hand-worked 1 x 1 x 32 product, linearity in each operand's scale byte, and
the transpose identity C(A, B)^T = C(B, A).
"""
import numpy as np
import pytest


def random_mx(orc, rows, k, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * 2.0 ** rng.integers(-4, 4, (rows, 1))).astype(np.float32)
    q = orc.quantize(x, orc.FMT_MXFP4, 32)
    return q["codes"], q["scales"]


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (5, 7, 96), (33, 17, 256), (16, 48, 1024)])
def test_gemm_is_numpy_matmul_of_dequantized(orc, m, n, k):
    ac, asc = random_mx(orc, m, k, [51, m, k])
    bc, bsc = random_mx(orc, n, k, [52, n, k])
    a = orc.dequantize(ac, asc, orc.FMT_MXFP4, 32, 1.0, m, k).astype(np.float64)
    b = orc.dequantize(bc, bsc, orc.FMT_MXFP4, 32, 1.0, n, k).astype(np.float64)
    want = a @ b.T   # products of E2M1 x 2^E values: exact; sums of few terms of bounded span
    got = orc.gemm_mxfp4(ac, asc, bc, bsc, m, n, k)
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)


def test_hand_worked_product(orc):
    """A = [6, -0.5, 0 x 30] with scale byte 128 (x2), B = [1.5, 4, 0 x 30] with
    byte 126 (x1/2): C = 12 * 0.75 + (-1) * 2 = 7."""
    a = np.zeros(32, np.uint8)
    b = np.zeros(32, np.uint8)
    a[0], a[1] = 7, 8 | 1          # 6, -0.5
    b[0], b[1] = 3, 6              # 1.5, 4
    pack = lambda c: (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None, :]
    got = orc.gemm_mxfp4(pack(a), np.array([[128]], np.uint8), pack(b),
                         np.array([[126]], np.uint8), 1, 1, 32)
    assert got[0, 0] == 7.0


def test_scale_byte_linearity_and_transpose(orc):
    ac, asc = random_mx(orc, 9, 128, 53)
    bc, bsc = random_mx(orc, 11, 128, 54)
    base = orc.gemm_mxfp4(ac, asc, bc, bsc, 9, 11, 128)
    up = orc.gemm_mxfp4(ac, (asc + 1).astype(np.uint8), bc, bsc, 9, 11, 128)
    np.testing.assert_array_equal(up, base * 2)
    down = orc.gemm_mxfp4(ac, asc, bc, (bsc - 3).astype(np.uint8), 9, 11, 128)
    np.testing.assert_array_equal(down, base / 8)
    np.testing.assert_array_equal(orc.gemm_mxfp4(bc, bsc, ac, asc, 11, 9, 128), base.T)
