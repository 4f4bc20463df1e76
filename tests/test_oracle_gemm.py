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


# ---------------------------------------------------------------- NVFP4 (R11)

def random_nv(orc, rows, k, seed, g=None):
    """Oracle-quantized NVFP4 operand (block 16, UE4M3): the dynamic g, or the
    given one."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * 2.0 ** rng.integers(-3, 3, (rows, 1))).astype(np.float32)
    q = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_DYNAMIC if g is None else orc.GMODE_GIVEN,
                     None if g is None else g)
    return q["codes"], q["scales"], q["g"]


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (5, 7, 48), (9, 17, 256), (16, 24, 512)])
def test_nv_gemm_is_numpy_matmul_of_dequantized(orc, m, n, k):
    ac, asc, ga = random_nv(orc, m, k, [61, m, k])
    bc, bsc, gb = random_nv(orc, n, k, [62, n, k])
    a = orc.dequantize(ac, asc, orc.FMT_UE4M3, 16, ga, m, k).astype(np.float64)
    b = orc.dequantize(bc, bsc, orc.FMT_UE4M3, 16, gb, n, k).astype(np.float64)
    want = a @ b.T
    got = orc.gemm_nvfp4(ac, asc, ga, bc, bsc, gb, m, n, k)
    # numpy sums in its own order; every term is exact, the sums round in binary64
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)


def test_nv_hand_worked_product(orc):
    """A = [6, -0.5, 0 x 14], scale byte 0x40 (UE4M3 2.0), g = 1; B = [1.5, 4,
    0 x 14], byte 0x34 (1.5 * 2^-1 = 0.75), g = 2 (d = 1.5):
    C = (12)(2.25) + (-1)(6) = 21."""
    a = np.zeros(16, np.uint8)
    b = np.zeros(16, np.uint8)
    a[0], a[1] = 7, 8 | 1          # 6, -0.5
    b[0], b[1] = 3, 6              # 1.5, 4
    pack = lambda c: (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None, :]
    got = orc.gemm_nvfp4(pack(a), np.array([[0x40]], np.uint8), 1.0, pack(b),
                         np.array([[0x34]], np.uint8), 2.0, 1, 1, 16)
    assert got[0, 0] == 21.0


def test_nv_gemm_equals_mx_gemm_on_power_of_two_scales(orc):
    """UE4M3 bytes with a zero mantissa are powers of two (2^(e-7)); with g = 1
    and both 16-blocks of every 32-block on the same such byte, the NVFP4 and
    MXFP4 readings of the same codes are the same matrices, so their products
    agree exactly."""
    rng = np.random.default_rng(63)
    m, n, k = 6, 5, 128
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ea = rng.integers(-6, 8, (m, k // 32))     # 2^e within the UE4M3 normal range
    eb = rng.integers(-6, 8, (n, k // 32))
    ue = lambda e: ((e + 7) << 3).astype(np.uint8)   # exponent field e + 7, mantissa 0
    nv_a = np.repeat(ue(ea), 2, axis=1)
    nv_b = np.repeat(ue(eb), 2, axis=1)
    got = orc.gemm_nvfp4(ac, nv_a, 1.0, bc, nv_b, 1.0, m, n, k)
    want = orc.gemm_mxfp4(ac, (ea + 127).astype(np.uint8), bc, (eb + 127).astype(np.uint8), m, n, k)
    np.testing.assert_array_equal(got, want)


def test_nv_g_linearity_and_transpose(orc):
    ac, asc, _ = random_nv(orc, 7, 64, 64, g=0.25)
    bc, bsc, _ = random_nv(orc, 9, 64, 65, g=0.5)
    base = orc.gemm_nvfp4(ac, asc, 0.25, bc, bsc, 0.5, 7, 9, 64)
    # powers of two in g scale every d and x_hat exactly (no subnormals here)
    np.testing.assert_array_equal(orc.gemm_nvfp4(ac, asc, 1.0, bc, bsc, 0.5, 7, 9, 64), base * 4)
    np.testing.assert_array_equal(orc.gemm_nvfp4(ac, asc, 0.25, bc, bsc, 0.0625, 7, 9, 64), base / 8)
    np.testing.assert_array_equal(orc.gemm_nvfp4(bc, bsc, 0.5, ac, asc, 0.25, 9, 7, 64), base.T)


def test_nv_gemm_rejects_ragged_k(orc):
    z = np.zeros((1, 4), np.uint8)
    with pytest.raises(orc.OracleError):
        orc.gemm_nvfp4(z, np.zeros((1, 1), np.uint8), 1.0, z, np.zeros((1, 1), np.uint8), 1.0, 1, 1, 8)
