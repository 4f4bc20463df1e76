"""Pins for the oracle's tensor functions: rotation, packing, dequantization,
the three-term MSE split and the per-tensor scale.

Checked against: scipy's Sylvester Hadamard matrix, closed forms derived by
hand from the definitions, numpy re-computations of the error terms from first
principles, invariants (sign symmetry, power-of-two scaling, idempotence,
Parseval) and the numerically integrated three-term model of the error for
Normal weights ("Is finer better? Limits of micro-scaling formats in LLMs",
Framework Teorico).
"""
import math
import zlib
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.linalg

from oracle import mse_model

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def unpack(codes: np.ndarray) -> np.ndarray:
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def code_values(c: np.ndarray) -> np.ndarray:
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


# ----------------------------------------------------------------- rotation
@pytest.mark.parametrize("n", [16, 32])
def test_hadamard_matrix_is_sylvester_and_orthogonal(orc, n):
    eye = np.eye(n, dtype=np.float32)
    cols = orc.hadamard(eye, n)  # row i = transform of unit vector e_i
    c = np.float32(1.0 / math.sqrt(n))
    H = cols / c
    assert np.all(np.abs(H) == 1.0)  # the butterfly of a unit vector is exact
    Hi = H.astype(np.int64)
    np.testing.assert_array_equal(Hi @ Hi.T, n * np.eye(n, dtype=np.int64))
    np.testing.assert_array_equal(Hi, scipy.linalg.hadamard(n))


def test_hadamard_norm_constant(orc):
    getcontext().prec = 60
    exact = Decimal(2).sqrt() / Decimal(8)  # 2^-2.5
    want = np.float32(float(exact))          # double then single rounding: far from a tie
    got = orc.hadamard(np.eye(32, dtype=np.float32), 32)[0, 0]
    assert got.view(np.uint32) == want.view(np.uint32) == 0x3E3504F3
    assert orc.hadamard(np.eye(16, dtype=np.float32), 16)[0, 0] == 0.25


@pytest.mark.parametrize("n", [16, 32])
def test_hadamard_against_fp64_matrix_and_involution(orc, n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal((64, 4 * n)) * 0.3).astype(np.float32)
    y = orc.hadamard(x, n)
    Hn = scipy.linalg.hadamard(n) / math.sqrt(n)
    ref = (x.astype(np.float64).reshape(-1, n) @ Hn.T).reshape(x.shape)
    scale = np.abs(x).reshape(-1, n).max(1).repeat(n).reshape(x.shape) * math.sqrt(n)
    assert np.max(np.abs(y - ref) / scale) < 8 * 2.0 ** -24 * math.log2(n)
    # involution (up to binary32 rounding) and Parseval per block
    z = orc.hadamard(y, n)
    assert np.max(np.abs(z - x)) < 1e-5 * np.max(np.abs(x))
    nx = (x.astype(np.float64).reshape(-1, n) ** 2).sum(1)
    ny = (y.astype(np.float64).reshape(-1, n) ** 2).sum(1)
    np.testing.assert_allclose(ny, nx, rtol=1e-5)


# ------------------------------------------------------- hand-derived examples
def test_hand_example_mxfp4(orc):
    """Block of 32: x = [1.875, 0.3125, -0.0625, 0.4375, 0 x 28].  m = 1.875,
    floor(log2 m) = 0, E = -2 -> scale byte 127 - 2 = 0x7D.  y = x * 4 =
    [7.5, 1.25, -0.25, 1.75] -> 6 (saturated, code 7), tie -> 1.0 (code 2),
    tie -> -0 (code 8), tie -> 2.0 (code 4).  Bytes 0x27, 0x48.  Dequantized
    [1.5, 0.25, -0, 0.5]; max-element error 0.375^2 = 0.140625; non-max error
    0.0625^2 + 0.0625^2 + 0.0625^2 = 0.01171875; MSE = 0.15234375 / 32."""
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [1.875, 0.3125, -0.0625, 0.4375]
    r = orc.quantize(x, orc.FMT_MXFP4, 32)
    assert r["scales"][0, 0] == 0x7D
    assert list(r["codes"][0, :2]) == [0x27, 0x48] and not r["codes"][0, 2:].any()
    assert r["terms"][0] == 0.01171875 and r["terms"][1] == 0.140625 and r["terms"][2] == 0
    assert r["block_mse"][0, 0] == np.float32(0.0047607421875)
    xh = orc.dequantize(r["codes"], r["scales"], orc.FMT_MXFP4, 32, 1.0, 1, 32)
    assert list(xh[0, :4]) == [1.5, 0.25, 0.0, 0.5] and np.signbit(xh[0, 2])
    # requantizing the dequantized block reproduces the same bytes with zero error
    r2 = orc.quantize(xh, orc.FMT_MXFP4, 32)
    assert r2["scales"][0, 0] == 0x7D and list(r2["codes"][0, :2]) == [0x27, 0x48]
    assert r2["block_mse"][0, 0] == 0 and not r2["terms"][:3].any()


def test_hand_example_nvfp4(orc):
    """Block of 16, g = 1: x = [0.75, -0.3125, 0.0625, 0 x 13].  s = 0.75/6 =
    0.125 = 2^-3 -> UE4M3 byte (e = 4, j = 0) = 0x20, d = 0.125.  y = [6, -2.5,
    0.5] -> codes 7, 0xC (tie -> -2), 1.  Bytes 0xC7, 0x01.  Errors 0, 0.0625,
    0 -> non-max 0.00390625, MSE 0.00390625 / 16."""
    x = np.zeros((1, 16), np.float32)
    x[0, :3] = [0.75, -0.3125, 0.0625]
    r = orc.quantize(x, orc.FMT_UE4M3, 16)
    assert r["scales"][0, 0] == 0x20
    assert list(r["codes"][0, :2]) == [0xC7, 0x01]
    assert list(r["terms"][:3]) == [0.00390625, 0.0, 0.0]
    assert r["block_mse"][0, 0] == np.float32(0.000244140625)


def test_hand_example_zero_rounding_boundary(orc):
    """g = 1, x = [1.5 * 2^-8, -0.75 * 2^-8, 0 x 14]: s = m/6 = 2^-10 exactly, a
    tie between UE4M3 values 0 and 2^-9, resolved to the even code 0: every
    element rounds to zero (a zero-rounding block, the third error source), Z =
    (1.5^2 + 0.75^2) 2^-16.  One bf16 step up, m = 0.005889892578125, the scale
    is 2^-9 (byte 0x01), y = m / 2^-9 = 3.015625 -> 3 (code 5) and the block is
    no longer zero-rounded."""
    x = np.zeros((1, 16), np.float32)
    x[0, :2] = [1.5 * 2 ** -8, -0.75 * 2 ** -8]
    r = orc.quantize(x, orc.FMT_UE4M3, 16)
    assert r["scales"][0, 0] == 0 and list(r["codes"][0, :1]) == [0x80]
    assert r["counts"][1] == 1
    assert r["terms"][2] == (1.5 ** 2 + 0.75 ** 2) * 2.0 ** -16
    assert r["terms"][0] == 0 and r["terms"][1] == 0
    x[0, 0] = 0.005889892578125
    r = orc.quantize(x, orc.FMT_UE4M3, 16)
    assert r["scales"][0, 0] == 1 and (r["codes"][0, 0] & 0xF) == 5 and r["counts"][1] == 0
    assert r["terms"][1] == (0.005889892578125 - 3 * 2.0 ** -9) ** 2


# ---------------------------------------------------- error split, from scratch
def numpy_terms(x, xh, b, kind):
    """Error terms recomputed with numpy from x and x_hat (float64)."""
    xb = x.astype(np.float64).reshape(-1, b)
    hb = xh.astype(np.float64).reshape(-1, b)
    e2 = (xb - hb) ** 2
    sse = e2.sum(1)
    m = np.abs(xb).max(1)
    istar = np.argmax(np.abs(xb) == m[:, None], axis=1)  # first index attaining m
    zero = (m > 0) & np.all(hb == 0, axis=1)
    emax = e2[np.arange(len(sse)), istar]
    terms = np.array([np.sum(np.where(zero, 0, sse - emax)), np.sum(np.where(zero, 0, emax)),
                      np.sum(np.where(zero, sse, 0)), np.sum(xb ** 2)])
    s2 = (xb ** 2).sum(1)
    blk = (sse / b) if kind == 0 else np.where(s2 > 0, sse / np.where(s2 > 0, s2, 1), 0)
    return terms, blk.astype(np.float32), int(zero.sum())


CASES = [("mx", 0, 32, 0), ("mx_rot", 0, 32, 32), ("nv16", 1, 16, 0), ("nv16_rot", 1, 16, 16),
         ("ue4m3_8", 1, 8, 0), ("ue4m3_64", 1, 64, 0), ("ue4m3_256", 1, 256, 0),
         ("ue4m3_32_rot", 1, 32, 32), ("ue5m3_16", 2, 16, 0)]


@pytest.mark.parametrize("name,fmt,b,rot", CASES)
@pytest.mark.parametrize("kind", [0, 1])
def test_error_split_matches_numpy(orc, name, fmt, b, rot, kind):
    rng = np.random.default_rng([zlib.crc32(name.encode()), kind])
    x = (rng.standard_normal((96, 512)) * 0.004).astype(np.float32)
    x[5, :] = 0.0                                  # all-zero blocks
    x[7, :64] = np.float32(2.0 ** -12)             # many ties for the argmax
    x[9] *= 1e-3                                   # zero-rounding blocks (UE4M3, g = 1)
    gm = orc.GMODE_DYNAMIC if (fmt == 1 and b == 16) else orc.GMODE_NONE
    r = orc.quantize(x, fmt, b, gm, rotate=rot, mse_kind=kind)
    xr = orc.hadamard(x, rot) if rot else x
    xh_rot = orc.dequantize(r["codes"], r["scales"], fmt, b, r["g"], *x.shape, rotate=0)
    terms, blk, nz = numpy_terms(xr, xh_rot, b, kind)
    np.testing.assert_allclose(r["terms"], terms, rtol=1e-12, atol=0)
    np.testing.assert_array_equal(r["block_mse"].ravel(), blk)
    assert r["counts"][0] == x.size // b and r["counts"][1] == nz
    # the standalone error function on the stored codes gives the same numbers
    mse2, acc2, cnt2 = orc.block_mse(x, r["codes"], r["scales"], fmt, b, r["g"], rot, kind)
    np.testing.assert_array_equal(mse2, r["block_mse"])
    np.testing.assert_array_equal(acc2, r["terms"])
    np.testing.assert_array_equal(cnt2, r["counts"])


def test_blocks_run_along_rows(orc):
    """Blocks are 32 consecutive elements of one row: every E8M0 byte equals
    frexp's exponent of that row segment's absmax (floor(log2 m) - 2 + 127),
    computed in numpy, and quantizing the transpose gives other bytes."""
    rng = np.random.default_rng(90)
    x = (rng.standard_normal((64, 96)) * 2.0 ** rng.integers(-6, 7, (64, 96))).astype(np.float32)
    got = orc.quantize(x, orc.FMT_MXFP4, 32)["scales"]
    m = np.abs(x).reshape(64, 3, 32).max(axis=2)
    e = np.frexp(m)[1]
    want = np.where(m > 0, np.clip(e - 1 - 2 + 127, 0, 254), 0).astype(np.uint8)
    np.testing.assert_array_equal(got, want)
    xt = np.ascontiguousarray(x[:, :64].T)  # 64 x 64: same block count, other direction
    assert not np.array_equal(orc.quantize(xt, orc.FMT_MXFP4, 32)["scales"].T.reshape(-1),
                              got[:, :2].reshape(-1))


def test_mx_dequant_is_exact_power_of_two_product(orc):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    r = orc.quantize(x, orc.FMT_MXFP4, 32)
    xh = orc.dequantize(r["codes"], r["scales"], orc.FMT_MXFP4, 32, 1.0, *x.shape)
    E = r["scales"].astype(np.int64) - 127
    want = np.ldexp(code_values(unpack(r["codes"])), np.repeat(E, 32, axis=1)).astype(np.float32)
    np.testing.assert_array_equal(xh, want)


# ----------------------------------------------------------------- invariants
@pytest.mark.parametrize("fmt,b,gm,rot", [(0, 32, 0, 0), (1, 16, 1, 0), (1, 8, 0, 0),
                                          (0, 32, 0, 32), (1, 16, 1, 16)])
def test_sign_symmetry(orc, fmt, b, gm, rot):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    a = orc.quantize(x, fmt, b, gm, rotate=rot)
    c = orc.quantize(-x, fmt, b, gm, rotate=rot)
    np.testing.assert_array_equal(c["codes"], a["codes"] ^ 0x88)
    np.testing.assert_array_equal(c["scales"], a["scales"])
    np.testing.assert_array_equal(c["terms"], a["terms"])


@pytest.mark.parametrize("k", [-9, -1, 3, 17])
def test_power_of_two_scaling(orc, k):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    xs = (x * np.float32(2.0 ** k)).astype(np.float32)
    a = orc.quantize(x, orc.FMT_MXFP4, 32)
    c = orc.quantize(xs, orc.FMT_MXFP4, 32)
    np.testing.assert_array_equal(c["codes"], a["codes"])
    np.testing.assert_array_equal(c["scales"].astype(int), a["scales"].astype(int) + k)
    np.testing.assert_allclose(c["terms"], a["terms"] * 4.0 ** k, rtol=1e-15)
    # UE4M3 with the dynamic per-tensor scale: same codes and bytes, g scales
    a = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_DYNAMIC)
    c = orc.quantize(xs, orc.FMT_UE4M3, 16, orc.GMODE_DYNAMIC)
    np.testing.assert_array_equal(c["codes"], a["codes"])
    np.testing.assert_array_equal(c["scales"], a["scales"])
    assert c["g"] == a["g"] * 2.0 ** k


def test_idempotent_on_grid_mx(orc):
    rng = np.random.default_rng(10)
    v = GRID[rng.integers(0, 8, (64, 256))] * np.where(rng.random((64, 256)) < 0.5, -1, 1)
    v[:, ::32] = rng.choice([4.0, -6.0, 6.0], size=(64, 8))  # a max of 4 or 6 per block
    E = rng.integers(-20, 20, (64, 8))
    x = np.ldexp(v, np.repeat(E, 32, axis=1)).astype(np.float32)
    r = orc.quantize(x, orc.FMT_MXFP4, 32)
    np.testing.assert_array_equal(r["scales"].astype(int) - 127, E)
    np.testing.assert_array_equal(code_values(unpack(r["codes"])), v)
    assert not r["terms"][:3].any() and not r["block_mse"].any()


def test_idempotent_on_grid_nv_dynamic(orc):
    """g = 2^-12, one block whose scale is 448 (so amax = 2688 g), every other
    block holding a +-6: D, s, d and every quotient are exact."""
    rng = np.random.default_rng(12)
    g = 2.0 ** -12
    vals = np.array([orc.ue4m3_value(b) for b in range(1, 0x7F)])
    shat = rng.choice(vals, size=(32, 16))
    shat[0, 0] = 448.0
    v = GRID[rng.integers(0, 8, (32, 256))] * np.where(rng.random((32, 256)) < 0.5, -1, 1)
    v[:, ::16] = rng.choice([6.0, -6.0], size=(32, 16))
    x = (v * np.repeat(shat, 16, axis=1) * g).astype(np.float32)
    r = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_DYNAMIC)
    assert r["g"] == g
    np.testing.assert_array_equal(np.array([orc.ue4m3_value(b) for b in r["scales"].ravel()]),
                                  shat.ravel())
    np.testing.assert_array_equal(code_values(unpack(r["codes"])), v)
    assert not r["terms"][:3].any()


def test_dynamic_g_is_amax_over_2688(orc):
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((64, 512)) * 0.03).astype(np.float32)
    r = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_DYNAMIC)
    assert r["g"] == np.float32(np.float32(np.abs(x).max()) / np.float32(2688.0))
    rr = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_DYNAMIC, rotate=16)
    assert rr["g"] == np.float32(np.float32(np.abs(orc.hadamard(x, 16)).max()) / np.float32(2688.0))
    z = orc.quantize(np.zeros((4, 32), np.float32), orc.FMT_UE4M3, 16, orc.GMODE_DYNAMIC)
    assert z["g"] == 1.0 and not z["codes"].any() and z["counts"][1] == 0


# ------------------------------------------------- three-term model agreement
MODEL_CASES = [("mxfp4", 32, 0.02, None), ("ue4m3", 16, 0.005, None), ("ue4m3", 8, 0.002, None),
               ("ue4m3", 16, 0.002, None), ("ue4m3", 64, 0.002, None), ("ue4m3", 16, 0.05, None),
               ("ue5m3", 16, 0.002, None), ("ue4m3", 16, 0.02, "dynamic")]


@pytest.mark.parametrize("fmt,b,sigma,gm", MODEL_CASES)
def test_terms_match_three_term_model(orc, fmt, b, sigma, gm):
    """Empirical non-max / max / zero-rounding terms on i.i.d. N(0, sigma) fp32
    input agree with the integrated model within 5 standard errors."""
    code = {"mxfp4": 0, "ue4m3": 1, "ue5m3": 2}[fmt]
    rng = np.random.default_rng([31, b, int(sigma * 1e4)])
    n_chunks, rows, cols = 16, 256, 2048
    per = []
    g = 1.0
    for i in range(n_chunks):
        x = (rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma))
        if gm == "dynamic":
            r = orc.quantize(x, code, b, orc.GMODE_GIVEN, g=0.02 * 4.5 / 2688.0)
            g = r["g"]
        else:
            r = orc.quantize(x, code, b)
        per.append(np.concatenate([r["terms"][:3] / x.size, [r["counts"][1] / r["counts"][0]]]))
    per = np.array(per)
    mean, se = per.mean(0), per.std(0, ddof=1) / math.sqrt(n_chunks)
    pred = mse_model.predict(sigma, b, fmt, g=g)
    want = np.array([pred["nonmax"], pred["max"], pred["zero"], pred["p_zero_block"]])
    n_blocks = n_chunks * rows * cols // b
    expected_zero_blocks = pred["p_zero_block"] * n_blocks
    for k, name in enumerate(["nonmax", "max", "zero", "p_zero"]):
        tol = 5 * se[k] + 1e-4 * abs(want[k]) + 1e-30
        if k >= 2:  # zero-rounding is a counted event: allow its Poisson spread
            tol += abs(want[k]) * 5.0 / math.sqrt(max(expected_zero_blocks, 1e-12))
        assert abs(mean[k] - want[k]) <= tol, (name, mean[k], want[k], se[k])


@pytest.mark.parametrize("b", [8, 16, 32])
def test_zero_block_fraction_closed_form(orc, b):
    """UE4M3 with g = 1: a block rounds to zero iff m/6 <= 2^-10, so the
    zero-rounded fraction is F(6 * 2^-10)^b for i.i.d. N(0, sigma) values."""
    sigma = 0.003
    rng = np.random.default_rng([32, b])
    x = rng.standard_normal((512, 4096), dtype=np.float32) * np.float32(sigma)
    r = orc.quantize(x, orc.FMT_UE4M3, b)
    p = mse_model.p_zero_block_closed_form(sigma, b, 6 * 2.0 ** -10)
    n = r["counts"][0]
    frac = r["counts"][1] / n
    assert abs(frac - p) <= 5 * math.sqrt(p * (1 - p) / n) + 1e-6


def test_small_block_inversion_under_ue4m3(orc):
    """Narrow weights under UE4M3 without a per-tensor scale: the total MSE at
    block 8 exceeds that at block 16 (the inversion the page reports), and the
    model predicts it too."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((256, 4096), dtype=np.float32) * np.float32(0.002)
    t8 = orc.quantize(x, orc.FMT_UE4M3, 8)["terms"][:3].sum()
    t16 = orc.quantize(x, orc.FMT_UE4M3, 16)["terms"][:3].sum()
    assert t8 > t16
    assert mse_model.predict(0.002, 8)["total"] > mse_model.predict(0.002, 16)["total"]


def test_model_fixture_is_current():
    """The stored three-term model table the benchmark prints equals the model."""
    import json
    import os
    import sys
    golden = os.path.join(os.path.dirname(__file__), "golden")
    sys.path.insert(0, golden)
    import make_mse_model
    stored = json.load(open(os.path.join(golden, "mse_model_llama8.json")))["terms"]
    fresh = make_mse_model.table()
    assert stored.keys() == fresh.keys()
    for k in fresh:
        for t in fresh[k]:
            assert stored[k][t] == pytest.approx(fresh[k][t], rel=1e-12, abs=1e-300), (k, t)
