"""Pins for the oracle's per-block scale search (reading R8: the max-based scale
code and its neighbours within a radius, scored by block SSE; "Bridging the Gap
Between Promise and Performance for Microscaling FP4 Quantization", Sommario
tecnico section 3 item 2, MSE-optimised scales).

Checked against: the already pinned max-based quantizer (radius 0), an
independent numpy evaluation of every candidate scale of every block (the
choice must be the SSE minimum and its codes must be the numpy codes), block
SSE monotone in the radius, power-of-two invariance of MXFP4, and two blocks
worked by hand from the definitions where a neighbouring scale wins.
"""
import numpy as np
import pytest

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MAX_BYTE = {0: 254, 1: 0x7E, 2: 0xF7}


def unpack(codes: np.ndarray) -> np.ndarray:
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def np_code(y: np.ndarray) -> np.ndarray:
    """E2M1 code by np.rint on the grid spacing (0.5 below 2, 1 below 4, 2
    above), ties to the even multiple, clamp at 6, sign bit from y."""
    a = np.minimum(np.abs(y), 6.0)
    q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(a / q) * q, 6.0)
    mag = np.searchsorted(GRID, r)
    return (np.signbit(y).astype(np.uint8) << 3) | mag.astype(np.uint8)


def np_scale_value(fmt: int, byte: int) -> float:
    """Scale value of a byte from the bit layout: E8M0 2^(byte-127); UE4M3 and
    UE5M3 with 3 mantissa bits, biases 7 and 15, subnormal below exponent 1."""
    if fmt == 0:
        return 2.0 ** (byte - 127)
    bias = 7 if fmt == 1 else 15
    e, j = byte >> 3, byte & 7
    if e == 0:
        return j * 2.0 ** (1 - bias - 3)
    return (1 + j / 8) * 2.0 ** (e - bias)


def np_block_sse(fmt: int, v: np.ndarray, byte: int, g: float):
    """Codes and binary64 SSE of one block under a given scale byte."""
    if fmt == 0:
        y = v.astype(np.float64) * 2.0 ** (127 - byte)        # exact
        c = np_code(y)
        xh = (np.where(c & 8, -1.0, 1.0) * GRID[c & 7] * 2.0 ** (byte - 127)).astype(np.float32)
    else:
        d = np.float32(np.float32(np_scale_value(fmt, byte)) * np.float32(g))
        if d == 0:
            c = (np.signbit(v).astype(np.uint8) << 3)
        else:
            c = np_code((v / d).astype(np.float32).astype(np.float64))
        xh = (np.where(c & 8, -1.0, 1.0).astype(np.float32) * GRID[c & 7].astype(np.float32)) * d
    e = v.astype(np.float64) - xh.astype(np.float64)
    return c, float(np.dot(e, e))


def blocks_of(x: np.ndarray, b: int) -> np.ndarray:
    return x.reshape(-1, b)


@pytest.mark.parametrize("fmt,block,gmode,rotate", [(0, 32, 0, 0), (1, 16, 1, 0), (1, 16, 1, 16),
                                                    (1, 64, 0, 0), (2, 16, 0, 0), (0, 32, 0, 32)])
def test_radius_zero_is_the_max_based_quantizer(orc, fmt, block, gmode, rotate):
    rng = np.random.default_rng([61, fmt, block, rotate])
    x = (rng.standard_t(4, (24, 256)) * 0.02).astype(np.float32)
    a = orc.quantize(x, fmt, block, gmode, None, rotate)
    b = orc.quantize_search(x, fmt, block, gmode, None, rotate, radius=0)
    for k in ("codes", "scales", "block_mse", "terms", "counts"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    assert a["g"] == b["g"]


@pytest.mark.parametrize("fmt,block,gmode", [(0, 32, 0), (1, 16, 1), (1, 8, 0), (1, 32, 2),
                                             (2, 16, 0)])
@pytest.mark.parametrize("radius", [1, 3])
def test_choice_is_the_sse_minimum_over_the_candidates(orc, fmt, block, gmode, radius):
    """Every block: evaluate all candidate bytes in numpy; the oracle's byte has
    the smallest SSE (within 1e-12 relative), keeps the max-based byte when that
    is within 2^-41 of the minimum, and its codes are numpy's codes."""
    rng = np.random.default_rng([62, fmt, block, radius])
    x = (rng.standard_t(3, (16, 512)) * 0.05).astype(np.float32)
    x[:, ::37] *= 8.0  # a few large values per row
    g = 0.01 if gmode == 2 else None
    base = orc.quantize(x, fmt, block, gmode, g)
    got = orc.quantize_search(x, fmt, block, gmode, g, 0, radius)
    gv = got["g"]
    vb = blocks_of(x, block)
    c0 = base["scales"].reshape(-1)
    chosen = got["scales"].reshape(-1)
    codes = blocks_of(unpack(got["codes"]), block)
    moved = 0
    for i in range(vb.shape[0]):
        cands = [c for c in range(c0[i] - radius, c0[i] + radius + 1) if 0 <= c <= MAX_BYTE[fmt]]
        sse = {c: np_block_sse(fmt, vb[i], c, gv)[1] for c in cands}
        best = min(sse.values())
        assert chosen[i] in sse, (i, chosen[i], cands)
        assert sse[chosen[i]] <= best * (1 + 1e-12) + 1e-300, (i, sse, chosen[i])
        if sse[c0[i]] <= best * (1 + 2.0 ** -41):
            assert chosen[i] == c0[i], (i, sse)
        want_codes, _ = np_block_sse(fmt, vb[i], int(chosen[i]), gv)
        np.testing.assert_array_equal(codes[i], want_codes, err_msg=f"block {i}")
        moved += chosen[i] != c0[i]
    assert moved > 0  # the search does change some scales on this input


@pytest.mark.parametrize("fmt,block,gmode", [(0, 32, 0), (1, 16, 1), (2, 16, 0)])
def test_block_sse_never_grows_with_the_radius(orc, fmt, block, gmode):
    rng = np.random.default_rng([63, fmt])
    x = (rng.laplace(0, 0.02, (32, 512))).astype(np.float32)
    prev = None
    for radius in range(4):
        q = orc.quantize_search(x, fmt, block, gmode, None, 0, radius)
        sse = q["block_mse"].astype(np.float64) * block  # ABS: SSE / b
        if prev is not None:
            assert np.all(sse <= prev * (1 + 1e-6) + 1e-30)
        prev = sse
    assert prev.sum() < orc.quantize(x, fmt, block, gmode)["block_mse"].sum() * block


def test_mxfp4_power_of_two_invariance(orc):
    """Scaling x by 2^t shifts every chosen E8M0 byte by t and keeps the codes."""
    rng = np.random.default_rng(64)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    a = orc.quantize_search(x, 0, 32, 0, None, 0, 2)
    for t in (-9, 5):
        b = orc.quantize_search(x * np.float32(2.0 ** t), 0, 32, 0, None, 0, 2)
        np.testing.assert_array_equal(b["scales"].astype(int), a["scales"].astype(int) + t)
        np.testing.assert_array_equal(b["codes"], a["codes"])


def test_hand_example_mxfp4_clipping_wins(orc):
    """Block [4.0, 0.25 x 31].  Max-based: floor(log2 4) - 2 = 0, byte 127, scale
    1: 4.0 -> 4 (code 6), 0.25 is the tie between 0 and 0.5 and goes to the even
    code 0: SSE = 31 * 0.0625 = 1.9375.  Byte 126 (scale 1/2): 4.0/0.5 = 8
    saturates to 6 -> 3.0 (error 1), 0.25/0.5 = 0.5 is code 1 -> 0.25 exactly:
    SSE = 1.0.  Byte 128 (scale 2): 4.0 -> 2 * 2 = 4 (code 4, exact), 0.125 -> 0
    (error 0.25 each): SSE 1.9375.  Radius 1 picks 126."""
    x = np.full((1, 32), 0.25, np.float32)
    x[0, 0] = 4.0
    r0 = orc.quantize_search(x, 0, 32, 0, None, 0, 0)
    r1 = orc.quantize_search(x, 0, 32, 0, None, 0, 1)
    assert r0["scales"][0, 0] == 127 and r1["scales"][0, 0] == 126
    assert r0["block_mse"][0, 0] * 32 == pytest.approx(1.9375, rel=1e-7)
    assert r1["block_mse"][0, 0] * 32 == pytest.approx(1.0, rel=1e-7)
    c = unpack(r1["codes"])[0]
    assert c[0] == 7 and np.all(c[1:] == 1)
    np.testing.assert_allclose(r1["terms"][:3], [0.0, 1.0, 0.0])  # the error sits on the max


def test_hand_example_ue4m3_next_code_wins(orc):
    """g = 1, block 16: [6.375, 1.25 x 15].  s = 6.375/6 = 1.0625 is the tie
    between UE4M3 1.0 (byte 0x38, even mantissa) and 1.125 (0x39): byte 0x38.
    Under d = 1: 6.375 -> 6 (error 0.375), 1.25 is the tie between 1 and 1.5 ->
    1 (even code; error 0.25): SSE 0.140625 + 15 * 0.0625 = 1.078125.  Under
    d = 1.125 (0x39): 6.375/1.125 = 5.67 -> 6 -> 6.75 (error 0.375), 1.25/1.125
    = 1.11 -> 1 -> 1.125 (error 0.125): SSE 0.140625 + 15 * 0.015625 = 0.375.
    Under d = 0.9375 (0x37): 6.375/0.9375 = 6.8 -> 6 -> 5.625 (error 0.75),
    1.25/0.9375 = 1.33 -> 1.5 -> 1.40625 (error 0.15625): SSE 0.5625 + 15 *
    0.0244140625 = 0.928.  Radius 1 picks 0x39."""
    x = np.full((1, 16), 1.25, np.float32)
    x[0, 0] = 6.375
    r0 = orc.quantize_search(x, 1, 16, 0, None, 0, 0)
    r1 = orc.quantize_search(x, 1, 16, 0, None, 0, 1)
    assert r0["scales"][0, 0] == 0x38 and r1["scales"][0, 0] == 0x39
    assert r0["block_mse"][0, 0] * 16 == pytest.approx(1.078125, rel=1e-7)
    assert r1["block_mse"][0, 0] * 16 == pytest.approx(0.375, rel=1e-7)
    np.testing.assert_allclose(r1["terms"][:3], [15 * 0.015625, 0.140625, 0.0])


def test_exact_ties_keep_the_max_based_code(orc):
    """On-grid blocks have SSE 0 under the max-based code; zero blocks have SSE 0
    under every code: the search must not move either."""
    rng = np.random.default_rng(65)
    v = GRID[rng.integers(0, 8, (4, 64))] * np.where(rng.random((4, 64)) < 0.5, -1, 1)
    v[:, ::32] = 6.0  # one maximum per block: the max-based exponent is 0
    x = (v * 2.0 ** -3).astype(np.float32)
    x[3] = 0.0
    a = orc.quantize(x, 0, 32)
    b = orc.quantize_search(x, 0, 32, 0, None, 0, 3)
    np.testing.assert_array_equal(a["scales"], b["scales"])
    np.testing.assert_array_equal(a["codes"], b["codes"])
    assert np.all(b["block_mse"] == 0)
