"""GPU parity of the MXFP4 GEMM (fp4_gemm_mxfp4, through the C ABI) against the
oracle's binary64 product of the dequantized operands.  The operands are
quantized by the oracle on the CPU.

Bar: with K <= 256 and scale bytes in [125, 129] every partial sum is exact in
binary32 (products are multiples of 2^-6 below 2^10, sums below 2^18), so C
must equal the oracle bit for bit; this pins the operand layout.  Otherwise
|C - C_oracle| <= (K/128 + 2) * 2^-23 * (|A_hat| |B_hat|^T): one binary32
rounding (at most 2^-24 of the partial sum) per 64-element matrix-core
instruction, with a factor 2 of headroom.  bf16 output is the binary32 result
rounded to nearest even, checked against the same bound plus half a bf16 ulp.
Shapes cover both epilogues (rows of C in whole 16-byte units, or not), ragged
M, N and K tails and odd K-stage counts, and both kernels: products of at
most 32 rows of A with K a multiple of 128 and 4-byte-aligned scale arrays
take the decode kernel (one K range per fragment of B, or several added by
the reduction), the others the tile kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import microscaling_fp4_quantization_amd as fq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def operand(rows, k, seed, spread=4):
    """Oracle-quantized MXFP4 operand of Normal values with a per-row scale spread."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * 2.0 ** rng.integers(-spread, spread + 1, (rows, 1)))
    q = oracle.quantize(x.astype(np.float32), oracle.FMT_MXFP4, 32)
    return q["codes"], q["scales"]


def dequant(c, s, rows, k):
    return oracle.dequantize(c, s, oracle.FMT_MXFP4, 32, 1.0, rows, k).astype(np.float64)


def run(ac, asc, bc, bsc, out_dtype=torch.float32):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return fq.fp4_gemm_mxfp4(t(ac), t(asc), t(bc), t(bsc), out_dtype).float().cpu().numpy()


def bound(ac, asc, bc, bsc, m, n, k):
    return (k / 128 + 2) * 2.0 ** -23 * (np.abs(dequant(ac, asc, m, k)) @ np.abs(dequant(bc, bsc, n, k)).T)


@pytest.mark.parametrize("m,n,k", [(16, 16, 128), (128, 128, 256), (130, 70, 96), (1, 300, 256),
                                   (257, 129, 32), (130, 70, 128), (257, 300, 256), (300, 517, 256)])
def test_gemm_exact_when_sums_are_exact(m, n, k):
    rng = np.random.default_rng([41, m, n, k])
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    asc = rng.integers(125, 130, (m, k // 32), dtype=np.uint8)
    bsc = rng.integers(125, 130, (n, k // 32), dtype=np.uint8)
    got = run(ac, asc, bc, bsc)
    want = oracle.gemm_mxfp4(ac, asc, bc, bsc, m, n, k)
    np.testing.assert_array_equal(got, want.astype(np.float32))


# Most of these split K into ranges (few tiles): the partial products are
# summed in binary64 and rounded once, which the bound already covers.
@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (64, 512, 4096), (200, 333, 1056), (128, 256, 3584),
                                   (33, 1000, 8192), (300, 517, 384), (520, 300, 512), (777, 1031, 1152),
                                   (1, 300, 2048), (16, 1000, 4096), (5, 520, 1056), (33, 260, 8192),
                                   (3, 257, 2048), (20, 520, 1024), (32, 264, 1024), (25, 33, 384),
                                   (12, 600, 128), (32, 15000, 512)])
def test_gemm_within_bound(m, n, k):
    ac, asc = operand(m, k, [42, m, k])
    bc, bsc = operand(n, k, [43, n, k])
    got = run(ac, asc, bc, bsc)
    want = oracle.gemm_mxfp4(ac, asc, bc, bsc, m, n, k)
    tol = bound(ac, asc, bc, bsc, m, n, k)
    err = np.abs(got - want)
    i = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"at {i}: got {got[i]!r} want {want[i]!r} tol {tol[i]!r}"


@pytest.mark.parametrize("m,n,k", [(96, 160, 512), (130, 158, 384), (70, 90, 96), (300, 264, 384),
                                   (7, 264, 3072), (9, 131, 1024), (3, 200, 256), (17, 15000, 768)])
def test_gemm_bf16_output(m, n, k):
    ac, asc = operand(m, k, 44)
    bc, bsc = operand(n, k, 45)
    got = run(ac, asc, bc, bsc, torch.bfloat16)
    want = oracle.gemm_mxfp4(ac, asc, bc, bsc, m, n, k)
    tol = bound(ac, asc, bc, bsc, m, n, k) + np.abs(want) * 2.0 ** -8
    assert np.all(np.abs(got - want) <= tol)


def test_gemm_zero_k_and_empty():
    z = torch.zeros((4, 0), dtype=torch.uint8, device=DEV)
    out = fq.fp4_gemm_mxfp4(z, z, torch.zeros((5, 0), dtype=torch.uint8, device=DEV),
                            torch.zeros((5, 0), dtype=torch.uint8, device=DEV))
    assert out.shape == (4, 5) and torch.all(out == 0)
    e = torch.zeros((0, 16), dtype=torch.uint8, device=DEV)
    s = torch.zeros((0, 1), dtype=torch.uint8, device=DEV)
    assert fq.fp4_gemm_mxfp4(e, s, e, s).shape == (0, 0)


def test_gemm_qwen7_up_projection_sampled_columns():
    """256 tokens x 3584 times the 18944 x 3584 up-projection: the kernel computes
    the whole product, the oracle 96 sampled output columns of it."""
    import fp4_workloads as wl
    m, n, k = 256, 18944, 3584
    w = wl.qwen7_mlp(0, 1).float().numpy()
    wq = oracle.quantize(w, oracle.FMT_MXFP4, 32)
    ac, asc = operand(m, k, 46, spread=2)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    got = fq.fp4_gemm_mxfp4(t(ac), t(asc), t(wq["codes"]), t(wq["scales"])).cpu().numpy()
    cols = np.sort(np.random.default_rng(47).choice(n, 96, replace=False))
    bc, bsc = wq["codes"][cols], wq["scales"][cols]
    want = oracle.gemm_mxfp4(ac, asc, bc, bsc, m, len(cols), k)
    tol = bound(ac, asc, bc, bsc, m, len(cols), k)
    assert np.all(np.abs(got[:, cols] - want) <= tol)


def sampled(m, n, k, seeds, cols, out_dtype=torch.float32, w=None):
    """The kernel computes the whole m x n product, the oracle `cols` sampled
    output columns of it."""
    ac, asc = operand(m, k, seeds[0], spread=2)
    if w is None:
        bc, bsc = operand(n, k, seeds[1], spread=2)
    else:
        wq = oracle.quantize(w, oracle.FMT_MXFP4, 32)
        bc, bsc = wq["codes"], wq["scales"]
    got = run(ac, asc, bc, bsc, out_dtype)
    sel = np.sort(np.random.default_rng(seeds[2]).choice(n, cols, replace=False))
    want = oracle.gemm_mxfp4(ac, asc, bc[sel], bsc[sel], m, len(sel), k)
    tol = bound(ac, asc, bc[sel], bsc[sel], m, len(sel), k)
    if out_dtype == torch.bfloat16:
        tol = tol + np.abs(want) * 2.0 ** -8
    err = np.abs(got[:, sel] - want)
    i = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"at {i}: got {got[:, sel][i]!r} want {want[i]!r} tol {tol[i]!r}"


def test_gemm_many_tiles_bf16_sampled():
    """2048 x 2048 x 512 in bf16: enough tiles that K is not split."""
    print("  case 2048x2048x512 bf16", flush=True)
    sampled(2048, 2048, 512, (48, 49, 50), 64, torch.bfloat16)


def test_gemm_decode_down_projection_sampled():
    """16 tokens x 18944 times the 3584 x 18944 down-projection: few tiles and
    a long K, the split-K path at a decode shape."""
    import fp4_workloads as wl
    print("  case 16x3584x18944", flush=True)
    w = wl.qwen7_mlp(1, 1).float().numpy()
    sampled(16, 3584, 18944, (51, None, 52), 48, w=w)


def test_gemm_decode_up_projection_sampled():
    """8 tokens x 3584 times the 18944 x 3584 up-projection: enough fragments
    of B that the decode kernel writes C directly (no K split)."""
    import fp4_workloads as wl
    print("  case 8x18944x3584", flush=True)
    w = wl.qwen7_mlp(0, 1).float().numpy()
    sampled(8, 18944, 3584, (53, None, 54), 64, torch.bfloat16, w=w)


def test_gemm_decode_unaligned_scales():
    """Scale arrays that do not start on a 4-byte boundary send a decode-sized
    product to the tile kernel; both must meet the bound, on the same data."""
    m, n, k = 6, 300, 1024
    ac, asc = operand(m, k, 55)
    bc, bsc = operand(n, k, 56)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    want = oracle.gemm_mxfp4(ac, asc, bc, bsc, m, n, k)
    tol = bound(ac, asc, bc, bsc, m, n, k)
    outs = []
    for shift in (0, 1):
        sa = torch.zeros(asc.size + shift, dtype=torch.uint8, device=DEV)
        sb = torch.zeros(bsc.size + shift, dtype=torch.uint8, device=DEV)
        sa[shift:] = t(asc).reshape(-1)
        sb[shift:] = t(bsc).reshape(-1)
        got = fq.fp4_gemm_mxfp4(t(ac), sa[shift:].view(m, k // 32), t(bc), sb[shift:].view(n, k // 32))
        outs.append(got.cpu().numpy())
        assert np.all(np.abs(outs[-1] - want) <= tol), shift


def bf16_round(x):
    """Binary32 values rounded to bf16 (nearest even), as binary32."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).bfloat16().float().numpy()


# Many tiles, one K range each: with scale bytes in [125, 127] and K <= 768
# every partial sum is a multiple of 2^-6 below 2^15, exact in binary32, so
# bf16 C must be the oracle's product rounded once to bf16.  Shapes: just
# over one and two workgroups per CU (272 and 306 tiles, the second with a
# ragged M and N whose rows of C are not whole 16-byte units, so the
# element-wise epilogue, and a K tail inside the last stage), and four per CU
# (1024 tiles).  Sampled columns (first and last included), every row.
@pytest.mark.parametrize("m,n,k", [(4352, 4096, 512), (4100, 4500, 544), (8192, 8192, 768)])
def test_gemm_many_tiles_exact_bf16(m, n, k):
    print(f"  case many tiles {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng([57, m, n, k])
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    asc = rng.integers(125, 128, (m, k // 32), dtype=np.uint8)
    bsc = rng.integers(125, 128, (n, k // 32), dtype=np.uint8)
    got = run(ac, asc, bc, bsc, torch.bfloat16)
    sel = np.sort(rng.choice(n, 64, replace=False))
    sel = np.unique(np.concatenate([sel, [0, n - 1]]))
    want = oracle.gemm_mxfp4(ac, asc, bc[sel], bsc[sel], m, len(sel), k)
    np.testing.assert_array_equal(got[:, sel], bf16_round(want))


def test_gemm_many_tiles_exact_f32():
    """512 tiles of binary32 C, one K range each (the two-pass epilogue
    through LDS straight into C): bit-exact against the oracle, sampled
    columns, every row (sums exact as above)."""
    m, n, k = 8192, 4096, 512
    print(f"  case many tiles {m}x{n}x{k} f32", flush=True)
    rng = np.random.default_rng([62, m, n, k])
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    asc = rng.integers(125, 128, (m, k // 32), dtype=np.uint8)
    bsc = rng.integers(125, 128, (n, k // 32), dtype=np.uint8)
    got = run(ac, asc, bc, bsc)
    sel = np.unique(np.concatenate([rng.choice(n, 64, replace=False), [0, n - 1]]))
    want = oracle.gemm_mxfp4(ac, asc, bc[sel], bsc[sel], m, len(sel), k)
    np.testing.assert_array_equal(got[:, sel], want.astype(np.float32))


def test_gemm_full_up_projection_sampled():
    """8192 tokens x 3584 times the 18944 x 3584 up-projection in bf16: the
    launch the MLP step times."""
    import fp4_workloads as wl
    print("  case 8192x18944x3584 bf16", flush=True)
    w = wl.qwen7_mlp(0, 1).float().numpy()
    sampled(8192, 18944, 3584, (58, None, 59), 40, torch.bfloat16, w=w)


def test_gemm_full_down_projection_sampled():
    """8192 tokens x 18944 times the 3584 x 18944 down-projection in bf16 (74
    K stages per tile, one K range)."""
    import fp4_workloads as wl
    print("  case 8192x3584x18944 bf16", flush=True)
    w = wl.qwen7_mlp(1, 1).float().numpy()
    sampled(8192, 3584, 18944, (60, None, 61), 16, torch.bfloat16, w=w)


# The bf16 epilogue of the tile kernel converts the very binary32 accumulators
# the binary32 epilogue stores (two at a time, in hardware), so with one K
# range bf16 C must be binary32 C rounded to nearest even, bit for bit, at any
# magnitude.  Each row's scale bytes are a base in 60 .. 175 plus 0 .. 3, so
# results range from about 2^-130 to 2^110.  Shapes: rows of C in whole
# 16-byte units (the epilogue through LDS) and not (the element-wise one), one
# K range each.
@pytest.mark.parametrize("m,n,k", [(8192, 4096, 1024), (4100, 4500, 544)])
def test_gemm_bf16_is_the_rounded_f32_result(m, n, k):
    print(f"  case bf16 vs f32 {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng([63, m, n, k])
    ac = t_dev(rng.integers(0, 256, (m, k // 2), dtype=np.uint8))
    bc = t_dev(rng.integers(0, 256, (n, k // 2), dtype=np.uint8))
    row_scales = lambda r: (rng.integers(60, 176, (r, 1)) + rng.integers(0, 4, (r, k // 32))).astype(np.uint8)
    asc, bsc = t_dev(row_scales(m)), t_dev(row_scales(n))
    f32 = fq.fp4_gemm_mxfp4(ac, asc, bc, bsc, torch.float32)
    b16 = fq.fp4_gemm_mxfp4(ac, asc, bc, bsc, torch.bfloat16)
    assert torch.equal(b16.view(torch.int16), f32.bfloat16().view(torch.int16))
    mag = f32.abs()
    assert bool(((mag > 0) & (mag < 2.0 ** -60)).any()) and bool((mag > 2.0 ** 60).any())


def t_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
