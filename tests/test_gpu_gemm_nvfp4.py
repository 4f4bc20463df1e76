"""GPU parity of the NVFP4 GEMM (fp4_gemm_nvfp4, through the C ABI) against the
oracle's binary64 product of the dequantized operands (oracle.gemm_nvfp4).
The operands are quantized by the oracle on the CPU (block 16, UE4M3 scale
bytes, a per-tensor g each).

Bar: with g = 1, scale bytes in [0x38, 0x3F] (values in [1, 2)) and K <= 128,
every element, product and partial sum is exact in binary32 (elements are
multiples of 2^-4 below 12, products multiples of 2^-8 below 2^8, sums below
2^15), so C must equal the oracle bit for bit; this pins the operand layout,
the decode of codes and scales, and the K pairing.  Otherwise
|C - C_oracle| <= (K/16 + 8) * 2^-23 * (|A_hat| |B_hat|^T): binary32
accumulation in 16-element steps with a factor 2 of headroom, plus the
roundings of the dequantized values (x_hat = RN32(v * RN32(s * g))) that the
kernel does not take (it multiplies by gA gB at the end).  bf16 output adds
half a bf16 ulp.  Shapes cover both epilogues, ragged M and N, K in whole
64-element stages, products split along K, and both kernels: products of at
most 32 rows of A take the decode kernel (one K range per fragment of B, or
several added by the reduction), the others the tile kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import microscaling_fp4_quantization_amd as fq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def operand(rows, k, seed, spread=3):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * 2.0 ** rng.integers(-spread, spread + 1, (rows, 1)))
    q = oracle.quantize(x.astype(np.float32), oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC)
    return q["codes"], q["scales"], q["g"]


def dequant(c, s, g, rows, k):
    return oracle.dequantize(c, s, oracle.FMT_UE4M3, 16, g, rows, k).astype(np.float64)


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run(ac, asc, ga, bc, bsc, gb, out_dtype=torch.float32):
    tg = lambda g: None if g is None else torch.tensor([g], dtype=torch.float32, device=DEV)
    return fq.fp4_gemm_nvfp4(t(ac), t(asc), tg(ga), t(bc), t(bsc), tg(gb), out_dtype).float().cpu().numpy()


def bound(ac, asc, ga, bc, bsc, gb, m, n, k):
    return (k / 16 + 8) * 2.0 ** -23 * (np.abs(dequant(ac, asc, ga, m, k)) @ np.abs(dequant(bc, bsc, gb, n, k)).T)


@pytest.mark.parametrize("m,n,k,given_g", [(16, 16, 64, False), (128, 128, 128, True), (130, 70, 64, False),
                                           (1, 300, 128, True), (257, 300, 128, False), (300, 517, 64, True)])
def test_nv_gemm_exact_when_sums_are_exact(m, n, k, given_g):
    rng = np.random.default_rng([71, m, n, k])
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    asc = rng.integers(0x38, 0x40, (m, k // 16), dtype=np.uint8)
    bsc = rng.integers(0x38, 0x40, (n, k // 16), dtype=np.uint8)
    g = 1.0 if given_g else None
    got = run(ac, asc, g, bc, bsc, g)
    want = oracle.gemm_nvfp4(ac, asc, 1.0, bc, bsc, 1.0, m, n, k)
    np.testing.assert_array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("m,n,k", [(1, 1, 64), (64, 512, 1024), (200, 333, 192), (128, 256, 3584),
                                   (33, 1000, 4096), (300, 517, 384), (520, 300, 512), (777, 1031, 1152),
                                   (1, 300, 2048), (16, 1000, 4096), (5, 520, 1088), (3, 257, 2048),
                                   (20, 300, 512), (32, 520, 1024), (17, 15000, 256), (25, 33, 64)])
def test_nv_gemm_within_bound(m, n, k):
    ac, asc, ga = operand(m, k, [72, m, k])
    bc, bsc, gb = operand(n, k, [73, n, k])
    got = run(ac, asc, ga, bc, bsc, gb)
    want = oracle.gemm_nvfp4(ac, asc, ga, bc, bsc, gb, m, n, k)
    tol = bound(ac, asc, ga, bc, bsc, gb, m, n, k)
    err = np.abs(got - want)
    i = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"at {i}: got {got[i]!r} want {want[i]!r} tol {tol[i]!r}"


@pytest.mark.parametrize("m,n,k", [(96, 160, 512), (130, 158, 384), (70, 90, 64), (7, 264, 3072)])
def test_nv_gemm_bf16_output(m, n, k):
    ac, asc, ga = operand(m, k, 74)
    bc, bsc, gb = operand(n, k, 75)
    got = run(ac, asc, ga, bc, bsc, gb, torch.bfloat16)
    want = oracle.gemm_nvfp4(ac, asc, ga, bc, bsc, gb, m, n, k)
    tol = bound(ac, asc, ga, bc, bsc, gb, m, n, k) + np.abs(want) * 2.0 ** -8
    assert np.all(np.abs(got - want) <= tol)


def test_nv_gemm_zero_k_and_empty():
    z = torch.zeros((4, 0), dtype=torch.uint8, device=DEV)
    out = fq.fp4_gemm_nvfp4(z, z, None, torch.zeros((5, 0), dtype=torch.uint8, device=DEV),
                            torch.zeros((5, 0), dtype=torch.uint8, device=DEV), None)
    assert out.shape == (4, 5) and torch.all(out == 0)
    e = torch.zeros((0, 32), dtype=torch.uint8, device=DEV)
    s = torch.zeros((0, 4), dtype=torch.uint8, device=DEV)
    assert fq.fp4_gemm_nvfp4(e, s, None, e, s, None).shape == (0, 0)


def test_nv_gemm_consumes_nvfp4_quantize_output():
    """The GPU quantizer's own NVFP4 output (dynamic g on the device) feeds the
    GEMM directly; the oracle multiplies the same codes, scales and g."""
    m, n, k = 96, 200, 512
    rng = np.random.default_rng(76)
    xa = torch.from_numpy((rng.standard_normal((m, k)) * 0.05).astype(np.float32)).to(DEV)
    xb = torch.from_numpy((rng.standard_normal((n, k)) * 0.02).astype(np.float32)).to(DEV)
    qa = fq.nvfp4_quantize(xa, 16, fq.FMT_UE4M3, fq.G_DYNAMIC, block_mse=False, stats=False)
    qb = fq.nvfp4_quantize(xb, 16, fq.FMT_UE4M3, fq.G_DYNAMIC, block_mse=False, stats=False)
    got = fq.fp4_gemm_nvfp4(qa.codes, qa.scales, qa.g, qb.codes, qb.scales, qb.g).cpu().numpy()
    ac, asc, ga = qa.codes.cpu().numpy(), qa.scales.cpu().numpy(), float(qa.g.cpu())
    bc, bsc, gb = qb.codes.cpu().numpy(), qb.scales.cpu().numpy(), float(qb.g.cpu())
    want = oracle.gemm_nvfp4(ac, asc, ga, bc, bsc, gb, m, n, k)
    assert np.all(np.abs(got - want) <= bound(ac, asc, ga, bc, bsc, gb, m, n, k))


def test_nv_gemm_qwen7_up_projection_sampled_columns():
    """256 tokens x 3584 times the NVFP4-quantized 18944 x 3584 up-projection:
    the kernel computes the whole product, the oracle 64 sampled columns."""
    import fp4_workloads as wl
    print("  case 256x18944x3584 nvfp4", flush=True)
    m, n, k = 256, 18944, 3584
    w = wl.qwen7_mlp(0, 1).float().numpy()
    wq = oracle.quantize(w, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC)
    ac, asc, ga = operand(m, k, 77, spread=2)
    got = run(ac, asc, ga, wq["codes"], wq["scales"], wq["g"], torch.bfloat16)
    cols = np.sort(np.random.default_rng(78).choice(n, 64, replace=False))
    bc, bsc = wq["codes"][cols], wq["scales"][cols]
    want = oracle.gemm_nvfp4(ac, asc, ga, bc, bsc, wq["g"], m, len(cols), k)
    tol = bound(ac, asc, ga, bc, bsc, wq["g"], m, len(cols), k) + np.abs(want) * 2.0 ** -8
    assert np.all(np.abs(got[:, cols] - want) <= tol)


def test_nv_gemm_decode_down_projection_sampled():
    """16 tokens x 18944 times the NVFP4 3584 x 18944 down projection: the
    decode kernel with K split into ranges."""
    import fp4_workloads as wl
    print("  case 16x3584x18944 nvfp4", flush=True)
    m, n, k = 16, 3584, 18944
    w = wl.qwen7_mlp(1, 1).float().numpy()
    wq = oracle.quantize(w, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC)
    ac, asc, ga = operand(m, k, 79, spread=2)
    got = run(ac, asc, ga, wq["codes"], wq["scales"], wq["g"])
    cols = np.sort(np.random.default_rng(80).choice(n, 48, replace=False))
    bc, bsc = wq["codes"][cols], wq["scales"][cols]
    want = oracle.gemm_nvfp4(ac, asc, ga, bc, bsc, wq["g"], m, len(cols), k)
    tol = bound(ac, asc, ga, bc, bsc, wq["g"], m, len(cols), k)
    assert np.all(np.abs(got[:, cols] - want) <= tol)


# Many tiles, one K range each, bf16 C: with g = 1, scale bytes in [0x38,
# 0x3F] and K = 128 every partial sum is exact in binary32 (as above), so C
# must be the oracle's product rounded once to bf16.  Just over one
# workgroup per CU (289 tiles, ragged M and N with rows of C that are not
# whole 16-byte units) and four per CU (1024 tiles).  Sampled columns (first
# and last included), every row.
@pytest.mark.parametrize("m,n,k", [(4100, 4300, 128), (8192, 8192, 128)])
def test_nv_gemm_many_tiles_exact_bf16(m, n, k):
    print(f"  case many tiles {m}x{n}x{k} nvfp4", flush=True)
    rng = np.random.default_rng([81, m, n, k])
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    asc = rng.integers(0x38, 0x40, (m, k // 16), dtype=np.uint8)
    bsc = rng.integers(0x38, 0x40, (n, k // 16), dtype=np.uint8)
    got = run(ac, asc, None, bc, bsc, None, torch.bfloat16)
    sel = np.unique(np.concatenate([rng.choice(n, 64, replace=False), [0, n - 1]]))
    want = oracle.gemm_nvfp4(ac, asc, 1.0, bc[sel], bsc[sel], 1.0, m, len(sel), k)
    want_bf16 = torch.from_numpy(want.astype(np.float32)).bfloat16().float().numpy()
    np.testing.assert_array_equal(got[:, sel], want_bf16)


def test_nv_gemm_full_up_projection_sampled():
    """8192 tokens x 3584 times the NVFP4 18944 x 3584 up-projection in bf16:
    the NVFP4 launch the MLP benchmark times."""
    import fp4_workloads as wl
    print("  case 8192x18944x3584 nvfp4 bf16", flush=True)
    m, n, k = 8192, 18944, 3584
    w = wl.qwen7_mlp(0, 1).float().numpy()
    wq = oracle.quantize(w, oracle.FMT_UE4M3, 16, oracle.GMODE_DYNAMIC)
    ac, asc, ga = operand(m, k, 82, spread=2)
    got = run(ac, asc, ga, wq["codes"], wq["scales"], wq["g"], torch.bfloat16)
    cols = np.sort(np.random.default_rng(83).choice(n, 32, replace=False))
    bc, bsc = wq["codes"][cols], wq["scales"][cols]
    want = oracle.gemm_nvfp4(ac, asc, ga, bc, bsc, wq["g"], m, len(cols), k)
    tol = bound(ac, asc, ga, bc, bsc, wq["g"], m, len(cols), k) + np.abs(want) * 2.0 ** -8
    err = np.abs(got[:, cols] - want)
    i = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"at {i}: got {got[:, cols][i]!r} want {want[i]!r} tol {tol[i]!r}"


# As for the MXFP4 GEMM: with one K range the bf16 epilogue rounds the
# binary32 result to nearest even, bit for bit (UE4M3 scale bytes over their
# whole range, given per-tensor scales; K a multiple of 64, as this GEMM takes).
@pytest.mark.parametrize("m,n,k", [(8192, 4096, 1024), (4100, 4500, 576)])
def test_nv_gemm_bf16_is_the_rounded_f32_result(m, n, k):
    print(f"  case nv bf16 vs f32 {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng([75, m, n, k])
    ac = t(rng.integers(0, 256, (m, k // 2), dtype=np.uint8))
    bc = t(rng.integers(0, 256, (n, k // 2), dtype=np.uint8))
    asc = t(rng.integers(1, 0x7F, (m, k // 16), dtype=np.uint8))
    bsc = t(rng.integers(1, 0x7F, (n, k // 16), dtype=np.uint8))
    ga = torch.tensor([0.3], dtype=torch.float32, device=DEV)
    gb = torch.tensor([1.7], dtype=torch.float32, device=DEV)
    f32 = fq.fp4_gemm_nvfp4(ac, asc, ga, bc, bsc, gb, torch.float32)
    b16 = fq.fp4_gemm_nvfp4(ac, asc, ga, bc, bsc, gb, torch.bfloat16)
    assert torch.equal(b16.view(torch.int16), f32.bfloat16().view(torch.int16))
