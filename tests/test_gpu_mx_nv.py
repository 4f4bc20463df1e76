"""fp4_quantize_mx_nv (MXFP4 and dynamic NVFP4 of one tensor in one call, the
NVFP4 per-tensor scale taken from the MXFP4 pass) against the two separate
calls, bit for bit, and against the oracle.

"Diagnosing FP4 inference", technical summary section 2: every layer's
tensors quantized in both formats.  The separate calls are themselves held to
the oracle elsewhere; here every output of the combined call must equal theirs
exactly (codes, scale bytes, per-block MSE, g and the tensor terms), except the
NVFP4 sum-of-squares term under the absolute MSE, which the combined call sums
in its quantize kernel instead of the amax pass (same value to rounding: the
oracle's bar applies)."""
import numpy as np
import pytest
import torch

import fp4_workloads as wl
import oracle
import microscaling_fp4_quantization_amd as fq
from parity_util import compare_quant, to_oracle_input

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def seeded(shape, seed, dtype=torch.bfloat16, sigma=0.02):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return torch.from_numpy(a).to(dtype).to(DEV)


def same(a: torch.Tensor, b: torch.Tensor):
    assert a.shape == b.shape and a.dtype == b.dtype
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def check_against_separate(x, nv_block, kind, block_mse=True, stats=True):
    m, v = fq.fp4_quantize_mx_nv(x, nv_block, mse_kind=kind, block_mse=block_mse, stats=stats)
    a = fq.mxfp4_quantize(x, mse_kind=kind, block_mse=block_mse, stats=stats)
    b = fq.nvfp4_quantize(x, nv_block, fq.FMT_UE4M3, fq.G_DYNAMIC, None, 0, mse_kind=kind,
                          block_mse=block_mse, stats=stats)
    torch.cuda.synchronize()
    same(m.codes, a.codes)
    same(m.scales, a.scales)
    same(v.codes, b.codes)
    same(v.scales, b.scales)
    same(v.g, b.g)
    if block_mse:
        same(m.block_mse, a.block_mse)
        same(v.block_mse, b.block_mse)
    if stats:
        same(m.stats, a.stats)
        if kind == fq.MSE_REL and block_mse:
            same(v.stats, b.stats)
        else:
            sv, sb = fq.stats_dict(v.stats), fq.stats_dict(b.stats)
            for k in ("sse_nonmax", "sse_max", "sse_zero", "n_blocks", "n_zero_blocks"):
                assert sv[k] == sb[k], k
            # Without the relative per-block MSE, the separate dynamic call
            # sums x^2 in its amax pass (binary64) and the combined call in its
            # NVFP4 quantize pass.  For bf16 values the quantize pass sums each
            # block in binary32 (within (4 + log2(b / 8)) 2^-24 of the exact
            # sum, relatively), else in binary64 like the amax pass.
            tol = 1e-6 if x.dtype == torch.bfloat16 else 1e-12
            assert abs(sv["sum_x2"] - sb["sum_x2"]) <= tol * sb["sum_x2"]
    return m, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", [fq.MSE_ABS, fq.MSE_REL])
@pytest.mark.parametrize("nv_block", [16, 32, 8])
def test_matches_separate_calls_and_oracle(dtype, kind, nv_block):
    x = seeded((67, 1536), [115, nv_block, kind], dtype)
    print(f"  mx_nv dtype={dtype} kind={kind} nv_block={nv_block}", flush=True)
    m, v = check_against_separate(x, nv_block, kind)
    xf = to_oracle_input(x)
    compare_quant(m, oracle.quantize(xf, oracle.FMT_MXFP4, 32, mse_kind=kind), xin=xf)
    compare_quant(v, oracle.quantize(xf, oracle.FMT_UE4M3, nv_block, oracle.GMODE_DYNAMIC,
                                     mse_kind=kind), xin=xf)


@pytest.mark.parametrize("block_mse,stats", [(False, False), (True, False), (False, True)])
def test_partial_outputs(block_mse, stats):
    x = seeded((300, 2048), 116)
    check_against_separate(x, 16, fq.MSE_REL, block_mse, stats)


def test_empty_tensor():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    m, v = fq.fp4_quantize_mx_nv(x)
    torch.cuda.synchronize()
    assert v.g.item() == 1.0
    for q in (m, v):
        st = fq.stats_dict(q.stats)
        assert st["n_blocks"] == 0 and st["sse_nonmax"] == 0.0 and st["sum_x2"] == 0.0


def test_all_zero_tensor_gives_unit_scale():
    x = torch.zeros((64, 512), dtype=torch.bfloat16, device=DEV)
    m, v = check_against_separate(x, 16, fq.MSE_REL)
    assert v.g.item() == 1.0


@pytest.mark.parametrize("proj", range(len(wl.QWEN14_PROJ)))
def test_qwen14_layer0_full_size(proj):
    """Every projection of layer 0 of the 14B-shaped stack, as the benchmark
    runs it (relative MSE, tensor terms), against the separate calls."""
    x = wl.qwen14_layer_tensor(0, proj).to(DEV)
    print(f"  mx_nv layer 0 {wl.QWEN14_PROJ[proj][0]}", flush=True)
    check_against_separate(x, 16, fq.MSE_REL)


def test_two_calls_in_a_row_reuse_the_workspace():
    """A large call then a small one on the same workspace: nothing of the
    first (maxima, partials) leaks into the second."""
    big = seeded((4096, 4096), 117, sigma=0.5)
    small = seeded((33, 512), 118)
    fq.fp4_quantize_mx_nv(big, mse_kind=fq.MSE_REL)
    check_against_separate(small, 16, fq.MSE_REL)


def check_batch_against_single(xs, nv_block, kind, block_mse=True, stats=True):
    """Every code byte, scale byte, per-block MSE and g of the batched call equals
    the single-tensor call's; the tensor terms equal it to rounding (partials
    follow each tensor's share of the grid)."""
    got = fq.fp4_quantize_mx_nv_batch(xs, nv_block, mse_kind=kind, block_mse=block_mse, stats=stats)
    for i, x in enumerate(xs):
        m, v = got[i]
        a, b = fq.fp4_quantize_mx_nv(x, nv_block, mse_kind=kind, block_mse=block_mse, stats=stats)
        torch.cuda.synchronize()
        print(f"  batch tensor {i} shape={tuple(x.shape)}", flush=True)
        for q, r in ((m, a), (v, b)):
            same(q.codes, r.codes)
            same(q.scales, r.scales)
            if block_mse:
                same(q.block_mse, r.block_mse)
            if stats:
                sq, sr = fq.stats_dict(q.stats), fq.stats_dict(r.stats)
                for k in ("n_blocks", "n_zero_blocks"):
                    assert sq[k] == sr[k], (i, k)
                for k in ("sse_nonmax", "sse_max", "sse_zero", "sum_x2"):
                    assert abs(sq[k] - sr[k]) <= 1e-12 * abs(sr[k]), (i, k, sq[k], sr[k])
        same(v.g, b.g)
    return got


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", [fq.MSE_ABS, fq.MSE_REL])
@pytest.mark.parametrize("nv_block", [16, 32])
def test_batch_matches_single_calls_and_oracle(dtype, kind, nv_block):
    shapes = [(67, 1536), (1, 64), (300, 2048), (64, 4096), (5, 96)]
    xs = [seeded(s, [119, i, nv_block], dtype, sigma=0.02 * (i + 1)) for i, s in enumerate(shapes)]
    print(f"  batch dtype={dtype} kind={kind} nv_block={nv_block}", flush=True)
    got = check_batch_against_single(xs, nv_block, kind)
    for (m, v), x in zip(got, xs):
        xf = to_oracle_input(x)
        compare_quant(m, oracle.quantize(xf, oracle.FMT_MXFP4, 32, mse_kind=kind), xin=xf)
        compare_quant(v, oracle.quantize(xf, oracle.FMT_UE4M3, nv_block, oracle.GMODE_DYNAMIC,
                                         mse_kind=kind), xin=xf)


@pytest.mark.parametrize("block_mse,stats", [(False, False), (True, False), (False, True)])
def test_batch_partial_outputs(block_mse, stats):
    xs = [seeded((300, 2048), 120), seeded((17, 512), 121)]
    check_batch_against_single(xs, 16, fq.MSE_REL, block_mse, stats)


def test_batch_with_empty_and_zero_tensors():
    xs = [torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), seeded((40, 256), 122),
          torch.zeros((8, 128), dtype=torch.bfloat16, device=DEV),
          torch.empty((0, 32), dtype=torch.bfloat16, device=DEV)]
    got = fq.fp4_quantize_mx_nv_batch(xs, 16, mse_kind=fq.MSE_REL)
    torch.cuda.synchronize()
    for i in (0, 3):
        m, v = got[i]
        assert v.g.item() == 1.0
        assert fq.stats_dict(m.stats)["n_blocks"] == 0 and fq.stats_dict(v.stats)["sse_max"] == 0.0
    assert got[2][1].g.item() == 1.0
    check_batch_against_single(xs[1:3], 16, fq.MSE_REL)


def test_batch_of_sixteen():
    xs = [seeded((16 + 8 * i, 256 + 32 * (i % 3)), [123, i]) for i in range(fq.MAX_BATCH)]
    check_batch_against_single(xs, 16, fq.MSE_REL)


def test_qwen14_layer_batch_full_size():
    """Layer 1 of the 14B-shaped stack as one batch, as the benchmark runs it:
    against the single-tensor calls and, element by element, the oracle."""
    from concurrent.futures import ThreadPoolExecutor
    hosts = [wl.qwen14_layer_tensor(1, p) for p in range(len(wl.QWEN14_PROJ))]
    xs = [h.to(DEV) for h in hosts]
    got = check_batch_against_single(xs, 16, fq.MSE_REL)
    with ThreadPoolExecutor(16) as pool:
        for i, ((m, v), x) in enumerate(zip(got, xs)):
            print(f"  oracle layer 1 {wl.QWEN14_PROJ[i][0]}", flush=True)
            xf = to_oracle_input(x)
            rows = xf.shape[0]
            cuts = np.linspace(0, rows, 33).astype(int)
            g = oracle.dynamic_g(oracle.tensor_amax(xf))
            for fmt, b, gmode, q in ((oracle.FMT_MXFP4, 32, oracle.GMODE_NONE, m),
                                     (oracle.FMT_UE4M3, 16, oracle.GMODE_GIVEN, v)):
                parts = list(pool.map(lambda k: oracle.quantize(xf[cuts[k]:cuts[k + 1]], fmt, b, gmode, g,
                                                                mse_kind=oracle.MSE_REL), range(32)))
                ref = {"codes": np.concatenate([p["codes"] for p in parts]),
                       "scales": np.concatenate([p["scales"] for p in parts]),
                       "block_mse": np.concatenate([p["block_mse"] for p in parts]),
                       "terms": np.sum([p["terms"] for p in parts], axis=0),
                       "counts": np.sum([p["counts"] for p in parts], axis=0), "g": g}
                compare_quant(q, ref)
