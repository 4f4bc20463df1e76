"""Helpers shared by the GPU parity tests: run the library and the oracle on the
same seeded input and compare.

Tolerances (each derived from the arithmetic the two sides perform):
  codes, scale bytes, g, counts        bit-exact
  dequantized values                   bit-exact (binary32 products, same order)
  per-block MSE                        |k - o| <= 1e-6 |o|, and exactly 0 where o is 0
  tensor terms (non-max, max, zero, sum x^2)
                                       |k - o| <= 1e-6 |o|
Both sides sum exact binary64 squares of the same binary32 errors, in
different orders; the library's non-max term is within b 2^-41 of a separate
sum, relatively, block by block (it sums it separately where a difference
would lose more).  The sum of squares of bf16 inputs (no rotation) is summed
per block in binary32 by the library: within (4 + log2(b / 8)) 2^-24 of the
exact sum (at most 5.4e-7 for b = 256), so the relative MSE is within
(6 + log2(b / 8)) 2^-24 (6.6e-7) of the oracle's.  Every term holds the
relative bar with no absolute floor.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import microscaling_fp4_quantization_amd as fq

RTOL = 1e-6


def to_oracle_input(x: torch.Tensor) -> np.ndarray:
    """Exact binary32 copy of a bf16/fp32 device tensor for the oracle."""
    return x.detach().to("cpu").to(torch.float32).numpy()


def assert_block_mse(k: np.ndarray, o: np.ndarray, what="block_mse"):
    k = np.asarray(k, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    assert k.shape == o.shape
    same = k == o  # includes exact zeros and equal infinities
    zero = o == 0
    assert np.all(k[zero] == 0), f"{what}: non-zero where the oracle has 0"
    chk = ~same
    assert np.all(np.isfinite(o[chk])), f"{what}: kernel {k[chk][:4]} vs oracle {o[chk][:4]}"
    rel = np.abs(k[chk] - o[chk]) / np.abs(o[chk])
    if rel.size:
        i = int(np.argmax(rel))
        assert rel[i] <= RTOL, f"{what}: rel err {rel[i]:.3e} at {i}: {k[chk][i]} vs {o[chk][i]}"


def assert_stats(kstats: dict, terms: np.ndarray, counts: np.ndarray):
    got = np.array([kstats["sse_nonmax"], kstats["sse_max"], kstats["sse_zero"], kstats["sum_x2"]])
    for k, name in enumerate(["sse_nonmax", "sse_max", "sse_zero", "sum_x2"]):
        assert abs(got[k] - terms[k]) <= RTOL * abs(terms[k]), \
            f"{name}: {got[k]!r} vs oracle {terms[k]!r}"
    assert kstats["n_blocks"] == counts[0]
    assert kstats["n_zero_blocks"] == counts[1], (kstats["n_zero_blocks"], counts[1])


def np_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def describe_mismatch(codes, scales, ref, xin):
    """Text naming the first mismatching blocks and elements with their inputs."""
    out = []
    if xin is None:
        return ""
    xb = np.asarray(xin, np.float32)
    cols = xb.shape[1]
    block = cols // scales.shape[1]
    bad = np.argwhere(scales != ref["scales"])[:4]
    for r, k in bad:
        blk = xb[r, k * block:(k + 1) * block]
        out.append(f"scale r={r} blk={k}: kernel {scales[r, k]} oracle {ref['scales'][r, k]} "
                   f"max|x|={np.abs(blk).max()!r} bits={hex(int(np.abs(blk).max().view(np.uint32)))}")
    bad = np.argwhere(codes != ref["codes"])[:6]
    for r, j in bad:
        k = (2 * j) // block
        out.append(f"code r={r} byte={j}: kernel {codes[r, j]:#04x} oracle {ref['codes'][r, j]:#04x} "
                   f"x={xb[r, 2 * j]!r},{xb[r, 2 * j + 1]!r} scale={ref['scales'][r, k]} "
                   f"blockmax={np.abs(xb[r, k * block:(k + 1) * block]).max()!r}")
    return "\n".join(out)


def compare_quant(q: fq.Quantized, ref: dict, rows=None, check_stats=True, xin=None):
    """q: library result; ref: oracle.quantize() of the same input (or of the
    selected rows when `rows` is given); xin: the oracle's input, for messages."""
    codes = np_u8(q.codes)
    scales = np_u8(q.scales)
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    if not (np.array_equal(scales, ref["scales"]) and np.array_equal(codes, ref["codes"])):
        print(describe_mismatch(codes, scales, ref, xin), flush=True)
    np.testing.assert_array_equal(scales, ref["scales"], err_msg="scale bytes")
    np.testing.assert_array_equal(codes, ref["codes"], err_msg="codes")
    if q.block_mse is not None:
        bm = q.block_mse.detach().cpu().numpy()
        if rows is not None:
            bm = bm[rows]
        assert_block_mse(bm, ref["block_mse"])
    if q.g is not None:
        assert np.float32(q.g.item()).view(np.uint32) == np.float32(ref["g"]).view(np.uint32), \
            (q.g.item(), ref["g"])
    if check_stats and q.stats is not None and rows is None:
        assert_stats(fq.stats_dict(q.stats), ref["terms"], ref["counts"])
