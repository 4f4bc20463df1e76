"""Three-term quantization-error model for i.i.d. Normal weights (test infrastructure).

Source: "Is finer better? Limits of micro-scaling formats in LLMs", Metodologia,
Framework Teorico.  The page states that weights follow N(0, sigma) and that the
MSE splits into three sources: the non-maximum elements, the block maximum (not
zero because the scale itself is quantized), and zero-rounding, where a block's
maximum falls below the smallest scale and the whole block rounds to zero.  The
page does not print the model; this module is a first-principles reading of it
(order statistics of the block maximum), evaluated by quadrature:

    A = |X| has density f(a) = (2/sigma) phi(a/sigma), CDF F(a) = erf(a/(sigma sqrt 2)).
    The block maximum m has density p(m) = b f(m) F(m)^(b-1); given m the other
    b-1 magnitudes are i.i.d. with density f/F(m) on [0, m].
    d(m) is the decode scale the format assigns to a block with maximum m.
    eps_d(a) = (a - d Q(a/d))^2, Q = nearest E2M1 magnitude (saturating at 6).

    E[max]     = int p(m) [d(m) > 0] eps_d(m) dm
    E[non-max] = int p(m) [d(m) > 0] (b-1)/F(m) int_0^m f(a) eps_d(a) da dm
    E[zero]    = int p(m) [d(m) = 0] (m^2 + (b-1)/F(m) int_0^m a^2 f(a) da) dm

and each term per element is the block expectation divided by b.

The inner integrals are closed-form Gaussian partial moments over the rounding
cells of Q; the outer integral is split at every point where d(m) changes or
m/d crosses a rounding boundary, and each piece gets Gauss-Legendre quadrature
in float64.  Continuous arithmetic is assumed (no binary32 rounding of m/D), so
agreement with a sampled tensor is statistical, not bitwise.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

# E2M1 magnitudes and the rounding-cell boundaries between them (units of d).
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
CELL_LO = np.array([0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
CELL_HI = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, np.inf])

_SQRT2PI = math.sqrt(2.0 * math.pi)


def _ue4m3_values():
    v = [j * 2.0 ** -9 for j in range(8)]
    for e in range(1, 16):
        for j in range(8):
            if e == 15 and j == 7:
                continue
            v.append((1 + j / 8) * 2.0 ** (e - 7))
    return np.array(sorted(set(v)))


def _ue5m3_values():
    v = [j * 2.0 ** -17 for j in range(8)]
    for e in range(1, 31):
        for j in range(8):
            v.append((1 + j / 8) * 2.0 ** (e - 15))
    return np.array(sorted(set(v)))


class _Half:
    """Half-normal |X|, X ~ N(0, sigma)."""

    def __init__(self, sigma: float):
        self.s = float(sigma)

    def F(self, a):
        return erf(np.asarray(a, dtype=np.float64) / (self.s * math.sqrt(2.0)))

    def f(self, a):
        t = np.asarray(a, dtype=np.float64) / self.s
        return 2.0 * np.exp(-0.5 * t * t) / (_SQRT2PI * self.s)

    def _phi(self, a):
        t = np.asarray(a, dtype=np.float64) / self.s
        return np.exp(-0.5 * t * t) / _SQRT2PI

    def moments(self, u, v):
        """(int f, int a f, int a^2 f) over [u, v] (arrays broadcast)."""
        u = np.asarray(u, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        Fu, Fv = self.F(u), self.F(v)
        pu, pv = self._phi(u), self._phi(v)
        pu = np.where(np.isinf(u), 0.0, pu)
        pv = np.where(np.isinf(v), 0.0, pv)
        uu = np.where(np.isinf(u), 0.0, u)
        vv = np.where(np.isinf(v), 0.0, v)
        i0 = Fv - Fu
        i1 = 2.0 * self.s * (pu - pv)
        i2 = self.s ** 2 * (Fv - Fu) - 2.0 * self.s * (vv * pv - uu * pu)
        return i0, i1, i2


def _inner_eps(h: _Half, d: float, m: np.ndarray) -> np.ndarray:
    """int_0^m f(a) eps_d(a) da for an array of m (fixed d > 0)."""
    out = np.zeros_like(m)
    for lo, hi, val in zip(CELL_LO, CELL_HI, GRID):
        u = lo * d
        v = np.minimum(hi * d, m)
        live = v > u
        if not live.any():
            continue
        i0, i1, i2 = h.moments(np.full_like(m, u), np.where(live, v, u))
        q = val * d
        out += np.where(live, i2 - 2.0 * q * i1 + q * q * i0, 0.0)
    return out


def _eps(d: float, a: np.ndarray) -> np.ndarray:
    y = a / d
    idx = np.searchsorted(CELL_HI, y, side="left")  # cell index (ties measure zero)
    idx = np.minimum(idx, 7)
    return (a - d * GRID[idx]) ** 2


def _pieces(fmt: str, g: float, m_hi: float):
    """List of (lo, hi, d) with d constant on [lo, hi]; d = 0 marks zero-rounding."""
    out = []
    if fmt == "mxfp4":
        k_lo = -150
        k = k_lo
        while 2.0 ** k < m_hi:
            lo, hi = 2.0 ** k, 2.0 ** (k + 1)
            e = max(min(k - 2, 127), -127)
            out.append((lo, min(hi, m_hi), 2.0 ** e))
            k += 1
        return out
    vals = _ue4m3_values() if fmt == "ue4m3" else _ue5m3_values()
    D = 6.0 * g
    mids = 0.5 * (vals[1:] + vals[:-1])
    # s in [0, mids[0]] -> 0 ; (mids[j-1], mids[j]) -> vals[j] ; beyond the top -> top value
    edges = np.concatenate([[0.0], mids, [np.inf]]) * D
    for j in range(len(vals)):
        lo, hi = edges[j], min(edges[j + 1], m_hi)
        if lo >= m_hi:
            break
        out.append((lo, hi, vals[j] * g))
    return out


def predict(sigma: float, block: int, fmt: str = "ue4m3", g: float = 1.0,
            nodes: int = 48) -> dict:
    """Expected per-element squared error terms for i.i.d. N(0, sigma) blocks.

    ``fmt`` is "mxfp4", "ue4m3" or "ue5m3"; ``g`` the per-tensor scale (UE4M3).
    Returns {"nonmax", "max", "zero", "total", "p_zero_block"}.
    """
    h = _Half(sigma)
    b = int(block)
    m_hi = sigma * (math.sqrt(2.0 * math.log(max(b, 2))) + 12.0)
    xg, wg = np.polynomial.legendre.leggauss(nodes)
    e_max = e_non = e_zero = p_zero = 0.0
    for lo, hi, d in _pieces(fmt, g, m_hi):
        if hi <= lo:
            continue
        # split at rounding-cell boundaries of m/d and at multiples of sigma
        cuts = [lo, hi]
        if d > 0:
            cuts += [t * d for t in CELL_LO[1:] if lo < t * d < hi]
        step = sigma / 2.0
        n_sub = int(math.ceil((hi - lo) / step))
        if n_sub > 1:
            cuts += list(np.linspace(lo, hi, min(n_sub, 400) + 1)[1:-1])
        cuts = np.unique(np.array(cuts))
        for a, c in zip(cuts[:-1], cuts[1:]):
            m = 0.5 * (c - a) * xg + 0.5 * (c + a)
            w = 0.5 * (c - a) * wg
            Fm = h.F(m)
            pm = b * h.f(m) * Fm ** (b - 1)
            with np.errstate(divide="ignore", invalid="ignore"):
                cond = np.where(Fm > 0, (b - 1) / Fm, 0.0)
            if d > 0:
                e_max += np.sum(w * pm * _eps(d, m))
                e_non += np.sum(w * pm * cond * _inner_eps(h, d, m))
            else:
                _, _, i2 = h.moments(np.zeros_like(m), m)
                e_zero += np.sum(w * pm * (m * m + cond * i2))
                p_zero += np.sum(w * pm)
    return {"nonmax": e_non / b, "max": e_max / b, "zero": e_zero / b,
            "total": (e_non + e_max + e_zero) / b, "p_zero_block": p_zero}


def p_zero_block_closed_form(sigma: float, block: int, threshold: float) -> float:
    """Probability that all |x_i| of a block lie below ``threshold``: F(t)^b."""
    return float(erf(threshold / (sigma * math.sqrt(2.0))) ** block)
