"""Lloyd-Max codebook for a Gaussian source, float64.

The IsoQuant page (section 3.1, step 2) quantizes the rotated unit-direction
blocks with a scalar Lloyd-Max quantizer but does not say how it is fitted.
Reading taken: the classical Lloyd fixed point for N(0, sigma^2) (Max, 1960),
since the coordinates of a uniformly random unit vector in d dimensions are
close to N(0, 1/d):

1. start from the Gaussian quantiles of the cell midpoints (k + 1/2) / 2^b;
2. thresholds are the midpoints of neighbouring centroids;
3. each centroid becomes the conditional mean of its cell,
   sigma * (phi(a/sigma) - phi(b/sigma)) / (Phi(b/sigma) - Phi(a/sigma));
4. repeat until no centroid moves by more than tol * sigma.
"""
from __future__ import annotations

import numpy as np
from scipy.stats import norm


def fit_gaussian(bits: int, sigma: float = 1.0, tol: float = 1e-13, max_iter: int = 200000) -> np.ndarray:
    """Ascending Lloyd-Max centroids (float64) for N(0, sigma^2) with 2^bits levels."""
    n = 2 ** bits
    c = norm.ppf((np.arange(n) + 0.5) / n)  # unit-variance start
    for _ in range(max_iter):
        tau = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-np.inf], tau))
        hi = np.concatenate((tau, [np.inf]))
        mass = norm.cdf(hi) - norm.cdf(lo)
        new = (norm.pdf(lo) - norm.pdf(hi)) / mass
        moved = np.max(np.abs(new - c))
        c = new
        if moved < tol:
            break
    return c * sigma


def gaussian_mse(centroids: np.ndarray, sigma: float = 1.0) -> float:
    """Mean squared error of nearest-centroid quantization of N(0, sigma^2) (closed form)."""
    c = np.asarray(centroids, dtype=np.float64) / sigma
    tau = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-np.inf], tau))
    hi = np.concatenate((tau, [np.inf]))
    # E[(X - c)^2; a < X < b] for X ~ N(0,1)
    def part(a, b, ck):
        pa = norm.pdf(a) if np.isfinite(a) else 0.0
        pb = norm.pdf(b) if np.isfinite(b) else 0.0
        apa = a * pa if np.isfinite(a) else 0.0
        bpb = b * pb if np.isfinite(b) else 0.0
        m0 = norm.cdf(b) - norm.cdf(a)
        m1 = pa - pb
        m2 = m0 + apa - bpb
        return m2 - 2 * ck * m1 + ck * ck * m0
    return float(sum(part(lo[k], hi[k], c[k]) for k in range(len(c)))) * sigma * sigma
