"""Step-time model of one expert pass and the dedup-vs-per-slot predictor.

"Speculative Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel
Bandwidth and the Best Draft Length" (abstract) models each engine's pass
time as the bytes its kernels request over their effective bandwidth plus a
fixed time, t = B / BW + t0.  With B_ps = N k B_e for the per-slot engine and
B_dd = U B_e = u B_ps for the deduplicating engine, and a common fixed cost,
dedup is faster exactly when the byte share u = U / (N k) is below the
bandwidth ratio r = BW_dd / BW_ps.

This module is host arithmetic only: ordinary least squares for (1/BW, t0)
with the standard errors of both, the predicted time and its first-order
uncertainty, r(n) with its uncertainty, and the predicted and measured
crossovers.  Bytes are in bytes, times in microseconds, bandwidths in GB/s.
"""
from dataclasses import dataclass
import math

import numpy as np


@dataclass
class LineFit:
    """t = slope * B + t0, slope in us per byte."""
    slope: float
    t0: float
    cov: np.ndarray          # 2x2 covariance of (slope, t0)
    resid_sd: float          # residual standard deviation (us)
    n_points: int

    @property
    def bw_GBs(self):
        return (1e-3 / self.slope) if self.slope > 0 else float("inf")

    @property
    def bw_sd_GBs(self):
        """First-order standard error of the bandwidth."""
        if self.slope <= 0:
            return float("nan")
        return 1e-3 * math.sqrt(max(self.cov[0, 0], 0.0)) / (self.slope ** 2)

    def predict(self, nbytes):
        """Predicted time and its standard error (from the fit's covariance)."""
        v = np.array([float(nbytes), 1.0])
        t = self.slope * float(nbytes) + self.t0
        sd = math.sqrt(max(float(v @ self.cov @ v), 0.0))
        return t, sd

    def as_dict(self):
        return {"bw_GBs": round(self.bw_GBs, 1), "bw_sd_GBs": round(self.bw_sd_GBs, 1),
                "t0_us": round(self.t0, 2),
                "t0_sd_us": round(math.sqrt(max(self.cov[1, 1], 0.0)), 2),
                "resid_sd_us": round(self.resid_sd, 2), "points": self.n_points}


def fit_line(nbytes, us):
    """Least-squares fit of us = slope * nbytes + t0.  Needs at least two
    distinct byte counts.  With exactly two points the fit is exact and the
    covariance is zero (no residual degrees of freedom)."""
    b = np.asarray(nbytes, dtype=np.float64).ravel()
    t = np.asarray(us, dtype=np.float64).ravel()
    if b.size != t.size:
        raise ValueError("bytes and times differ in length")
    if b.size < 2 or np.unique(b).size < 2:
        raise ValueError("need at least two distinct byte counts to fit a line")
    # scale bytes to keep the normal equations well conditioned
    scale = float(np.max(np.abs(b)))
    A = np.stack([b / scale, np.ones_like(b)], axis=1)
    coef, _, _, _ = np.linalg.lstsq(A, t, rcond=None)
    resid = t - A @ coef
    dof = b.size - 2
    s2 = float(resid @ resid) / dof if dof > 0 else 0.0
    cov_s = s2 * np.linalg.inv(A.T @ A)
    D = np.diag([1.0 / scale, 1.0])
    cov = D @ cov_s @ D
    return LineFit(slope=float(coef[0] / scale), t0=float(coef[1]), cov=cov,
                   resid_sd=math.sqrt(s2), n_points=int(b.size))


def bandwidth_ratio(fit_dd: LineFit, fit_ps: LineFit):
    """r = BW_dd / BW_ps = slope_ps / slope_dd, with a first-order standard
    error from the two (independent) slope variances."""
    a_ps, a_dd = fit_ps.slope, fit_dd.slope
    r = a_ps / a_dd
    rel2 = fit_ps.cov[0, 0] / a_ps ** 2 + fit_dd.cov[0, 0] / a_dd ** 2
    return r, abs(r) * math.sqrt(max(rel2, 0.0))


def predicted_saving(fit_ps: LineFit, fit_dd: LineFit, b_ps, b_dd):
    """Predicted per-pass saving t_ps - t_dd (us) of dedup over per-slot and
    its first-order standard error (the two fits independent)."""
    t_ps, s_ps = fit_ps.predict(b_ps)
    t_dd, s_dd = fit_dd.predict(b_dd)
    return t_ps - t_dd, math.sqrt(s_ps ** 2 + s_dd ** 2)


def first_n(ns, flags):
    """Smallest n whose flag holds, or "never"."""
    for n, f in zip(ns, flags):
        if f:
            return int(n)
    return "never"
