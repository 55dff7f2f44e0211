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


@dataclass
class PlaneFit:
    """t = a * B_first + b * B_repeat + t0 (us; a, b in us per byte): the
    per-slot pass with its requested bytes split into each routed expert's
    first read (U B_e) and the repeated reads of experts that several slots
    share ((N k - U) B_e), which a pass may serve partly from cache."""
    coef: np.ndarray         # (a, b, t0)
    cov: np.ndarray          # 3x3 covariance
    resid_sd: float
    n_points: int

    def predict(self, b_first, b_repeat):
        v = np.array([float(b_first), float(b_repeat), 1.0])
        return float(self.coef @ v), math.sqrt(max(float(v @ self.cov @ v), 0.0))

    def as_dict(self):
        def bw(c):
            return round(float(1e-3 / c), 1) if c > 0 else None
        return {"bw_first_GBs": bw(self.coef[0]), "bw_repeat_GBs": bw(self.coef[1]),
                "t0_us": round(float(self.coef[2]), 2),
                "t0_sd_us": round(math.sqrt(max(self.cov[2, 2], 0.0)), 2),
                "resid_sd_us": round(self.resid_sd, 2), "points": self.n_points}


def fit_plane(b_first, b_repeat, us):
    """Least-squares fit of us = a * b_first + b * b_repeat + t0, with the
    covariance of (a, b, t0).  Needs the three columns to be independent."""
    x1 = np.asarray(b_first, dtype=np.float64).ravel()
    x2 = np.asarray(b_repeat, dtype=np.float64).ravel()
    t = np.asarray(us, dtype=np.float64).ravel()
    if not (x1.size == x2.size == t.size):
        raise ValueError("columns differ in length")
    scale = float(max(np.max(np.abs(x1)), np.max(np.abs(x2)), 1.0))
    A = np.stack([x1 / scale, x2 / scale, np.ones_like(x1)], axis=1)
    if x1.size < 3 or np.linalg.matrix_rank(A) < 3:
        raise ValueError("need first-read bytes, repeat bytes and a constant that vary independently")
    coef, _, _, _ = np.linalg.lstsq(A, t, rcond=None)
    resid = t - A @ coef
    dof = x1.size - 3
    s2 = float(resid @ resid) / dof if dof > 0 else 0.0
    D = np.diag([1.0 / scale, 1.0 / scale, 1.0])
    cov = D @ (s2 * np.linalg.inv(A.T @ A)) @ D
    return PlaneFit(coef=D @ coef, cov=cov, resid_sd=math.sqrt(s2), n_points=int(x1.size))


def predicted_saving_trace(plane_ps: PlaneFit, fit_dd: LineFit, b_first, b_repeat):
    """The saving predicted from a trace's own split: per-slot from the
    plane at (U B_e, (N k - U) B_e), dedup from its line at U B_e.  Returns
    (saving, first-order standard error, interval standard deviation with
    both fits' residual scatter)."""
    t_ps, s_ps = plane_ps.predict(b_first, b_repeat)
    t_dd, s_dd = fit_dd.predict(b_first)
    sd = math.sqrt(s_ps ** 2 + s_dd ** 2)
    return t_ps - t_dd, sd, math.sqrt(sd ** 2 + plane_ps.resid_sd ** 2 + fit_dd.resid_sd ** 2)


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


def saving_interval_sd(fit_ps: LineFit, fit_dd: LineFit, b_ps, b_dd):
    """Standard deviation of a new measured saving about the prediction: the
    first-order error of the prediction plus each fit's residual scatter
    (the spread of single measured passes about their line).  A measured
    saving within two of these of the prediction is consistent with the
    model."""
    _, sd = predicted_saving(fit_ps, fit_dd, b_ps, b_dd)
    return math.sqrt(sd ** 2 + fit_ps.resid_sd ** 2 + fit_dd.resid_sd ** 2)


def with_bandwidth(fit: LineFit, bw_GBs):
    """The same line with its bandwidth replaced (slope = 1 / BW), fixed time
    and covariance kept: the model under a bandwidth error."""
    return LineFit(slope=1e-3 / float(bw_GBs), t0=fit.t0, cov=fit.cov, resid_sd=fit.resid_sd,
                   n_points=fit.n_points)


def first_n(ns, flags):
    """Smallest n whose flag holds, or "never"."""
    for n, f in zip(ns, flags):
        if f:
            return int(n)
    return "never"
