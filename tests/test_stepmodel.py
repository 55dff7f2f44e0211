"""Host logic of the step-time model and the crafted routings used to
calibrate it (CPU only)."""
import math

import numpy as np
import pytest
from scipy import stats

from speculative_decode_verify_gate_amd import stepmodel as M
from speculative_decode_verify_gate_amd import synth


def _line(bw_GBs, t0, nbytes):
    return np.asarray(nbytes, dtype=np.float64) / (bw_GBs * 1e3) + t0


def test_exact_line_is_recovered():
    b = np.array([1e8, 3e8, 7e8, 1.6e9])
    f = M.fit_line(b, _line(6400.0, 11.5, b))
    assert f.bw_GBs == pytest.approx(6400.0, rel=1e-10)
    assert f.t0 == pytest.approx(11.5, rel=1e-10)
    assert f.resid_sd == pytest.approx(0.0, abs=1e-9)
    t, sd = f.predict(5e8)
    assert t == pytest.approx(5e8 / 6.4e6 + 11.5, rel=1e-12)
    assert sd == pytest.approx(0.0, abs=1e-6)


def test_fit_and_errors_match_scipy_linregress():
    rng = np.random.default_rng(7)
    b = np.linspace(1e8, 1.7e9, 16)
    t = _line(5500.0, 9.0, b) + rng.normal(0.0, 2.0, b.size)
    f = M.fit_line(b, t)
    ref = stats.linregress(b, t)
    assert f.slope == pytest.approx(ref.slope, rel=1e-9)
    assert f.t0 == pytest.approx(ref.intercept, rel=1e-9)
    assert math.sqrt(f.cov[0, 0]) == pytest.approx(ref.stderr, rel=1e-6)
    assert math.sqrt(f.cov[1, 1]) == pytest.approx(ref.intercept_stderr, rel=1e-6)


def test_fit_needs_two_distinct_points():
    with pytest.raises(ValueError):
        M.fit_line([1e8], [10.0])
    with pytest.raises(ValueError):
        M.fit_line([1e8, 1e8], [10.0, 11.0])
    with pytest.raises(ValueError):
        M.fit_line([1e8, 2e8], [10.0])


def test_ratio_and_saving_on_exact_lines():
    b = np.array([1e8, 5e8, 9e8])
    ps = M.fit_line(b, _line(6000.0, 10.0, b))
    dd = M.fit_line(b, _line(4500.0, 10.0, b))
    r, r_sd = M.bandwidth_ratio(dd, ps)
    assert r == pytest.approx(0.75, rel=1e-10)
    assert r_sd == pytest.approx(0.0, abs=1e-9)
    b_ps = 1.2e9
    for u in (0.5, 0.75, 0.9):
        sav, sd = M.predicted_saving(ps, dd, b_ps, u * b_ps)
        assert sav == pytest.approx(b_ps / 6e6 - u * b_ps / 4.5e6, rel=1e-9)
        # common fixed time: dedup saves time exactly when u < r
        if u != 0.75:
            assert (sav > 0) == (u < r)
        else:
            assert sav == pytest.approx(0.0, abs=1e-9)


def test_ratio_error_propagation_matches_monte_carlo():
    rng = np.random.default_rng(3)
    b = np.linspace(2e8, 1.6e9, 12)
    ps = M.fit_line(b, _line(6000.0, 10.0, b) + rng.normal(0, 3.0, b.size))
    dd = M.fit_line(b, _line(4000.0, 14.0, b) + rng.normal(0, 3.0, b.size))
    r, r_sd = M.bandwidth_ratio(dd, ps)
    a_ps = rng.normal(ps.slope, math.sqrt(ps.cov[0, 0]), 200_000)
    a_dd = rng.normal(dd.slope, math.sqrt(dd.cov[0, 0]), 200_000)
    mc = a_ps / a_dd
    assert r == pytest.approx(float(np.median(mc)), rel=0.02)
    assert r_sd == pytest.approx(float(np.std(mc)), rel=0.1)


def test_saving_interval_covers_new_measurements():
    # repeated experiments: fit both lines on noisy passes, then measure one
    # new pass of each engine; the measured saving falls within two interval
    # standard deviations of the prediction about 95% of the time
    rng = np.random.default_rng(5)
    b = np.linspace(2e8, 1.6e9, 10)
    b_ps, b_dd = 1.3e9, 0.45e9
    inside, trials = 0, 4000
    for _ in range(trials):
        ps = M.fit_line(b, _line(6000.0, 10.0, b) + rng.normal(0, 2.0, b.size))
        dd = M.fit_line(b, _line(4500.0, 14.0, b) + rng.normal(0, 3.0, b.size))
        sav, _ = M.predicted_saving(ps, dd, b_ps, b_dd)
        sd = M.saving_interval_sd(ps, dd, b_ps, b_dd)
        meas = (b_ps / 6e6 + 10.0 + rng.normal(0, 2.0)) - (b_dd / 4.5e6 + 14.0 + rng.normal(0, 3.0))
        inside += abs(meas - sav) <= 2 * sd
    assert 0.92 <= inside / trials <= 0.985
    # exact lines: no scatter, the interval collapses to zero
    ps = M.fit_line(b, _line(6000.0, 10.0, b))
    dd = M.fit_line(b, _line(4500.0, 14.0, b))
    assert M.saving_interval_sd(ps, dd, b_ps, b_dd) == pytest.approx(0.0, abs=1e-6)


def test_plane_recovers_exact_coefficients_and_rejects_dependent_columns():
    rng = np.random.default_rng(6)
    x1 = rng.uniform(1e8, 1e9, 20)
    x2 = rng.uniform(0, 8e8, 20)
    t = x1 / 6e6 + x2 / 9e6 + 12.0
    f = M.fit_plane(x1, x2, t)
    assert f.coef[0] == pytest.approx(1 / 6e6, rel=1e-9)
    assert f.coef[1] == pytest.approx(1 / 9e6, rel=1e-9)
    assert f.coef[2] == pytest.approx(12.0, abs=1e-6)
    assert f.as_dict()["bw_first_GBs"] == pytest.approx(6000.0, rel=1e-6)
    with pytest.raises(ValueError):
        M.fit_plane(x1, 2 * x1, t)                  # repeat bytes tied to first reads
    with pytest.raises(ValueError):
        M.fit_plane(x1[:2], x2[:2], t[:2])


def test_plane_errors_match_the_spread_of_repeated_fits():
    # the reported standard errors equal the spread of the estimates over
    # repeated noisy experiments on the same design (Monte Carlo)
    rng = np.random.default_rng(7)
    x1 = np.repeat(np.linspace(1e8, 1e9, 6), 4)
    x2 = np.tile(np.linspace(0, 6e8, 4), 6)
    truth = x1 / 6e6 + x2 / 9e6 + 12.0
    est, sds = [], []
    for _ in range(3000):
        f = M.fit_plane(x1, x2, truth + rng.normal(0, 2.0, x1.size))
        est.append(f.coef)
        sds.append(np.sqrt(np.diag(f.cov)))
    est, sds = np.array(est), np.array(sds)
    np.testing.assert_allclose(est.std(axis=0), sds.mean(axis=0), rtol=0.08)
    np.testing.assert_allclose(est.mean(axis=0), [1 / 6e6, 1 / 9e6, 12.0], rtol=0.02)


def test_trace_saving_reduces_to_the_line_model_without_repeats_cost():
    # repeated reads priced like first reads: the plane is the per-slot line
    b = np.array([1e8, 3e8, 5e8, 7e8, 9e8])
    rep = np.array([0.0, 2e8, 1e8, 4e8, 3e8])
    plane = M.fit_plane(b - rep, rep, (b - rep) / 6e6 + rep / 6e6 + 10.0)
    line = M.fit_line(b, b / 6e6 + 10.0)
    dd = M.fit_line(b, b / 4.5e6 + 14.0)
    for U_bytes, rep_bytes in ((2e8, 4e8), (5e8, 1e8)):
        s_trace, _, _ = M.predicted_saving_trace(plane, dd, U_bytes, rep_bytes)
        s_line, _ = M.predicted_saving(line, dd, U_bytes + rep_bytes, U_bytes)
        assert s_trace == pytest.approx(s_line, rel=1e-9)


def test_first_n():
    assert M.first_n([1, 2, 3, 4], [False, False, True, True]) == 3
    assert M.first_n([1, 2, 3], [False, False, False]) == "never"


@pytest.mark.parametrize("N,k,E,U", [(1, 6, 64, 6), (16, 6, 64, 6), (16, 6, 64, 64),
                                     (16, 6, 64, 37), (4, 2, 8, 8), (64, 8, 256, 256),
                                     (3, 2, 8, 5)])
def test_crafted_routing_has_exactly_U_experts(N, k, E, U):
    idx, w = synth.crafted_routing(N, k, E, U, seed=N * 1000 + U)
    assert idx.shape == (N, k) and idx.dtype == np.int32
    assert np.unique(idx).size == U
    assert idx.min() >= 0 and idx.max() < E
    for row in idx:
        assert np.unique(row).size == k
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)


def test_crafted_routing_rejects_impossible_U():
    with pytest.raises(ValueError):
        synth.crafted_routing(2, 6, 64, 5, seed=0)     # U < k
    with pytest.raises(ValueError):
        synth.crafted_routing(2, 6, 64, 13, seed=0)    # U > N k
    with pytest.raises(ValueError):
        synth.crafted_routing(16, 2, 8, 9, seed=0)     # U > E


def test_with_bandwidth_replaces_only_the_slope():
    """The model under a bandwidth error: t = B / BW' + t0 with the fit's own
    fixed time, exactly."""
    f = M.fit_line([1e8, 2e8, 4e8], [30.0, 43.0, 71.0])
    g = M.with_bandwidth(f, 5000.0)
    assert g.t0 == f.t0 and abs(g.bw_GBs - 5000.0) < 1e-9
    assert abs(g.predict(3e8)[0] - (3e8 / 5000.0 / 1e3 + f.t0)) < 1e-9
