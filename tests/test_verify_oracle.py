"""Pins of the CPU oracle's speculative-decoding verification round (CPU
only).  The round follows "Building a Terminal Based LLM Inference
Internals Explorer - Part 3: Speculative Decoding", sections "The
Accept/Reject Mechanism", "A Worked Example" and "Sampling vs Greedy"."""
import json
import os

import numpy as np
import pytest

import oracle as O

CAT, DOG, FOX = 0, 1, 2

# the page's worked example (fixture with its citation)
with open(os.path.join(os.path.dirname(__file__), "golden", "verify_worked_example.json")) as fh:
    EX = json.load(fh)


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def _example():
    """The example's verifier row (plus an arbitrary bonus row) and draft row."""
    p = _f32([EX["p_verify"], [0.2, 0.3, 0.5]])
    q = _f32([EX["p_draft"]])
    return p, q


def test_worked_example_accept_probability():
    # the draft token survives exactly when u < the printed accept probability
    p, q = _example()
    x = EX["draft_token"]
    a = EX["accept_prob"]
    assert min(1.0, EX["p_verify"][x] / EX["p_draft"][x]) == pytest.approx(a)
    n, t = O.verify_gate(p, [x], q=q, u=[np.nextafter(np.float32(a), np.float32(0))], r=0)
    assert n == 1 and t[0] == x
    n, t = O.verify_gate(p, [x], q=q, u=[a], r=0)
    assert n == 0 and t[1] == -1


def test_worked_example_residual_draw():
    # the printed residual and its normalisation (to the printed decimals):
    # the rejected token can never be the correction; the next token takes
    # the first two thirds of the draw range
    p, q = _example()
    res = np.maximum(p[0].astype(np.float64) - q[0].astype(np.float64), 0)
    np.testing.assert_allclose(res, EX["residual"], atol=1e-7)
    np.testing.assert_allclose(np.round(res / res.sum(), EX["normalized_residual_decimals"]),
                               EX["normalized_residual"], atol=1e-12)
    seen = set()
    for r in np.linspace(0, 2**32 - 1, 301).astype(np.uint64):
        n, t = O.verify_gate(p, [CAT], q=q, u=[0.9], r=int(r))
        assert n == 0
        seen.add(int(t[0]))
        assert t[0] == (DOG if r < (2 / 3) * 2**32 - 2**12 else t[0])
        assert t[0] == (FOX if r > (2 / 3) * 2**32 + 2**12 else t[0])
    assert seen == {DOG, FOX}


def _searchsorted_sample(w, r):
    q = np.floor(w.astype(np.float64) * 2.0**40).astype(np.uint64)
    W = int(q.sum(dtype=np.uint64))
    if W == 0:
        return -1
    target = (W * int(r)) >> 32
    cum = np.cumsum(q, dtype=np.uint64)
    return int(np.searchsorted(cum, np.uint64(target), side="right"))


def test_sampler_matches_searchsorted():
    rng = np.random.default_rng(3)
    for V in (1, 2, 7, 1000, 50_000):
        w = rng.random(V).astype(np.float32)
        w[rng.random(V) < 0.3] = 0.0
        w /= max(w.sum(), 1e-30)
        for r in list(rng.integers(0, 2**32, 20)) + [0, 2**32 - 1]:
            assert O.sample_index(w, r) == _searchsorted_sample(w, r)
    assert O.sample_index(_f32([0, 0, 0]), 123) == -1
    assert O.sample_index(_f32([0, 1e-13, 0]), 123) == -1  # below 2^-40
    assert O.sample_index(_f32([0, 0, 1]), 0) == 2


def test_accept_plus_resample_reproduces_the_verifier_distribution():
    # drawing x ~ q, accepting with min(1, p/q) and otherwise drawing from
    # the normalised residual yields exactly p
    rng = np.random.default_rng(11)
    V = 6
    p = rng.dirichlet(np.ones(V)).astype(np.float32)
    q = rng.dirichlet(np.ones(V)).astype(np.float32)
    P = np.stack([p, rng.dirichlet(np.ones(V)).astype(np.float32)])
    trials = 60_000
    xs = rng.choice(V, size=trials, p=q.astype(np.float64) / q.sum())
    us = rng.random(trials).astype(np.float32)
    rs = rng.integers(0, 2**32, trials)
    counts = np.zeros(V)
    for x, u, r in zip(xs, us, rs):
        _, t = O.verify_gate(P, [x], q=q[None, :], u=[u], r=int(r))
        counts[t[0]] += 1
    freq = counts / trials
    sd = np.sqrt(p * (1 - p) / trials)
    assert np.all(np.abs(freq - p) < 5 * sd + 1e-6), (freq, p)


def test_greedy_round():
    p = _f32([[0.1, 0.7, 0.2], [0.5, 0.2, 0.3], [0.2, 0.2, 0.6]])
    n, t = O.verify_gate(p, [1, 0], mode=O.GREEDY)
    assert n == 2 and list(t) == [1, 0, 2]        # all accepted, bonus argmax
    n, t = O.verify_gate(p, [1, 2], mode=O.GREEDY)
    assert n == 1 and list(t) == [1, 0, -1]       # mismatch: verifier's argmax
    n, t = O.verify_gate(_f32([[0.4, 0.4, 0.2], [0.1, 0.1, 0.8]]), [1], mode=O.GREEDY)
    assert n == 0 and list(t) == [0, -1]          # tie goes to the lower index


def test_zero_draft_probability_rejects_and_zero_residual_falls_back():
    p = _f32([[0.25, 0.25, 0.5], [1, 0, 0]])
    q = _f32([[0.25, 0.25, 0.5]])
    # q(x) = p(x): always accepted, whatever u
    n, _ = O.verify_gate(p, [2], q=q, u=[0.999], r=0)
    assert n == 1
    # q(x) = 0 is never accepted; with q = p elsewhere too the residual is
    # zero, so the correction is drawn from p
    q0 = _f32([[0.25, 0.75, 0.0]])
    p0 = _f32([[0.25, 0.75, 0.0], [1, 0, 0]])
    n, t = O.verify_gate(p0, [2], q=q0, u=[0.0], r=2**31)
    assert n == 0 and t[0] == O.sample_index(p0[0], 2**31) == 1


def test_rejects_bad_arguments():
    p = _f32([[0.5, 0.5], [0.5, 0.5]])
    with pytest.raises(ValueError):
        O.verify_gate(p, [2], q=p[:1], u=[0.1])      # token outside the vocabulary
    with pytest.raises(ValueError):
        O.verify_gate(p, [0], q=None, u=[0.1])       # sampling needs q


# ------------------------------------------------ logits -> filtered distributions

def test_filter_without_top_p_is_the_temperature_softmax():
    import scipy.special
    rng = np.random.default_rng(21)
    for V, T in [(5, 1.0), (1000, 0.7), (4099, 2.5)]:
        lg = (rng.standard_normal(V) * 3).astype(np.float32)
        lg[rng.random(V) < 0.01] = -np.inf                    # masked tokens
        got, _ = O.filter_probs(lg, T, 1.0)
        ref = scipy.special.softmax(lg.astype(np.float64) / T)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)


def test_filter_hand_computed():
    # probabilities 0.5, 0.3, 0.2 (as logits): the nucleus grows by whole
    # tokens in probability order until it holds top_p of the mass
    lg = np.log(np.array([0.2, 0.5, 0.3], np.float32))
    p, _ = O.filter_probs(lg, 1.0, 0.45)
    np.testing.assert_allclose(p, [0, 1, 0], atol=1e-12)
    p, _ = O.filter_probs(lg, 1.0, 0.7)
    np.testing.assert_allclose(p, [0, 0.625, 0.375], atol=1e-7)
    p, _ = O.filter_probs(lg, 1.0, 0.81)
    np.testing.assert_allclose(p, [0.2, 0.5, 0.3], atol=1e-7)
    # equal probabilities: the lower index comes first
    p, _ = O.filter_probs(np.array([1, 1, 1, 0], np.float32), 1.0, 0.5)
    np.testing.assert_allclose(p, [0.5, 0.5, 0, 0], atol=1e-12)


def test_filter_keeps_the_minimal_prefix_of_the_sorted_order():
    rng = np.random.default_rng(22)
    for trial in range(40):
        V = int(rng.integers(2, 400))
        lg = (rng.standard_normal(V) * rng.uniform(0.3, 4)).astype(np.float32)
        if trial % 5 == 0:
            lg[: V // 3] = lg[0]                               # many exact ties
        T, top_p = float(rng.uniform(0.3, 2.0)), float(rng.uniform(0.05, 0.99))
        full, _ = O.filter_probs(lg, T, 1.0)
        got, _ = O.filter_probs(lg, T, top_p)
        order = sorted(range(V), key=lambda j: (-full[j], j))
        kept = [j for j in order if got[j] > 0]
        n = len(kept)
        assert kept == order[:n]                               # a prefix
        mass = full[kept].sum()
        assert mass >= top_p and mass - full[kept[-1]] < top_p  # minimal
        np.testing.assert_allclose(got[kept], full[kept] / mass, rtol=1e-12)
        assert abs(got.sum() - 1.0) < 1e-12
