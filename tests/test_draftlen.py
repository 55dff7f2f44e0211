"""Draft-length arithmetic (CPU only), pinned to the values the pages print
and to the i.i.d. closed form."""
import json
import math
import os

import numpy as np
import pytest

from speculative_decode_verify_gate_amd import draftlen as D

# the values the speculative-decoding page prints (fixture with its citation)
with open(os.path.join(os.path.dirname(__file__), "golden", "draft_length_printed.json")) as fh:
    GOLDEN = json.load(fh)
PRINTED = [(row["acceptance"], row["gamma"], table["c"], row["speedup"])
           for table in GOLDEN["tables"] for row in table["rows"]]


@pytest.mark.parametrize("alpha,gamma,c,printed", PRINTED)
def test_cost_ratio_speedup_reproduces_the_printed_table(alpha, gamma, c, printed):
    got = round(D.cost_ratio_speedup(alpha, gamma, c), GOLDEN["printed_decimals"])
    assert got == pytest.approx(printed, abs=1e-9)


def test_breakeven_range_for_the_closer_draft():
    # the same page: with the closer draft the acceptance needed to reach
    # 1.0x spans the printed percentages over the draft lengths (3 .. 8)
    b = GOLDEN["breakeven"]
    assert round(100 * D.breakeven_alpha(3, b["c"])) == b["percent_low"]
    assert round(100 * D.breakeven_alpha(8, b["c"])) == b["percent_high"]
    for g in range(3, 9):
        a = D.breakeven_alpha(g, b["c"])
        assert D.cost_ratio_speedup(a, g, b["c"]) == pytest.approx(1.0, abs=1e-9)


def test_expected_tokens_closed_form():
    for g in range(0, 12):
        assert D.expected_tokens(0.0, g) == 1.0
        assert D.expected_tokens(1.0, g) == g + 1
        for a in (0.1, 0.5, 0.93, 0.999):
            assert D.expected_tokens(a, g) == pytest.approx(sum(a ** i for i in range(g + 1)),
                                                            rel=1e-12)


def test_block_walk_hand_computed():
    a = [1, 1, 0, 1, 1, 1, 0, 0, 1]
    # gamma 2: blocks at 0 (run 2 -> +3), 3 (run 2 -> +3), 6 (run 0 -> +1),
    # 7 (run 0 -> +1); a block at 8 would read past the end
    r = D.block_walk(a, 2)
    assert (r.tokens, r.blocks) == (8, 4)
    # gamma 1: every block reads one flag
    r = D.block_walk(a, 1)
    # p=0 run1 ->2, p=2 run0 ->3, p=3 run1 ->5, p=5 run1 ->7, p=7 run0 ->8, p=8 run1 ->10
    assert (r.tokens, r.blocks) == (10, 6)
    assert D.block_walk([0] * 10, 3).per_block == 1.0
    r = D.block_walk([1] * 12, 3)
    assert (r.tokens, r.blocks) == (12, 3)


@pytest.mark.parametrize("alpha", [0.3, 0.7, 0.93])
@pytest.mark.parametrize("gamma", [1, 4, 8])
def test_block_walk_matches_iid_closed_form(alpha, gamma):
    rng = np.random.default_rng(int(alpha * 1000) + gamma)
    stream = rng.random(400_000) < alpha
    r = D.block_walk(stream, gamma)
    e = D.expected_tokens(alpha, gamma)
    # per-block yield: mean of a capped geometric; 5 standard errors
    var = sum((i + 1) ** 2 * (alpha ** i * (1 - alpha) if i < gamma else alpha ** gamma)
              for i in range(gamma + 1)) - e * e
    assert abs(r.per_block - e) < 5 * math.sqrt(var / r.blocks)


def test_constant_pass_time_is_the_cost_ratio_model():
    t = lambda n: 1.0
    for a in (0.4, 0.8):
        for g in (1, 5):
            assert D.round_rate(a, g, t, 0.2) == pytest.approx(D.cost_ratio_speedup(a, g, 0.2))


def test_best_gamma_is_a_monotone_staircase():
    # for any positive pass-time curve the best length never decreases as
    # alpha grows (log E[k] has increasing differences in (alpha, gamma))
    rng = np.random.default_rng(5)
    alphas = np.linspace(0.0, 0.995, 200)
    for trial in range(40):
        a, b = rng.uniform(1, 20), rng.uniform(5, 40)
        wiggle = rng.uniform(0, 3, 20)
        t = {n: b + a * n + wiggle[n] for n in range(1, 18)}
        td = rng.uniform(0.0, 30.0)
        st = D.staircase(alphas, t, td, 16)
        assert all(x <= y for x, y in zip(st, st[1:])), st
        assert st[0] == 0  # alpha = 0: speculation yields one token at a higher cost


def test_speculation_wins_agrees_with_best_gamma():
    t = {n: 20.0 + 14.0 * n for n in range(1, 18)}
    for a in (0.2, 0.5, 0.8, 0.95):
        g = D.best_gamma(a, t, 3.0, 16)
        assert (g > 0) == any(D.speculation_wins(a, x, t, 3.0) for x in range(1, 17))
