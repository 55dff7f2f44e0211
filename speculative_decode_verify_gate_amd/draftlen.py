"""Draft length from measured verify-pass times (host arithmetic).

A speculative round drafts gamma tokens and verifies them in one pass of
n = gamma + 1 tokens ("Building a Terminal Based LLM Inference Internals
Explorer - Part 3: Speculative Decoding", section "The Flow").  Under
geometric acceptance with marginal rate alpha -- each drafted token accepted
independently -- a round yields
    E[k] = (1 - alpha^(gamma+1)) / (1 - alpha)
tokens: the accepted prefix plus the verifier's correction or bonus token
(github.com/v-code01/overdisp, first section; the same closed form drives
the cost-ratio speedup quoted on the speculative-decoding page, section
"Hypothesis 1": E[k] / (gamma c + 1) with c the draft-to-verifier cost
ratio).

With t(n) the measured time of one verify pass of n tokens and t_d the
draft's time per token, a round of length gamma delivers E[k] tokens in
t(gamma + 1) + gamma t_d, against one token per t(1) for plain decoding; so
speculation at gamma is faster exactly when
    E[k] / (t(gamma + 1) + gamma t_d) > 1 / t(1),
and the best draft length maximises the left side ("Speculative Decoding for
Mixture-of-Experts Models: Expert Bytes, Kernel Bandwidth and the Best Draft
Length", abstract, which also states that this best length is a monotone
staircase in alpha).  gamma = 0 stands for plain decoding.

The block walk replays an exact accept/reject stream a_0, a_1, ... (a_t = 1
iff the draft's token at position t is accepted) for one draft length: a
block reads up to gamma flags from the current position, advances past the
leading accepted ones plus the verifier's own token, and counts one block
(overdisp page, first section).
"""
from dataclasses import dataclass

import numpy as np


def expected_tokens(alpha, gamma):
    """E[k] = (1 - alpha^(gamma+1)) / (1 - alpha) tokens per round (gamma + 1
    at alpha = 1)."""
    alpha = float(alpha)
    if gamma < 0:
        raise ValueError("gamma must be >= 0")
    if alpha >= 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def cost_ratio_speedup(alpha, gamma, c):
    """Speedup over plain decoding when a verify pass costs the same as one
    plain step and a drafted token costs c of it: E[k] / (gamma c + 1)."""
    return expected_tokens(alpha, gamma) / (gamma * c + 1.0)


def breakeven_alpha(gamma, c, tol=1e-12):
    """The acceptance rate at which cost_ratio_speedup equals 1 (bisection;
    the speedup rises monotonically in alpha)."""
    lo, hi = 0.0, 1.0
    if cost_ratio_speedup(hi, gamma, c) < 1.0:
        return float("nan")
    while hi - lo > tol:
        mid = 0.5 * (lo + hi)
        if cost_ratio_speedup(mid, gamma, c) < 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def round_rate(alpha, gamma, t_of_n, t_draft):
    """Tokens per unit time of speculation at draft length gamma (gamma = 0:
    plain decoding, 1 / t(1)).  t_of_n: callable or mapping n -> pass time."""
    t = t_of_n if callable(t_of_n) else (lambda n: t_of_n[n])
    if gamma == 0:
        return 1.0 / t(1)
    return expected_tokens(alpha, gamma) / (t(gamma + 1) + gamma * t_draft)


def speculation_wins(alpha, gamma, t_of_n, t_draft):
    return round_rate(alpha, gamma, t_of_n, t_draft) > round_rate(alpha, 0, t_of_n, t_draft)


def best_gamma(alpha, t_of_n, t_draft, gamma_max):
    """The draft length in 0..gamma_max with the highest token rate (the
    smallest such length on exact ties)."""
    rates = [round_rate(alpha, g, t_of_n, t_draft) for g in range(gamma_max + 1)]
    return int(np.argmax(rates))


def staircase(alphas, t_of_n, t_draft, gamma_max):
    """best_gamma over a grid of acceptance rates."""
    return [best_gamma(a, t_of_n, t_draft, gamma_max) for a in alphas]


@dataclass
class WalkResult:
    tokens: int    # positions advanced
    blocks: int    # verify passes

    @property
    def per_block(self):
        return self.tokens / self.blocks if self.blocks else float("nan")


def block_walk(accept, gamma):
    """Replay an accept stream with draft length gamma >= 1.  A block at
    position p takes the run of accepted flags accept[p], accept[p+1], ...
    (at most gamma of them) and advances by that run plus one (the
    verifier's correction, or its bonus token after a fully accepted block).
    The walk stops when a block would read past the end of the stream."""
    a = np.asarray(accept, dtype=bool)
    if gamma < 1:
        raise ValueError("gamma must be >= 1")
    p, tokens, blocks = 0, 0, 0
    n = a.size
    while p + gamma <= n:
        run = 0
        while run < gamma and a[p + run]:
            run += 1
        p += run + 1
        tokens += run + 1
        blocks += 1
    return WalkResult(tokens, blocks)
