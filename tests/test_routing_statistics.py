"""Statistical sanity of the synthetic routing (CPU, oracle routing).

With independent hidden states (rho = 0) and N(0, 0.02) gates, every token
picks its k experts almost like a uniform draw of k of the E, so the expected
number of distinct experts in a pass of N tokens is close to
E (1 - (1 - k/E)^N).  The gate rows of one fixed draw are not exactly
exchangeable, so this is a sanity band, not an identity.
"""
import numpy as np

import oracle as O
from speculative_decode_verify_gate_amd import synth
from helpers import oshape


def _u_bar(cfg, n, layers, reps, rho):
    s = oshape(cfg)
    shares = []
    for layer in range(layers):
        gate = synth.make_gate(cfg, "cpu", layer).numpy()
        for rep in range(reps):
            x = synth.make_hidden(cfg, n, rep, "cpu", rho=rho, rho_index=layer).numpy()
            idx = O.route(s, gate, x)["idx"]
            shares.append(np.unique(idx).size / idx.size)
    return float(np.mean(shares))


def test_independent_tokens_share_experts_like_uniform_draws():
    cfg = synth.CONFIGS["v2stack"]          # the rho-sweep stack: E 64, k 6
    for n in (4, 16):
        N = cfg.tokens(n)
        expect = cfg.E * (1 - (1 - cfg.k / cfg.E) ** N) / (N * cfg.k)
        got = _u_bar(cfg, n, layers=6, reps=12, rho=0.0)
        assert abs(got - expect) < 0.04, (n, got, expect)


def test_correlated_tokens_share_more():
    # the AR(1) correlation only ever lowers the byte share at fixed n
    cfg = synth.CONFIGS["v2stack"]
    lo = _u_bar(cfg, 16, layers=2, reps=6, rho=0.99)
    hi = _u_bar(cfg, 16, layers=2, reps=6, rho=0.0)
    assert lo < 0.5 * hi
