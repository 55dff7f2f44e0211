"""Pins of the oracle's layer variants (CPU only).

Biased routing follows the DeepSeek-style routing sketch in "Deep Dive into
Mixture of Experts: From 1991 to DeepSeek-V3", section 5 (a per-expert bias
added to the gate's scores, then top-k and softmax over the selected values).
Grouped dedup applies the deduplicating engine of "Speculative Decoding for
Mixture-of-Experts Models: Expert Bytes, Kernel Bandwidth and the Best Draft
Length" (abstract) inside each group of tokens, e.g. per sequence of a batch.
"""
import itertools

import numpy as np
import pytest

import oracle as O
from test_oracle import _layer_np


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- biased routing

def test_bias_is_a_constant_input_feature():
    # x @ Wg + b equals [x, 1] @ [Wg | b]: the biased route must equal the
    # plain route of the augmented problem in every output, bit for bit
    rng = _rng(1)
    for d, E, k, n in [(8, 8, 2, 5), (16, 64, 6, 7), (32, 256, 8, 3), (4, 5, 5, 2)]:
        s = O.Shape(d, E, k, 16, 0, O.F32)
        gw = rng.standard_normal((E, d)).astype(np.float32)
        b = (rng.standard_normal(E) * 0.7).astype(np.float32)
        x = rng.standard_normal((n, d)).astype(np.float32)
        got = O.route(s, gw, x, bias=b)
        s1 = O.Shape(d + 1, E, k, 16, 0, O.F32)
        ref = O.route(s1, np.concatenate([gw, b[:, None]], axis=1),
                      np.concatenate([x, np.ones((n, 1), np.float32)], axis=1))
        for key in ("logits", "idx", "w", "margin", "flags"):
            assert np.array_equal(got[key], ref[key]), key


def test_bias_enters_the_softmax_hand_computed():
    # d = 2, E = 3, k = 2; x = (1, 0); gate rows (1, 0), (0.5, 0), (0, 0);
    # bias (0, 0, 2): biased logits (1, 0.5, 2) -> experts 2 then 0, weights
    # softmax(2, 1) = (1 / (1 + e^-1), e^-1 / (1 + e^-1)).  Were the bias
    # used for the selection only, the weights would be softmax(0, 1).
    s = O.Shape(2, 3, 2, 16, 0, O.F32)
    gw = np.array([[1, 0], [0.5, 0], [0, 0]], np.float32)
    r = O.route(s, gw, np.array([[1, 0]], np.float32), bias=np.array([0, 0, 2], np.float32))
    assert list(r["idx"][0]) == [2, 0]
    e = np.exp(-1.0)
    np.testing.assert_allclose(r["w"][0], [1 / (1 + e), e / (1 + e)], rtol=1e-15)
    assert r["margin"][0] == pytest.approx(0.5, abs=1e-15)
    np.testing.assert_array_equal(r["logits"][0], [1.0, 0.5, 2.0])


def test_uniform_bias_changes_nothing_but_the_logits():
    # softmax and the order are invariant to a shift shared by all experts
    rng = _rng(2)
    s = O.Shape(16, 64, 6, 16, 0, O.F32)
    gw = rng.standard_normal((64, 16)).astype(np.float32)
    x = rng.standard_normal((12, 16)).astype(np.float32)
    plain = O.route(s, gw, x)
    shifted = O.route(s, gw, x, bias=np.full(64, 0.25, np.float32))
    ok = plain["flags"] == 0
    assert np.array_equal(plain["idx"][ok], shifted["idx"][ok])
    np.testing.assert_allclose(shifted["w"], plain["w"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(shifted["logits"], plain["logits"] + 0.25, rtol=0, atol=1e-12)


def test_biased_selection_brute_force():
    # every k-subset scored by its biased logit sum; the best one (the
    # lexicographically smallest index set among exact ties) is the selection
    rng = _rng(3)
    for trial in range(30):
        E, d = int(rng.integers(2, 8)), 3
        k = int(rng.integers(1, E + 1))
        s = O.Shape(d, E, k, 16, 0, O.F32)
        gw = rng.integers(-3, 4, (E, d)).astype(np.float32)  # small integers: exact ties
        b = rng.integers(-2, 3, E).astype(np.float32)
        x = rng.integers(-2, 3, (1, d)).astype(np.float32)
        L = (gw.astype(np.float64) @ x[0].astype(np.float64)) + b
        best = max(itertools.combinations(range(E), k),
                   key=lambda c: (sum(L[list(c)]), [-i for i in c]))
        got = O.route(s, gw, x, bias=b)["idx"][0]
        assert sorted(got) == list(best)
        # slot order: value descending, index ascending
        assert list(got) == sorted(got, key=lambda e: (-L[e], e))


def test_large_bias_forces_an_expert_into_every_token():
    rng = _rng(4)
    s = O.Shape(16, 32, 4, 16, 0, O.F32)
    gw = rng.standard_normal((32, 16)).astype(np.float32)
    x = rng.standard_normal((20, 16)).astype(np.float32)
    b = np.zeros(32, np.float32)
    b[11] = 1000.0
    r = O.route(s, gw, x, bias=b)
    assert (r["idx"][:, 0] == 11).all()
    assert (r["w"][:, 0] == 1.0).all()     # exp(-1000) underflows against it
    # the other slots are the plain route's top (k - 1) among the others
    plain = O.route(O.Shape(16, 31, 3, 16, 0, O.F32), np.delete(gw, 11, axis=0), x)
    others = np.where(plain["idx"] >= 11, plain["idx"] + 1, plain["idx"])
    ok = plain["flags"] == 0
    assert np.array_equal(r["idx"][ok, 1:], others[ok])


# ---------------------------------------------------------------- grouped dedup

def _small_layer(seed, d=32, E=8, k=2, f=32, S=1):
    s = O.Shape(d, E, k, f, S, O.BF16)
    return s, _layer_np(s, seed)


def _routing(rng, n, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(n)]).astype(np.int32)


def _weights(rng, n, k):
    w = rng.random((n, k))
    return w / w.sum(axis=1, keepdims=True)


def test_one_group_is_the_dedup_engine_and_one_token_groups_the_per_slot_engine():
    rng = _rng(5)
    s, lay = _small_layer(5)
    n = 6
    x = rng.standard_normal((n, s.d)).astype(np.float32)
    idx = _routing(rng, n, s.E, s.k)
    w = _weights(rng, n, s.k)
    args = (s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x, idx, w)
    y_ps, b_ps, sh_ps, _ = O.layer(*args, engine="perslot")
    y_dd, b_dd, sh_dd, u_dd = O.layer(*args, engine="dedup")
    y1, b1, sh1, u1 = O.layer_grouped(*args, [0, n])
    assert np.array_equal(y1, y_dd) and b1 == b_dd and sh1 == sh_dd and list(u1) == [u_dd]
    yn, bn, shn, un = O.layer_grouped(*args, list(range(n + 1)))
    assert np.array_equal(yn, y_ps) and bn == b_ps and shn == sh_ps
    assert (un == s.k).all()


def test_group_counts_match_sets_and_union_bound():
    rng = _rng(6)
    s, lay = _small_layer(6, E=16, k=3)
    n = 12
    x = rng.standard_normal((n, s.d)).astype(np.float32)
    # correlated routing so groups share experts
    base = _routing(rng, 1, s.E, s.k)[0]
    idx = np.stack([base if rng.random() < 0.6 else rng.permutation(s.E)[:s.k]
                    for _ in range(n)]).astype(np.int32)
    w = _weights(rng, n, s.k)
    Be = O.expert_bytes(s)
    union = len(set(idx.ravel().tolist()))
    y_ref = None
    for gs in ([0, 12], [0, 3, 6, 9, 12], [0, 1, 5, 12], [0, 4, 8, 12], list(range(13))):
        y, b, sh, u = O.layer_grouped(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"],
                                      x, idx, w, gs)
        sets = [set(idx[gs[g]:gs[g + 1]].ravel().tolist()) for g in range(len(gs) - 1)]
        assert list(u) == [len(q) for q in sets]
        assert b == sum(len(q) for q in sets) * Be
        assert union <= sum(u) <= n * s.k
        # the layer output does not depend on how the tokens are grouped
        if y_ref is None:
            y_ref = y
        assert np.array_equal(y, y_ref)
    # refining a grouping never lowers the total
    coarse = O.layer_grouped(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x, idx, w,
                             [0, 6, 12])[3].sum()
    fine = O.layer_grouped(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x, idx, w,
                           [0, 3, 6, 9, 12])[3].sum()
    assert coarse <= fine


def test_grouped_rejects_bad_boundaries():
    rng = _rng(7)
    s, lay = _small_layer(7)
    x = rng.standard_normal((4, s.d)).astype(np.float32)
    idx = _routing(rng, 4, s.E, s.k)
    w = _weights(rng, 4, s.k)
    for gs in ([1, 4], [0, 3], [0, 2, 2, 4], [0, 3, 2, 4], [0]):
        with pytest.raises(ValueError):
            O.layer_grouped(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x, idx, w, gs)


def test_grouped_output_equals_torch_mixture_on_a_tiny_case():
    # two groups; y from torch's own matmul/silu per slot, rounding points
    # as in the bf16 reading
    from test_oracle import _torch_swiglu
    rng = _rng(8)
    s, lay = _small_layer(8, d=32, E=4, k=2, f=32, S=1)
    n = 3
    x = rng.standard_normal((n, s.d)).astype(np.float32)
    idx = np.array([[0, 1], [1, 2], [3, 0]], np.int32)
    w = _weights(rng, n, s.k)
    y, b, _, u = O.layer_grouped(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"],
                                 x, idx, w, [0, 2, 3])
    assert list(u) == [3, 2]
    for t in range(n):
        ref = sum(w[t, j] * _torch_swiglu(s, lay["w13"][idx[t, j], 0], lay["w13"][idx[t, j], 1],
                                          lay["w2"][idx[t, j]], x[t]) for j in range(s.k))
        ref = ref + _torch_swiglu(s, lay["ws13"][0, 0], lay["ws13"][0, 1], lay["ws2"][0], x[t])
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-12)
