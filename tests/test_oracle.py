"""Pins for the CPU oracle, each against something other than the oracle:
library routines (torch / numpy / itertools), closed forms, invariants the
pages fix, special cases, and brute force on tiny inputs.

Sources: "Deep Dive into Mixture of Experts: From 1991 to DeepSeek-V3"
(sections 1, 2 and 5: dense mixture, top-k sparse gating, shared experts) and
"Speculative Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel
Bandwidth and the Best Draft Length" (abstract: per-slot vs dedup bytes).
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
from speculative_decode_verify_gate_amd import synth


def _rng(seed):
    return np.random.default_rng(seed)


def _layer_np(shape, seed, E=None):
    """Small random layer as host numpy arrays (bf16 as uint16 bits)."""
    E = shape.E if E is None else E
    g = torch.Generator().manual_seed(seed)
    tdt = torch.bfloat16 if shape.wdtype == O.BF16 else torch.float32

    def draw(*sz):
        return (torch.randn(sz, generator=g) * 0.3).to(tdt)

    lay = dict(gate_w=(torch.randn((E, shape.d), generator=g)).numpy(),
               w13=draw(E, 2, shape.f, shape.d), w2=draw(E, shape.d, shape.f),
               ws13=draw(shape.S, 2, shape.f, shape.d) if shape.S else None,
               ws2=draw(shape.S, shape.d, shape.f) if shape.S else None)
    for key in ("w13", "w2", "ws13", "ws2"):
        lay[key] = synth.to_host_bits(lay[key])
    return lay


def _as_f64(shape, a):
    if shape.wdtype == O.BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _torch_swiglu(shape, W1, W3, W2, x):
    """SwiGLU FFN with torch's own matmul / silu / bf16 casts (library
    routines), rounding points as in the bf16 reading."""
    W1, W3, W2 = (torch.from_numpy(_as_f64(shape, a)) for a in (W1, W3, W2))
    xt = torch.from_numpy(np.asarray(x, dtype=np.float32))
    if shape.wdtype == O.BF16:
        xt = xt.to(torch.bfloat16)
    xt = xt.double()
    a = torch.nn.functional.silu(xt @ W1.T) * (xt @ W3.T)
    if shape.wdtype == O.BF16:
        a = a.float().to(torch.bfloat16)
    return (a.double() @ W2.T).numpy()


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rne_matches_torch_cast():
    rng = _rng(1)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45],
                 dtype=np.float32),
    ])
    # exact ties: the dropped 16 bits equal 0x8000, both even and odd kept lsb
    hi = rng.standard_normal(1000).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (hi | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([vals, ties])
    ours = O.bf16_rne(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_ties_to_even_closed_form():
    # 1 + 2^-8 lies halfway between bf16 1.0 (0x3F80) and 1+2^-7 (0x3F81)
    assert O.bf16_rne(np.float32(1.0 + 2**-8))[()] == 0x3F80
    # 1 + 3*2^-8 lies halfway between 0x3F81 (odd) and 0x3F82 (even)
    assert O.bf16_rne(np.float32(1.0 + 3 * 2**-8))[()] == 0x3F82
    assert O.bf16_rne(np.float32(np.nan))[()] & 0x7FC0 == 0x7FC0


def _bf16_grid():
    """Every finite non-negative bf16 value as an exact fraction, ascending,
    with its bit pattern; 2^128 (the infinity pattern) closes the grid, as
    IEEE overflow rounding treats it."""
    from fractions import Fraction
    pats = np.arange(0, 0x7F81, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    grid = [Fraction(float(v)) for v in vals[:-1]] + [Fraction(2) ** 128]
    return grid, pats


def _exact_nearest_even(v, grid, pats):
    """bf16 pattern nearest to the double v, ties to the even pattern, by
    exact comparison against the whole grid (bisection)."""
    import bisect
    from fractions import Fraction
    if v != v:
        return None
    sign = 0x8000 if np.signbit(v) else 0
    if np.isinf(v) or Fraction(abs(float(v))) >= grid[-1]:
        return sign | 0x7F80
    a = Fraction(abs(float(v)))
    i = bisect.bisect_left(grid, a)
    if i < len(grid) and grid[i] == a:
        return sign | int(pats[i])
    lo, hi = i - 1, i
    dlo, dhi = a - grid[lo], grid[hi] - a
    if dlo < dhi or (dlo == dhi and pats[lo] % 2 == 0):
        return sign | int(pats[lo])
    return sign | int(pats[hi])


def test_bf16_rne_f64_is_the_exact_nearest_even():
    """One-step fp64 -> bf16 rounding against exact arithmetic on the whole
    bf16 grid: random doubles over the normal and subnormal bf16 ranges and
    beyond its largest value, doubles a hair off and exactly on midpoints
    (the fp32 rounding of a double can land on a midpoint that the double
    itself is not on), signed zeros and infinities."""
    from fractions import Fraction
    grid, pats = _bf16_grid()
    rng = _rng(12)
    vals = [float(v) for v in rng.standard_normal(1500)]
    vals += [float(v) for v in rng.standard_normal(300) * 2.0 ** rng.integers(-140, -120, 300)]
    vals += [float(v) for v in rng.standard_normal(200) * 2.0 ** 127]
    mids = rng.integers(1, 0x7F7F, 600)
    for p_ in mids:
        m = (grid[p_] + grid[p_ + 1]) / 2
        for rel in (0.0, 2.0 ** -30, -(2.0 ** -30), 2.0 ** -52, -(2.0 ** -52)):
            vals.append(float(m * (1 + Fraction(rel))))
    vals += [0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, 3.4e38, 2.0 ** -133,
             2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -140]
    ours = O.bf16_rne_f64(np.array(vals, dtype=np.float64))
    for v, got in zip(vals, ours):
        assert int(got) == _exact_nearest_even(v, grid, pats), v
    assert O.bf16_rne_f64(np.float64(np.nan))[()] & 0x7FC0 == 0x7FC0


def test_bf16_rne_f64_rounds_once_not_through_fp32():
    """1 + 2^-8 + 2^-30 lies just above the midpoint of bf16 1.0 and 1 + 2^-7,
    so its nearest bf16 is 1 + 2^-7 (0x3F81).  Its fp32 rounding is the
    midpoint itself, which then ties to the even 1.0 (0x3F80): the oracle's
    activation rounding must take the first, single-step answer."""
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert O.bf16_rne_f64(np.float64(v))[()] == 0x3F81
    assert O.bf16_rne(np.float32(v))[()] == 0x3F80


# ---------------------------------------------------------------- gate + top-k

def test_gate_logits_match_numpy_matmul():
    s = O.Shape(d=48, E=12, k=3, f=32)
    rng = _rng(2)
    gw = rng.standard_normal((12, 48)).astype(np.float32)
    x = rng.standard_normal((5, 48)).astype(np.float32)
    L = O.gate_logits(s, gw, x)
    ref = x.astype(np.float64) @ gw.astype(np.float64).T
    assert np.allclose(L, ref, rtol=0, atol=1e-12)


def test_hand_checked_route_d2_e3_k2():
    # x = (1, 2); gate rows (1,0), (0,1), (1,1) -> logits 1, 2, 3.
    # top-2 = experts 2 then 1; weights softmax(3, 2) = (e, 1) / (e + 1).
    s = O.Shape(d=2, E=3, k=2, f=2)
    gw = np.array([[1, 0], [0, 1], [1, 1]], dtype=np.float32)
    x = np.array([[1, 2]], dtype=np.float32)
    r = O.route(s, gw, x)
    assert r["idx"].tolist() == [[2, 1]]
    assert np.allclose(r["w"], [[math.e / (math.e + 1), 1 / (math.e + 1)]], rtol=0, atol=1e-15)
    assert r["margin"][0] == pytest.approx(1.0)
    assert r["logits"].tolist() == [[1.0, 2.0, 3.0]]


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (256, 8), (8, 8), (5, 1)])
def test_topk_matches_stable_sort(E, k):
    s = O.Shape(d=64, E=E, k=k, f=32)
    rng = _rng(E * 10 + k)
    gw = rng.standard_normal((E, 64)).astype(np.float32)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    r = O.route(s, gw, x)
    key = torch.from_numpy(r["logits"].astype(np.float32))
    order = torch.sort(key, dim=1, descending=True, stable=True).indices[:, :k]
    assert np.array_equal(r["idx"], order.numpy().astype(np.int32))
    # softmax over the selected logits, by scipy-free closed form in numpy
    sel = np.take_along_axis(r["logits"], r["idx"].astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    assert np.allclose(r["w"], ex / ex.sum(axis=1, keepdims=True), rtol=0, atol=1e-14)
    # margin is the gap between the k-th and (k+1)-th largest logits
    srt = -np.sort(-r["logits"], axis=1)
    if k < E:
        assert np.allclose(r["margin"], srt[:, k - 1] - srt[:, k], atol=1e-12)
    else:
        assert np.all(np.isinf(r["margin"]))


def test_weights_sum_to_one_and_top1_is_exactly_one():
    rng = _rng(3)
    for E, k in [(8, 2), (64, 6), (256, 8)]:
        s = O.Shape(d=32, E=E, k=k, f=32)
        r = O.route(s, rng.standard_normal((E, 32)).astype(np.float32),
                    rng.standard_normal((20, 32)).astype(np.float32))
        assert np.allclose(r["w"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert np.all(r["w"] > 0) and np.all(np.diff(r["w"], axis=1) <= 0)
    s1 = O.Shape(d=32, E=16, k=1, f=32)
    r = O.route(s1, rng.standard_normal((16, 32)).astype(np.float32),
                rng.standard_normal((20, 32)).astype(np.float32))
    assert np.all(r["w"] == 1.0)
    assert np.array_equal(r["idx"][:, 0], np.argmax(r["logits"], axis=1))


def test_order_is_taken_on_the_fp64_logits():
    """Two logits that differ by 2^-40, far below fp32 resolution at 1: the
    larger one is selected first although its index is higher (an fp32
    comparison would see a tie and take the lower index), and the token is
    flagged, since its gap is under the near-tie threshold."""
    s = O.Shape(d=2, E=3, k=2, f=16)
    gw = np.array([[1.0, 0.0], [1.0, 1.0], [0.5, 0.0]], dtype=np.float32)
    x = np.array([[1.0, 2.0 ** -40]], dtype=np.float32)
    r = O.route(s, gw, x)
    assert r["logits"][0, 1] - r["logits"][0, 0] == 2.0 ** -40
    assert r["idx"].tolist() == [[1, 0]]
    assert r["flags"][0] & O.FLAG_ORDER and not r["flags"][0] & O.FLAG_BOUNDARY


def test_exact_ties_pick_lowest_index_and_are_flagged():
    s = O.Shape(d=16, E=6, k=2, f=16)
    rng = _rng(4)
    gw = rng.standard_normal((6, 16)).astype(np.float32)
    x = rng.standard_normal((8, 16)).astype(np.float32)
    L = x.astype(np.float64) @ gw.astype(np.float64).T
    best = np.argmax(L[0])
    # duplicate the best gate row into every other position: all logits of
    # expert `best` and its copies are equal for every token
    gw2 = gw.copy()
    gw2[:] = gw[best]
    r = O.route(s, gw2, x)
    assert np.all(r["idx"] == np.array([0, 1], dtype=np.int32))
    assert np.all(r["flags"] & O.FLAG_BOUNDARY)
    assert np.all(r["flags"] & O.FLAG_ORDER)
    assert np.allclose(r["w"], 0.5, rtol=0, atol=0)


def test_bruteforce_topk_on_quantised_logits():
    """Enumerate every k-subset: the selection is the max-sum subset, the one
    with the smallest indices among equal sums; logits are exact dyadic values
    so no rounding can reorder them."""
    rng = _rng(5)
    for trial in range(60):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        d = int(rng.integers(1, 17))
        N = int(rng.integers(1, 5))
        gw = (rng.integers(-2, 3, (E, d)) / 8.0).astype(np.float32)
        x = (rng.integers(-4, 5, (N, d)) / 4.0).astype(np.float32)
        s = O.Shape(d=d, E=E, k=k, f=4)
        r = O.route(s, gw, x)
        L = x.astype(np.float64) @ gw.astype(np.float64).T
        for t in range(N):
            best = None
            for sub in itertools.combinations(range(E), k):
                tot = sum(L[t, e] for e in sub)
                if best is None or tot > best[0]:
                    best = (tot, sub)
            assert sorted(r["idx"][t].tolist()) == list(best[1])
            vals = L[t, r["idx"][t]]
            assert np.all(np.diff(vals) <= 0)
            for j in range(k - 1):
                if vals[j] == vals[j + 1]:
                    assert r["idx"][t, j] < r["idx"][t, j + 1]


# ---------------------------------------------------------------- experts, layer

@pytest.mark.parametrize("wdtype", [O.F32, O.BF16])
def test_single_expert_matches_torch_swiglu(wdtype):
    s = O.Shape(d=32, E=1, k=1, f=48, S=0, wdtype=wdtype)   # f != d catches transposes
    lay = _layer_np(s, 6)
    x = _rng(6).standard_normal((3, 32)).astype(np.float32)
    idx = np.zeros((3, 1), dtype=np.int32)
    y, rb, sb, U = O.layer(s, lay["w13"], lay["w2"], None, None, x, idx, np.ones((3, 1)))
    ref = np.stack([_torch_swiglu(s, lay["w13"][0, 0], lay["w13"][0, 1], lay["w2"][0], x[t])
                    for t in range(3)])
    tol = 1e-12 if wdtype == O.F32 else 2e-3
    assert np.max(np.abs(y - ref)) <= tol * np.max(np.abs(ref))
    assert (rb, sb, U) == (3 * O.expert_bytes(s), 0, 1)


def test_top_k_equals_dense_mixture_when_k_is_E():
    for wdtype in (O.F32, O.BF16):
        s = O.Shape(d=24, E=5, k=5, f=40, S=1, wdtype=wdtype)
        lay = _layer_np(s, 7)
        x = _rng(7).standard_normal((4, 24)).astype(np.float32)
        r = O.route(s, lay["gate_w"], x)
        y, _, _, _ = O.layer(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x,
                             r["idx"], r["w"])
        yd = O.dense_mixture(s, lay["gate_w"], lay["w13"], lay["w2"], lay["ws13"],
                             lay["ws2"], x)
        assert np.max(np.abs(y - yd)) <= 1e-12 * np.max(np.abs(yd))


def test_layer_is_weighted_sum_of_torch_experts_plus_shared():
    s = O.Shape(d=32, E=6, k=2, f=24, S=2, wdtype=O.BF16)
    lay = _layer_np(s, 8)
    x = _rng(8).standard_normal((3, 32)).astype(np.float32)
    r = O.route(s, lay["gate_w"], x)
    y, rb, sb, U = O.layer(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x,
                           r["idx"], r["w"])
    for t in range(3):
        ref = np.zeros(32)
        for j in range(2):
            e = r["idx"][t, j]
            ref += r["w"][t, j] * _torch_swiglu(s, lay["w13"][e, 0], lay["w13"][e, 1],
                                                lay["w2"][e], x[t])
        for sh in range(2):
            ref += _torch_swiglu(s, lay["ws13"][sh, 0], lay["ws13"][sh, 1], lay["ws2"][sh], x[t])
        assert np.max(np.abs(y[t] - ref)) <= 2e-3 * np.max(np.abs(ref))
    assert sb == 2 * O.expert_bytes(s)


def test_perslot_and_dedup_identical_and_bytes():
    s = O.Shape(d=32, E=8, k=3, f=16, S=1, wdtype=O.BF16)
    lay = _layer_np(s, 9)
    x = _rng(9).standard_normal((7, 32)).astype(np.float32)
    r = O.route(s, lay["gate_w"], x)
    outs = {}
    for eng in ("perslot", "dedup"):
        for th in (1, 3):
            outs[(eng, th)] = O.layer(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x,
                                      r["idx"], r["w"], engine=eng, n_threads=th)
    y0 = outs[("perslot", 1)][0]
    for key, (y, rb, sb, U) in outs.items():
        assert np.array_equal(y, y0), key
    Be = O.expert_bytes(s)
    U = len(set(r["idx"].ravel().tolist()))
    assert outs[("perslot", 1)][1:] == (7 * 3 * Be, Be, U)
    assert outs[("dedup", 1)][1:] == (U * Be, Be, U)
    assert O.pass_bytes(s, r["idx"]) == (7 * 3 * Be, U * Be, Be, U)


def test_pass_bytes_bounds_and_single_token():
    rng = _rng(10)
    for E, k in [(8, 2), (64, 6), (256, 8)]:
        s = O.Shape(d=2048, E=E, k=k, f=1408, S=2)
        for N in (1, 2, 5, 16, 64):
            if N * k > 512:
                continue
            idx = np.stack([rng.choice(E, k, replace=False) for _ in range(N)]).astype(np.int32)
            ps, dd, sh, U = O.pass_bytes(s, idx)
            assert k <= U <= min(E, N * k)
            Be = 3 * 2048 * 1408 * 2
            assert (ps, dd, sh) == (N * k * Be, U * Be, 2 * Be)
            if N == 1:
                assert U == k and dd == ps
    # 64-bit counts: V3-shaped per-slot bytes exceed 2^32
    s3 = O.Shape(d=7168, E=256, k=8, f=2048, S=1)
    idx = np.tile(np.arange(8, dtype=np.int32), (64, 1))
    ps, dd, sh, U = O.pass_bytes(s3, idx)
    assert ps == 64 * 8 * 88080384 == 45097156608 and dd == 8 * 88080384 and U == 8


def test_equivariance_token_permutation_and_expert_relabelling():
    s = O.Shape(d=32, E=8, k=2, f=24, S=1, wdtype=O.BF16)
    lay = _layer_np(s, 11)
    x = _rng(11).standard_normal((6, 32)).astype(np.float32)
    r = O.route(s, lay["gate_w"], x)
    y, _, _, U = O.layer(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x, r["idx"], r["w"])
    perm = np.array([3, 0, 5, 1, 4, 2])
    rp = O.route(s, lay["gate_w"], x[perm])
    yp, _, _, Up = O.layer(s, lay["w13"], lay["w2"], lay["ws13"], lay["ws2"], x[perm],
                           rp["idx"], rp["w"])
    assert np.array_equal(rp["idx"], r["idx"][perm]) and np.array_equal(yp, y[perm]) and Up == U
    # relabel experts: new expert q is old expert pi[q]
    pi = np.array([5, 2, 7, 0, 1, 6, 3, 4])
    inv = np.argsort(pi)
    rr = O.route(s, lay["gate_w"][pi], x)
    assert np.array_equal(rr["idx"], inv[r["idx"]].astype(np.int32))
    yr, _, _, _ = O.layer(s, lay["w13"][pi], lay["w2"][pi], lay["ws13"], lay["ws2"], x,
                          rr["idx"], rr["w"])
    assert np.array_equal(yr, y)


def test_compaction_bruteforce_and_invariants():
    rng = _rng(12)
    for trial in range(40):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        N = int(rng.integers(1, 17))
        s = O.Shape(d=32, E=E, k=k, f=32)
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(N)]).astype(np.int32)
        c = O.compact(s, idx)
        flat = idx.ravel()
        assert sorted(c["list"].tolist()) == list(range(N * k))
        assert c["uniq"].tolist() == sorted(set(flat.tolist()))
        assert c["n_unique"] == len(set(flat.tolist()))
        for e in range(E):
            members = [i for i in range(N * k) if flat[i] == e]
            assert c["counts"][e] == len(members)
            assert c["list"][c["offs"][e]:c["offs"][e + 1]].tolist() == members
        assert c["offs"][E] == N * k


def test_oracle_rejects_bad_input():
    s = O.Shape(d=8, E=4, k=2, f=8)
    with pytest.raises(ValueError):
        O.pass_bytes(s, np.array([[0, 4]], dtype=np.int32))
    with pytest.raises(ValueError):
        O.route(O.Shape(d=8, E=4, k=5, f=8), np.zeros((4, 8), np.float32),
                np.zeros((1, 8), np.float32))


def test_uncorrelated_routing_unique_share_is_near_uniform_prediction():
    """Statistical sanity: with rho = 0 and random gates, the unique-expert
    count tracks E(1 - (1 - k/E)^N) (not exact: gate rows are not exchangeable)."""
    s = O.Shape(d=64, E=64, k=6, f=8)
    rng = _rng(13)
    gw = (rng.standard_normal((64, 64)) * 0.02).astype(np.float32)
    shares = []
    for rep in range(40):
        x = rng.standard_normal((16, 64)).astype(np.float32)
        r = O.route(s, gw, x)
        shares.append(len(set(r["idx"].ravel().tolist())) / (16 * 6))
    pred = 64 * (1 - (1 - 6 / 64) ** 16) / 96
    assert abs(np.mean(shares) - pred) < 0.08
