"""GPU verification round (moe_verify_gate) against the CPU oracle, through
the C ABI.  Decisions are exact on both sides, so n_accepted and the tokens
must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from speculative_decode_verify_gate_amd import binding as B

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _dists(rng, rows, V, peaked):
    """rows x V probability rows (fp32): Dirichlet-like from exponentials,
    optionally sharpened so argmaxes and acceptances vary."""
    e = rng.exponential(size=(rows, V))
    if peaked:
        e = e ** 4
    e /= e.sum(axis=1, keepdims=True)
    return e.astype(np.float32)


def _case(rng, S, gamma, V, mode):
    p = np.stack([_dists(rng, gamma + 1, V, peaked=True) for _ in range(S)])
    if mode == B.VERIFY_SAMPLING:
        q = np.stack([_dists(rng, gamma, V, peaked=True) for _ in range(S)])
        # drafted tokens drawn from the draft distributions
        def draw(row):
            w = row.astype(np.float64)
            return rng.choice(V, p=w / w.sum())
        x = np.array([[draw(q[s, i]) for i in range(gamma)] for s in range(S)],
                     dtype=np.int32).reshape(S, gamma)
        u = rng.random((S, gamma)).astype(np.float32)
        r = rng.integers(0, 2**32, S, dtype=np.uint64)
    else:
        q = u = r = None
        # about two thirds of the drafts are the verifier's argmax
        x = np.where(rng.random((S, gamma)) < 0.7, p[:, :gamma].argmax(axis=2),
                     rng.integers(0, V, (S, gamma))).astype(np.int32)
    return p, q, x, u, r


def _run_gpu(p, q, x, u, r, mode, ws=None):
    S = p.shape[0]
    dev = dict(p=torch.from_numpy(p).cuda(), x=torch.from_numpy(x).cuda().reshape(S, -1))
    if mode == B.VERIFY_SAMPLING:
        dev.update(q=torch.from_numpy(q).cuda(), u=torch.from_numpy(u).cuda(),
                   r=torch.from_numpy(r.astype(np.uint32).view(np.int32)).cuda())
    n, t = B.verify_gate(dev["p"], dev["x"], q=dev.get("q"), u=dev.get("u"), r=dev.get("r"),
                         mode=mode, ws=ws)
    torch.cuda.synchronize()
    return n.cpu().numpy(), t.cpu().numpy()


def _run_oracle(p, q, x, u, r, mode):
    S, G1, _ = p.shape
    ns, ts = [], []
    for s in range(S):
        n, t = O.verify_gate(p[s], x[s], q=None if q is None else q[s],
                             u=None if u is None else u[s], r=0 if r is None else int(r[s]),
                             mode=mode)
        ns.append(n)
        ts.append(t)
    return np.array(ns, np.int32), np.stack(ts).astype(np.int32)


@pytest.mark.parametrize("mode", [B.VERIFY_GREEDY, B.VERIFY_SAMPLING])
@pytest.mark.parametrize("S,gamma,V", [(1, 0, 5), (1, 1, 3), (4, 4, 1000), (2, 8, 2048),
                                       (3, 7, 4097), (4, 8, 102400), (2, 16, 152064),
                                       (1, 63, 300)])
def test_round_matches_oracle(S, gamma, V, mode):
    rng = np.random.default_rng(S * 1000 + gamma * 10 + V % 97 + mode)
    _say(f"[verify] mode={mode} S={S} gamma={gamma} V={V}")
    for rep in range(3):
        p, q, x, u, r = _case(rng, S, gamma, V, mode)
        n_g, t_g = _run_gpu(p, q, x, u, r, mode)
        n_o, t_o = _run_oracle(p, q, x, u, r, mode)
        np.testing.assert_array_equal(n_g, n_o)
        np.testing.assert_array_equal(t_g, t_o)


def test_worked_example():
    _say("[verify] worked example")
    p = np.array([[[0.3, 0.5, 0.2], [0.2, 0.3, 0.5]]], np.float32)
    q = np.array([[[0.6, 0.3, 0.1]]], np.float32)
    x = np.array([[0]], np.int32)
    for u, r, want_n, want0 in [(0.4999, 0, 1, 0), (0.5, 0, 0, 1), (0.5, 2**32 - 1, 0, 2)]:
        n, t = _run_gpu(p, q, x, np.array([[u]], np.float32), np.array([r], np.uint64),
                        B.VERIFY_SAMPLING)
        assert n[0] == want_n and t[0, 0] == want0


def test_zero_residual_draws_from_the_verifier():
    _say("[verify] zero residual")
    V = 4099
    rng = np.random.default_rng(9)
    row = _dists(rng, 1, V, peaked=False)[0]
    row[7] = 0.0
    row /= row.sum()
    p = np.stack([row, _dists(rng, 1, V, False)[0]])[None].astype(np.float32)
    q = row[None, None].copy()
    x = np.array([[7]], np.int32)   # q(x) = 0: rejected; p = q: residual zero
    for r in (0, 12345, 2**31, 2**32 - 1):
        args = (p, q, x, np.array([[0.0]], np.float32), np.array([r], np.uint64))
        n_g, t_g = _run_gpu(*args, B.VERIFY_SAMPLING)
        n_o, t_o = _run_oracle(*args, B.VERIFY_SAMPLING)
        assert n_g[0] == n_o[0] == 0
        assert t_g[0, 0] == t_o[0, 0] == O.sample_index(row, r)


def test_all_accepted_gives_the_bonus_token_and_workspace_is_reusable():
    _say("[verify] full acceptance, workspace reuse")
    rng = np.random.default_rng(4)
    S, gamma, V = 4, 6, 5000
    p = np.stack([_dists(rng, gamma + 1, V, True) for _ in range(S)])
    q = p[:, :gamma].copy()                           # p = q: every draft kept
    x = p[:, :gamma].argmax(axis=2).astype(np.int32)
    ws = B.Workspace()
    for rep in range(5):
        u = rng.random((S, gamma)).astype(np.float32)
        r = rng.integers(0, 2**32, S, dtype=np.uint64)
        n_g, t_g = _run_gpu(p, q, x, u, r, B.VERIFY_SAMPLING, ws=ws)
        n_o, t_o = _run_oracle(p, q, x, u, r, B.VERIFY_SAMPLING)
        assert (n_g == gamma).all()
        np.testing.assert_array_equal(t_g, t_o)
        # the arrival counters at the head of the workspace are back to zero
        assert int(ws.buf[:256].cpu().count_nonzero()) == 0


def test_out_of_vocabulary_draft_token_is_rejected():
    _say("[verify] out-of-vocabulary draft token")
    rng = np.random.default_rng(6)
    S, gamma, V = 2, 5, 3000
    p = np.stack([_dists(rng, gamma + 1, V, True) for _ in range(S)])
    x = p[:, :gamma].argmax(axis=2).astype(np.int32)
    bad = x.copy()
    bad[:, 2] = V + 5
    n_g, t_g = _run_gpu(p, None, bad, None, None, B.VERIFY_GREEDY)
    # the same round with an in-vocabulary token that is not the argmax
    alt = x.copy()
    alt[:, 2] = (x[:, 2] + 1) % V
    n_o, t_o = _run_oracle(p, None, alt, None, None, B.VERIFY_GREEDY)
    assert (n_g == 2).all()
    np.testing.assert_array_equal(n_g, n_o)
    np.testing.assert_array_equal(t_g, t_o)


def test_draw_without_weight_gives_no_token():
    # a bonus row of zeros (not a distribution) has nothing to draw: -1, as
    # in the oracle
    _say("[verify] empty bonus row")
    p = np.zeros((1, 2, 5000), np.float32)
    p[0, 0, 3] = 1.0
    q = p[:, :1].copy()
    x = np.array([[3]], np.int32)
    args = (p, q, x, np.array([[0.5]], np.float32), np.array([99], np.uint64))
    n_g, t_g = _run_gpu(*args, B.VERIFY_SAMPLING)
    n_o, t_o = _run_oracle(*args, B.VERIFY_SAMPLING)
    assert n_g[0] == n_o[0] == 1
    np.testing.assert_array_equal(t_g, t_o)
    assert t_g[0, 1] == -1
