"""GPU verification round (moe_verify_gate) against the CPU oracle, through
the C ABI.  Decisions are exact on both sides, so n_accepted and the tokens
must match bit for bit."""
import math

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


# ------------------------------------------------ logits -> filtered distributions

FILTER_TOL = 2e-5  # relative: what fp32 softmax arithmetic can move a probability by


def _check_nucleus(got, lg, T, top_p):
    """The GPU's filtered rows against the exact (fp64) softmax: its kept set
    differs from the oracle's only by near-ties of the boundary probability,
    is itself a valid nucleus up to the tolerance (its exact mass reaches
    top_p, and would not without its smallest member), and its values are
    the exact probabilities renormalised over it."""
    full, _ = O.filter_probs(lg, T, 1.0)
    ref, _ = O.filter_probs(lg, T, top_p)
    for g, f, r in zip(got.reshape(-1, lg.shape[-1]), full.reshape(-1, lg.shape[-1]),
                       ref.reshape(-1, lg.shape[-1])):
        kg, ko = g > 0, r > 0
        diff = kg ^ ko
        last = f[ko].min()
        assert np.all(np.abs(f[diff] - last) <= FILTER_TOL * last), "nuclei differ beyond near-ties"
        mass = f[kg].sum()
        if top_p < 1:
            assert mass >= top_p * (1 - FILTER_TOL), "GPU nucleus below top_p"
            assert mass - f[kg].min() < top_p * (1 + FILTER_TOL), "GPU nucleus not minimal"
        np.testing.assert_allclose(g[kg], f[kg] / mass, rtol=FILTER_TOL, atol=1e-12)
        assert abs(g.sum() - 1.0) < 1e-4


def _logit_rows(rng, rows, V, ties=False, masked=False):
    lg = (rng.standard_normal((rows, V)) * rng.uniform(0.5, 4.0, (rows, 1))).astype(np.float32)
    if ties:
        lg[:, : V // 4] = lg[:, :1]
    if masked:
        lg[rng.random((rows, V)) < 0.05] = -np.inf
        lg[:, 0] = 1.0
    return lg


@pytest.mark.parametrize("V", [1, 5, 1000, 4099, 102400, 152064])
@pytest.mark.parametrize("T,top_p", [(1.0, 1.0), (0.7, 0.9), (1.3, 0.5), (0.3, 0.95)])
def test_filter_matches_oracle(V, T, top_p):
    rng = np.random.default_rng(V + int(T * 100) + int(top_p * 1000))
    _say(f"[filter] V={V} T={T} top_p={top_p}")
    rows = 6 if V > 10000 else 12
    for ties, masked in ((False, False), (True, False), (False, True)):
        lg = _logit_rows(rng, rows, V, ties, masked)
        got = B.verify_probs(torch.from_numpy(lg).cuda(), T, top_p).cpu().numpy()
        _check_nucleus(got, lg, T, top_p)
        if ties:
            # exact ties are decided by index on both sides: same kept set
            ref, _ = O.filter_probs(lg, T, top_p)
            f, _ = O.filter_probs(lg, T, 1.0)
            for g, r, fr in zip(got, ref, f):
                if np.count_nonzero(fr == fr[0]) > 1 and r[0] > 0 and (r > 0).sum() < V:
                    tied = fr == fr[0]
                    np.testing.assert_array_equal(g[tied] > 0, r[tied] > 0)


def test_filter_more_workgroups_than_the_chip_holds_at_once():
    # 300 rows x 8 chunks = 2,400 workgroups per launch, more than are
    # resident at once: late workgroups of a launch must still start from
    # the selection state of the launch before
    rng = np.random.default_rng(41)
    rows, V = 300, 32000
    _say(f"[filter] rows={rows} V={V}")
    lg = _logit_rows(rng, rows, V, ties=False, masked=True)
    got = B.verify_probs(torch.from_numpy(lg).cuda(), 0.8, 0.9).cpu().numpy()
    _check_nucleus(got, lg, 0.8, 0.9)


@pytest.mark.parametrize("V,top_p", [(102400, 0.9), (4099, 0.5), (129280, 1.0), (129280, 0.9),
                                     (32000, 0.95)])
def test_filter_one_launch_equals_four_launches(V, top_p):
    """The same rows filtered in a call of more than FILTER_ONE_LAUNCH_ROWS
    rows (four launches), in calls of 16 rows (at most 512 workgroups, which
    the chip holds at once: one launch whose workgroups meet at row
    barriers) and in a call of 68 rows (at V = 102,400 and 129,280 two
    chunks per workgroup): bit for bit the same, with rows whose boundary bin holds long candidate lists (radix
    resolve) among them; no call writes the workspace head."""
    R = B.FILTER_ONE_LAUNCH_ROWS
    rng = np.random.default_rng(V + int(top_p * 100) + 7)
    _say(f"[filter] one launch vs four, V={V} top_p={top_p}")
    lg = _logit_rows(rng, R + 8, V, ties=True)
    lg[3, : V // 3] = lg[3, :1]                    # a third of the row tied
    lg[5] = 1.5                                    # every entry tied
    lg[R + 2] = np.round(lg[R + 2] * 4) / 4        # many small tie groups
    lg[R + 4, : V // 2] = -np.inf                  # half masked
    dev = torch.from_numpy(lg).cuda()
    ws = B.Workspace()
    four = B.verify_probs(dev, 0.7, top_p, ws=ws).clone()
    torch.cuda.synchronize()
    assert int(ws.buf[:256].count_nonzero()) == 0
    for r0 in range(0, R + 8, 16):
        one = B.verify_probs(dev[r0:r0 + 16], 0.7, top_p, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.buf[:256].count_nonzero()) == 0
        assert torch.equal(four[r0:r0 + 16].view(torch.int32), one.view(torch.int32)), r0
    # 68 rows: at V = 102,400, 1,700 one-chunk workgroups, more than the
    # one-launch kernel holds at six per CU (two chunks per workgroup take
    # them)
    one = B.verify_probs(dev[:68], 0.7, top_p, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(four[:68].view(torch.int32), one.view(torch.int32))
    _check_nucleus(four[:8].cpu().numpy(), lg[:8], 0.7, top_p)


@pytest.mark.parametrize("top_p", [0.9, 1.0])
def test_filter_two_chunks_per_workgroup(top_p):
    """32 rows of 63 chunks minus a ragged tail (2,016 workgroups at one
    chunk each, more than either one-chunk kernel holds at once): one launch
    with two chunks per workgroup, the last workgroup of each row holding
    one, bit for bit what the four launches of a 136-row call give, with
    tied rows (long candidate lists) among them."""
    V = 63 * 4096 - 100
    rng = np.random.default_rng(63 + int(top_p * 10))
    _say(f"[filter] two chunks per workgroup, V={V} top_p={top_p}")
    lg = _logit_rows(rng, B.FILTER_ONE_LAUNCH_ROWS + 8, V, masked=True)
    lg[1, : V // 2] = lg[1, :1]                    # a long candidate list
    lg[4] = 0.25                                   # every entry tied
    lg[7, 4096:] = -np.inf                         # all mass in the first chunk
    lg[9, : V - 50] = -np.inf                      # all mass in the last one
    dev = torch.from_numpy(lg).cuda()
    ws = B.Workspace()
    four = B.verify_probs(dev, 0.8, top_p, ws=ws).clone()
    for r0 in (0, 32):
        one = B.verify_probs(dev[r0:r0 + 32], 0.8, top_p, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.buf[:256].count_nonzero()) == 0
        assert torch.equal(four[r0:r0 + 32].view(torch.int32), one.view(torch.int32)), r0
    _check_nucleus(four[:10].cpu().numpy(), lg[:10], 0.8, top_p)


@pytest.mark.parametrize("rows,V", [(36, 102400), (68, 129280)])
def test_filter_barrier_timeout_writes_nan_and_ends(rows, V):
    """The one-launch filter's failure path, forced from the host: with the
    row barriers' waits cut to one poll, workgroups give up while the row's
    others are still on their way.  Some must: the bin a workgroup waits for
    after its histogram can only be handed out after the first workgroup has
    seen that workgroup's flag and summed every slot, several memory round
    trips after the one poll.  The call still ends, each 4096-entry chunk of
    the output is either NaN throughout (its workgroup gave up) or bit for
    bit the normal result, the workspace head stays zero, and with the
    default limit back the next call (a new tag, nothing cleared) is exact
    again."""
    rng = np.random.default_rng(rows)
    _say(f"[filter] barrier time-out, rows={rows} V={V}")
    lg = torch.from_numpy(_logit_rows(rng, rows, V, masked=True)).cuda()
    ws = B.Workspace()
    ref = B.verify_probs(lg, 0.7, 0.9, ws=ws).clone()
    torch.cuda.synchronize()
    try:
        B.filter_spin_limit(1)
        got = B.verify_probs(lg, 0.7, 0.9, ws=ws).clone()
        torch.cuda.synchronize()
    finally:
        B.filter_spin_limit(0)
    assert int(ws.buf[:256].count_nonzero()) == 0
    g, r = got.cpu().numpy(), ref.cpu().numpy()
    n_nan = 0
    for row in range(rows):
        for c0 in range(0, V, 4096):
            gc, rc = g[row, c0:c0 + 4096], r[row, c0:c0 + 4096]
            isn = np.isnan(gc)
            if isn.any():
                assert isn.all(), (row, c0)
                n_nan += 1
            else:
                np.testing.assert_array_equal(gc.view(np.int32), rc.view(np.int32))
    _say(f"   {n_nan} of {rows * ((V + 4095) // 4096)} chunks gave up")
    assert n_nan > 0
    again = B.verify_probs(lg, 0.7, 0.9, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int32), ref.view(torch.int32))


def test_filter_one_launch_at_the_longest_vocabulary():
    """FILTER_ONE_LAUNCH_VOCAB entries (64 workgroups per row, each reading
    every chunk's statistics and candidate count): 8 rows in one launch,
    bit for bit what the four launches of a 129-row call give them."""
    V = B.FILTER_ONE_LAUNCH_VOCAB
    rng = np.random.default_rng(42)
    _say(f"[filter] one launch, V={V}")
    lg = _logit_rows(rng, B.FILTER_ONE_LAUNCH_ROWS + 1, V, masked=True)
    lg[2, : V // 2] = lg[2, :1]                    # a long candidate list
    dev = torch.from_numpy(lg).cuda()
    ws = B.Workspace()
    four = B.verify_probs(dev, 0.8, 0.9, ws=ws).clone()
    one = B.verify_probs(dev[:8], 0.8, 0.9, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(four[:8].view(torch.int32), one.view(torch.int32))


def test_filter_all_tied_rows():
    # every token of the row tied: all V entries are candidates at the
    # boundary and the index cut decides; the kept set is the first k
    # indices, k within one token of the oracle's (exact integer masses
    # against the oracle's fp64 running sum)
    V = 102400
    lg = np.zeros((3, V), np.float32)
    lg[1] = 2.5
    lg[2, V // 2:] = -np.inf                      # half masked, the rest tied
    for top_p in (0.3, 0.77):
        _say(f"[filter] all tied, top_p={top_p}")
        got = B.verify_probs(torch.from_numpy(lg).cuda(), 1.0, top_p).cpu().numpy()
        ref, _ = O.filter_probs(lg, 1.0, top_p)
        _check_nucleus(got, lg, 1.0, top_p)
        for g, r in zip(got, ref):
            k = int(np.count_nonzero(g))
            assert np.all(g[:k] > 0) and abs(k - int(np.count_nonzero(r))) <= 1


MASS_ATOL = 1e-6  # absolute: what fp32 probabilities can move a running mass by


def _check_nucleus_mass(got, lg, T, top_p):
    """For top_p so close to 1 that the boundary lies where single tokens
    weigh less than the fp32 rounding of the running mass: the GPU's kept
    set is a prefix of the exact order up to near-ties, its exact mass
    reaches top_p and is minimal within MASS_ATOL, and its values are the
    exact probabilities renormalised over it."""
    full, _ = O.filter_probs(lg, T, 1.0)
    for g, f in zip(got.reshape(-1, lg.shape[-1]), full.reshape(-1, lg.shape[-1])):
        kg = g > 0
        assert f[kg].min() >= f[~kg].max() * (1 - FILTER_TOL) if (~kg).any() else True
        mass = f[kg].sum()
        assert mass >= top_p - MASS_ATOL and mass - f[kg].min() < top_p + MASS_ATOL
        np.testing.assert_allclose(g[kg], f[kg] / mass, rtol=FILTER_TOL, atol=1e-12)


@pytest.mark.parametrize("T,top_p", [(0.01, 0.9), (50.0, 0.9), (1.0, 1e-6), (0.05, 0.999),
                                     (1.0, 1 - 1e-7)])
def test_filter_degenerate_settings(T, top_p):
    # a near one-hot softmax, a near-flat one, a nucleus of one token and a
    # nucleus of (almost) everything
    rng = np.random.default_rng(int(T * 100) + int(top_p * 1e6))
    _say(f"[filter] degenerate T={T} top_p={top_p}")
    lg = _logit_rows(rng, 6, 50000)
    got = B.verify_probs(torch.from_numpy(lg).cuda(), T, top_p).cpu().numpy()
    if top_p > 1 - 1e-5:
        _check_nucleus_mass(got, lg, T, top_p)
    else:
        _check_nucleus(got, lg, T, top_p)
    if top_p == 1e-6:
        assert np.all(np.count_nonzero(got, axis=1) == 1)
        assert np.array_equal(got.argmax(axis=1), lg.argmax(axis=1))


def test_filter_unaligned_rows_and_single_finite_logits():
    # rows that start 4 bytes past a 16-byte boundary (the scalar load path
    # although V is a multiple of 4), a row with one finite logit, and a row
    # with two equal finite logits (the lower index alone reaches 0.5)
    rng = np.random.default_rng(47)
    rows, V = 5, 4096 * 3
    flat = torch.empty(rows * V + 1, dtype=torch.float32, device="cuda")
    lg = _logit_rows(rng, rows, V)
    lg[3] = -np.inf
    lg[3, 1234] = 0.0
    lg[4] = -np.inf
    lg[4, 100] = lg[4, 9000] = 2.0
    dev = flat[1:].view(rows, V)
    dev.copy_(torch.from_numpy(lg))
    assert dev.data_ptr() % 16 == 4
    out = torch.empty(rows * V + 1, dtype=torch.float32, device="cuda")[1:].view(rows, V)
    got = B.verify_probs(dev, 0.8, 0.5, out=out).cpu().numpy()
    _check_nucleus(got[:3], lg[:3], 0.8, 0.5)
    assert got[3, 1234] == 1.0 and np.count_nonzero(got[3]) == 1
    assert got[4, 100] == 1.0 and np.count_nonzero(got[4]) == 1
    # the same with top_p = 1: both tied tokens share the mass
    full = B.verify_probs(dev, 0.8, 1.0, out=out).cpu().numpy()
    assert full[4, 100] == full[4, 9000] == 0.5


def _exact_nucleus(P, top_p):
    """The filter's decision written out on given fp32 probabilities P
    [V]: integer masses floor(P 2^52), target ceil(top_p W) in fp64 with
    top_p as the fp32 the call takes, the order (P descending, index
    ascending), the first prefix whose mass reaches the target, and the kept
    entries divided by that mass in fp32."""
    m = np.floor(P.astype(np.float64) * 2.0 ** 52).astype(np.uint64)
    W = int(m.sum(dtype=np.uint64))
    target = max(1, math.ceil(float(np.float32(top_p)) * float(W)))
    order = np.lexsort((np.arange(P.size), -P))
    run = np.cumsum(m[order], dtype=np.uint64)
    last = int(np.searchsorted(run, np.uint64(target), side="left"))
    total = np.float32(float(run[last]) / 2.0 ** 52)
    out = np.zeros_like(P)
    keep = order[: last + 1]
    out[keep] = P[keep] / total
    return out


def test_filter_decision_is_exact_on_its_own_probabilities():
    """The kept set and values are exactly what the filter's integer-mass
    rule gives on the fp32 probabilities the same library computes without
    top-p (the same expression, the same row max and sum): bit for bit,
    whether the row's boundary bin holds a few candidates (ranked directly)
    or many (radix selection: long runs of exact ties)."""
    rng = np.random.default_rng(53)
    V = 102400
    lg = _logit_rows(rng, 8, V)
    lg[4:6, : V // 3] = lg[4:6, :1]                # a third of the row tied
    lg[6] = 1.5                                    # every entry tied
    lg[7] = np.round(lg[7] * 4) / 4                # many small tie groups
    dev = torch.from_numpy(lg).cuda()
    for T, top_p in ((0.7, 0.9), (1.0, 0.5), (0.3, 0.95), (1.0, 0.3)):
        _say(f"[filter] exact decision T={T} top_p={top_p}")
        P = B.verify_probs(dev, T, 1.0).cpu().numpy()
        got = B.verify_probs(dev, T, top_p).cpu().numpy()
        for r in range(lg.shape[0]):
            want = _exact_nucleus(P[r], top_p)
            np.testing.assert_array_equal(got[r].view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("V,top_p", [(102400, 0.9), (129280, 0.9), (4099, 0.5), (1000, 1.0),
                                     (32000, 0.95)])
def test_filter_pair_equals_two_single_calls(V, top_p):
    """moe_verify_probs_pair filters the verifier's and the draft's rows in
    one launch sequence: bit for bit what two moe_verify_probs calls give,
    also with a ragged vocabulary (scalar loads), row sets of different
    sizes, and one workspace shared with the single calls."""
    rng = np.random.default_rng(V + int(top_p * 100))
    _say(f"[filter] pair V={V} top_p={top_p}")
    lp = torch.from_numpy(_logit_rows(rng, 9, V, ties=True)).cuda()
    lq = torch.from_numpy(_logit_rows(rng, 5, V, masked=True)).cuda()
    ws = B.Workspace()
    p1 = B.verify_probs(lp, 0.7, top_p, ws=ws).clone()
    q1 = B.verify_probs(lq, 0.7, top_p, ws=ws).clone()
    p2, q2 = B.verify_probs_pair(lp, lq, 0.7, top_p, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(p1.view(torch.int32), p2.view(torch.int32))
    assert torch.equal(q1.view(torch.int32), q2.view(torch.int32))
    # the draft's rows first this time: the same bits again
    q3, p3 = B.verify_probs_pair(lq, lp, 0.7, top_p, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(p1.view(torch.int32), p3.view(torch.int32))
    assert torch.equal(q1.view(torch.int32), q3.view(torch.int32))


def test_filter_nucleus_hand_computed():
    lg = np.log(np.array([[0.2, 0.5, 0.3], [0.2, 0.5, 0.3], [0.2, 0.5, 0.3]], np.float32))
    cases = [(0.45, [0, 1, 0]), (0.7, [0, 0.625, 0.375]), (0.81, [0.2, 0.5, 0.3])]
    for top_p, want in cases:
        got = B.verify_probs(torch.from_numpy(lg).cuda(), 1.0, top_p).cpu().numpy()
        np.testing.assert_allclose(got, np.array([want] * 3), atol=1e-6)
    # ties: the lower indices first
    got = B.verify_probs(torch.tensor([[1.0, 1.0, 1.0, 0.0]], device="cuda"), 1.0, 0.5)
    np.testing.assert_allclose(got.cpu().numpy(), [[0.5, 0.5, 0, 0]], atol=1e-7)


def test_greedy_round_reads_logits_directly():
    """Greedy mode uses only each row's argmax, which softmax, temperature
    and top-p keep: the round on the raw logits equals the round on the
    filtered distributions."""
    rng = np.random.default_rng(33)
    S, gamma, V = 4, 8, 50000
    vl = _logit_rows(rng, S * (gamma + 1), V, masked=True).reshape(S, gamma + 1, V)
    vl[0, 2, 7] = vl[0, 2, 11] = vl[0, 2].max() + 1.0      # a tie for the argmax
    x = np.where(rng.random((S, gamma)) < 0.7, vl[:, :gamma].argmax(axis=2),
                 rng.integers(0, V, (S, gamma))).astype(np.int32)
    p = B.verify_probs(torch.from_numpy(vl).cuda(), 0.7, 0.9).cpu().numpy()
    n_l, t_l = _run_gpu(vl, None, x, None, None, B.VERIFY_GREEDY)
    n_p, t_p = _run_gpu(p, None, x, None, None, B.VERIFY_GREEDY)
    np.testing.assert_array_equal(n_l, n_p)
    np.testing.assert_array_equal(t_l, t_p)
    assert (np.argmax(vl[0, 2]) == 7) and (7 in t_l[0] or n_l[0] < 2)


def test_greedy_argmax_signed_zeros_tie():
    """-0.0 and +0.0 are equal values: where a row's maximum is zero and
    occurs as both, the argmax is the lower index, whichever sign it has
    (across chunks and inside one chunk)."""
    V = 5000
    vl = np.full((1, 3, V), -1.0, dtype=np.float32)
    vl[0, 0, 100], vl[0, 0, 4000] = -0.0, 0.0      # different 2048-entry chunks
    vl[0, 1, 10], vl[0, 1, 11] = -0.0, 0.0         # one chunk
    vl[0, 2, 7], vl[0, 2, 3000] = 0.0, -0.0        # +0 first
    for x0, x1 in ((100, 10), (4000, 11)):
        x = np.array([[x0, x1]], dtype=np.int32)
        n_g, t_g = _run_gpu(vl, None, x, None, None, B.VERIFY_GREEDY)
        n_o, t_o = _run_oracle(vl, None, x, None, None, B.VERIFY_GREEDY)
        np.testing.assert_array_equal(n_g, n_o)
        np.testing.assert_array_equal(t_g, t_o)
    assert list(t_g[0]) == [100, -1, -1] and n_g[0] == 0


def test_round_from_logits_matches_oracle():
    """Logits -> filtered p and q on the GPU -> the GPU round; the oracle's
    round on those same distributions decides identically."""
    rng = np.random.default_rng(31)
    S, gamma, V, T, top_p = 4, 6, 32000, 0.7, 0.9
    vl = _logit_rows(rng, S * (gamma + 1), V).reshape(S, gamma + 1, V)
    dl = (vl[:, :gamma] + 0.5 * rng.standard_normal((S, gamma, V))).astype(np.float32)
    p = B.verify_probs(torch.from_numpy(vl).cuda(), T, top_p)
    q = B.verify_probs(torch.from_numpy(dl).cuda(), T, top_p)
    qn = q.cpu().numpy()
    x = np.array([[rng.choice(V, p=qn[s, i].astype(np.float64) / qn[s, i].astype(np.float64).sum())
                   for i in range(gamma)] for s in range(S)], dtype=np.int32)
    u = rng.random((S, gamma)).astype(np.float32)
    r = rng.integers(0, 2**32, S, dtype=np.uint64)
    n_g, t_g = _run_gpu(p.cpu().numpy(), qn, x, u, r, B.VERIFY_SAMPLING)
    n_o, t_o = _run_oracle(p.cpu().numpy(), qn, x, u, r, B.VERIFY_SAMPLING)
    np.testing.assert_array_equal(n_g, n_o)
    np.testing.assert_array_equal(t_g, t_o)
    # every kept or drawn token lies in the verifier's nucleus
    pn = p.cpu().numpy()
    for s in range(S):
        for i in range(n_g[s] + 1):
            tok = t_g[s, i]
            if tok >= 0:
                assert pn[s, min(i, gamma)][tok] > 0 or i < n_g[s]
