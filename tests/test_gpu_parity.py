"""GPU parity: the gfx950 library against the CPU oracle, through the C ABI.

Bars: routing indices and byte counts bit-exact (ties to the lower index;
tokens whose oracle margin or in-top-k gap is below 1e-4 are flagged and
exempt from the index comparison, and counted); gate logits within 1e-4
absolute; layer outputs within 1e-2 (bf16 weights, fp32 accumulation) or
1e-5 (fp32 weights) of max|y_ref|; per-slot and dedup outputs bitwise
identical.
"""
import numpy as np
import pytest
import torch

import oracle as O
from speculative_decode_verify_gate_amd import binding as B
from speculative_decode_verify_gate_amd import synth
from helpers import (LOGIT_ATOL, OUT_RTOL, TIE_EPS, WEIGHT_ATOL, host_layer, oracle_y,
                     oshape, rel_err, small_config, to_dev)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _check_route(cfg, gate_w_dev, x_dev, gate_w_np, x_np):
    shape = B.shape_of(cfg)
    n = x_dev.shape[0]
    logits = torch.empty((n, cfg.E), dtype=torch.float32, device="cuda")
    margin = torch.empty((n,), dtype=torch.float32, device="cuda")
    idx, w = B.route(shape, gate_w_dev, x_dev, logits=logits, margin=margin)
    torch.cuda.synchronize()
    ref = O.route(oshape(cfg), gate_w_np, x_np, tie_eps=TIE_EPS)
    assert np.max(np.abs(logits.cpu().numpy() - ref["logits"])) <= LOGIT_ATOL
    ok = ref["flags"] == 0
    gi = idx.cpu().numpy()
    assert np.array_equal(gi[ok], ref["idx"][ok]), "routing differs on an unflagged token"
    # flagged tokens still select a valid top-k of the GPU's own logits
    gw = w.cpu().numpy()
    assert np.all(np.abs(gw.sum(axis=1) - 1.0) <= 1e-6)
    assert np.all(np.abs(gw[ok] - ref["w"][ok]) <= WEIGHT_ATOL)
    if cfg.k < cfg.E:
        assert np.all(np.abs(margin.cpu().numpy()[ok] - ref["margin"][ok]) <= LOGIT_ATOL)
    for t in range(n):
        assert len(set(gi[t].tolist())) == cfg.k and gi[t].min() >= 0 and gi[t].max() < cfg.E
    return idx, w, ref, int((~ok).sum())


def _pack_numpy(W, step):
    """MOE_LAYOUT_TILED of one row-major [R][K] matrix, from the header's
    definition: fragment (rt, s) is 1 KB at (rt * K/step + s) * 1 KB; its
    16-byte unit L holds row 16 rt + L % 16, columns step*s + (L//16)*step/4."""
    R, K = W.shape
    q = step // 4
    n_s = K // step
    out = np.empty(R * K, W.dtype)
    for rt in range(R // 16):
        for s_ in range(n_s):
            base = (rt * n_s + s_) * 64 * q
            for L in range(64):
                c0 = step * s_ + (L // 16) * q
                out[base + L * q: base + (L + 1) * q] = W[16 * rt + L % 16, c0:c0 + q]
    return out


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_pack_matches_layout_definition(wdt):
    cfg = small_config("pack", 128, 3, 1, 96, 1, wdt)
    lay = synth.make_layer(cfg, "cpu")
    shape = B.shape_of(cfg)
    packed = B.pack_weights(shape, to_dev(lay))
    torch.cuda.synchronize()
    step = 32 if wdt == "bf16" else 16
    for key in ("w13", "w2", "ws13", "ws2"):
        src = synth.to_host_bits(lay[key])
        got = synth.to_host_bits(packed[key]).reshape(src.shape[0], -1)
        mats = src.reshape(-1, src.shape[-2], src.shape[-1])
        want = np.concatenate([_pack_numpy(m, step).reshape(-1) for m in mats])
        assert np.array_equal(got.reshape(-1), want), key


def _run_both(cfg, lay_dev, x_dev, idx_dev, w_dev):
    shape = B.shape_of(cfg)
    y_ps = B.expert_pass_perslot(shape, lay_dev, x_dev, idx_dev, w_dev)
    nu = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ws = B.Workspace()
    y_dd = B.expert_pass_dedup(shape, lay_dev, x_dev, idx_dev, w_dev, n_unique=nu, ws=ws)
    torch.cuda.synchronize()
    return y_ps, y_dd, int(nu.item()), ws


def _check_record(cfg, ws, idx):
    """The compaction record the dedup pass leaves from byte 256 of its
    workspace (the head belongs to arrival counters and stays zero), checked
    bit-exactly against the oracle's compaction of the same routing."""
    E, slots = cfg.E, idx.size
    c = O.compact(oshape(cfg), idx)
    assert int(ws.buf[:256].count_nonzero()) == 0
    rec = ws.buf[256: 256 + 4 * (3 * E + 2 + slots)].view(torch.int32).cpu().numpy()
    U = int(c["n_unique"])
    assert rec[0] == U
    assert np.array_equal(rec[1:1 + E], c["counts"])
    assert np.array_equal(rec[1 + E:2 + 2 * E], c["offs"])
    assert np.array_equal(rec[2 + 2 * E:2 + 2 * E + U], c["uniq"])
    assert np.array_equal(rec[2 + 3 * E:2 + 3 * E + slots], c["list"])


# ------------------------------------------------------------- small shapes

SMALL = [
    # name, d, E, k, f, S, wdtype  (f=192: row groups with a ragged tail)
    ("f32-ragged", 256, 8, 2, 192, 1, "f32"),
    ("bf16-ragged", 256, 8, 2, 192, 1, "bf16"),
    ("bf16-v2like", 512, 64, 6, 352, 2, "bf16"),
    ("bf16-top1", 256, 16, 1, 128, 0, "bf16"),
    ("bf16-single-expert", 128, 1, 1, 96, 0, "bf16"),
    # d = 160: 10 row tiles, not whole workgroups of eight, so the short
    # d_ff takes the four-waves-per-tile down kernel
    ("bf16-rows-in-tens", 160, 8, 2, 192, 1, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("n", [1, 3, 16, 17, 64])
def test_small_layer_parity(case, n):
    name, d, E, k, f, S, wdt = case
    if n * k > B.MAX_SLOTS:
        pytest.skip("beyond the slot limit")
    cfg = small_config(name, d, E, k, f, S, wdt)
    _say(f"[small] {name} n={n}")
    lay = synth.make_layer(cfg, "cpu")
    x = synth.make_hidden(cfg, n, 0, "cpu")
    host = host_layer(lay)
    x_np = x.numpy()
    lay_dev, x_dev = to_dev(lay), x.cuda()
    idx, w, ref, flagged = _check_route(cfg, lay_dev["gate_w"], x_dev, host["gate_w"], x_np)
    # the expert passes are compared on the oracle's routing, so that a
    # near-tie cannot move an output between experts
    idx_o = torch.from_numpy(ref["idx"]).cuda()
    w_o = torch.from_numpy(ref["w"].astype(np.float32)).cuda()
    y_ps, y_dd, U, ws = _run_both(cfg, lay_dev, x_dev, idx_o, w_o)
    y_ref, rb, sb, U_ref = oracle_y(cfg, host, x_np, ref["idx"], ref["w"].astype(np.float32))
    assert U == U_ref
    assert torch.equal(y_ps, y_dd), "per-slot and dedup outputs differ"
    # the tiled weight layout feeds the MFMA the same operands: same bits
    tiled = B.pack_weights(B.shape_of(cfg), lay_dev)
    y_ps_t, y_dd_t, U_t, _ = _run_both(cfg, tiled, x_dev, idx_o, w_o)
    assert U_t == U and torch.equal(y_ps_t, y_ps) and torch.equal(y_dd_t, y_dd)
    err = rel_err(y_ps.cpu().numpy(), y_ref)
    _say(f"   rel err {err:.3e}  U={U}  flagged={flagged}")
    assert err <= OUT_RTOL[wdt]
    _check_record(cfg, ws, ref["idx"])
    # byte counts: host library call vs oracle, bit-exact
    assert B.pass_bytes(B.shape_of(cfg), ref["idx"]) == O.pass_bytes(oshape(cfg), ref["idx"])


def test_dedup_heavy_expert_over_64_tokens():
    """One expert chosen by every token of a 64-token pass (m = 64) and by
    several slots of the same token (duplicates in a caller's routing)."""
    cfg = small_config("heavy", 256, 8, 4, 128, 1, "bf16")
    n = 64
    lay = synth.make_layer(cfg, "cpu")
    x = synth.make_hidden(cfg, n, 0, "cpu")
    host = host_layer(lay)
    rng = np.random.default_rng(3)
    idx = np.stack([np.concatenate([[5], rng.choice([0, 1, 2, 3, 4, 6, 7], 3, replace=False)])
                    for _ in range(n)]).astype(np.int32)
    idx[7] = [5, 5, 5, 2]          # duplicates: expert 5 appears 66 times in all
    w = rng.random((n, 4)).astype(np.float32)
    lay_dev = to_dev(lay)
    y_ps, y_dd, U, _ = _run_both(cfg, lay_dev, x.cuda(), torch.from_numpy(idx).cuda(),
                                 torch.from_numpy(w).cuda())
    y_ref, _, _, U_ref = oracle_y(cfg, host, x.numpy(), idx, w)
    assert U == U_ref
    assert torch.equal(y_ps, y_dd)
    assert rel_err(y_ps.cpu().numpy(), y_ref) <= OUT_RTOL["bf16"]


def test_out_of_range_routing_is_an_empty_slot():
    cfg = small_config("oob", 256, 8, 2, 128, 0, "bf16")
    lay = synth.make_layer(cfg, "cpu")
    x = synth.make_hidden(cfg, 4, 0, "cpu")
    host = host_layer(lay)
    idx = np.array([[1, 2], [3, 99], [-1, 0], [4, 5]], dtype=np.int32)
    w = np.full((4, 2), 0.5, dtype=np.float32)
    y_ps, y_dd, U, _ = _run_both(cfg, to_dev(lay), x.cuda(), torch.from_numpy(idx).cuda(),
                                 torch.from_numpy(w).cuda())
    assert torch.equal(y_ps, y_dd) and U == 6
    # reference: the invalid slots contribute nothing
    keep = (idx >= 0) & (idx < 8)
    y_ref = np.zeros((4, 256))
    for t in range(4):
        for j in range(2):
            if keep[t, j]:
                e = idx[t, j]
                o = O.expert(oshape(cfg), host["w13"][e, 0], host["w13"][e, 1], host["w2"][e],
                             x.numpy()[t])
                y_ref[t] += w[t, j] * o
    assert rel_err(y_ps.cpu().numpy(), y_ref) <= OUT_RTOL["bf16"]


def test_k_equals_E_matches_dense_mixture():
    cfg = small_config("dense", 256, 8, 8, 128, 1, "f32")
    lay = synth.make_layer(cfg, "cpu")
    x = synth.make_hidden(cfg, 5, 0, "cpu")
    host = host_layer(lay)
    lay_dev = to_dev(lay)
    idx, w = B.route(B.shape_of(cfg), lay_dev["gate_w"], x.cuda())
    y_ps, y_dd, U, _ = _run_both(cfg, lay_dev, x.cuda(), idx, w)
    yd = O.dense_mixture(oshape(cfg), host["gate_w"], host["w13"], host["w2"], host["ws13"],
                         host["ws2"], x.numpy())
    assert U == 8 and torch.equal(y_ps, y_dd)
    assert rel_err(y_ps.cpu().numpy(), yd) <= OUT_RTOL["f32"]


def test_router_ties_pick_lowest_index():
    cfg = small_config("ties", 256, 16, 3, 64, 0, "f32")
    lay = synth.make_layer(cfg, "cpu")
    gw = lay["gate_w"].clone()
    gw[9] = gw[2]
    gw[11] = gw[2]
    x = synth.make_hidden(cfg, 8, 0, "cpu")
    idx, w = B.route(B.shape_of(cfg), gw.cuda(), x.cuda())
    ref = O.route(oshape(cfg), gw.numpy(), x.numpy())
    gi = idx.cpu().numpy()
    for t in range(8):
        sel = gi[t].tolist()
        for a_, b_ in [(2, 9), (9, 11), (2, 11)]:
            if b_ in sel:
                assert a_ in sel and sel.index(a_) < sel.index(b_)
    assert np.array_equal(gi, ref["idx"])


@pytest.mark.parametrize("E,d", [(64, 512), (256, 2048)])
def test_route_reuses_its_workspace(E, d):
    """One routing workspace across many calls (its arrival counter must be
    back at zero after every call); each call checked against the oracle."""
    cfg = small_config("reuse", d, E, 6, 64, 0, "bf16")
    lay = synth.make_layer(cfg, "cpu")
    gw = lay["gate_w"].cuda()
    ws = B.Workspace()
    for rep, n in enumerate([1, 16, 3, 64, 7, 16, 1, 33] * 2):
        if n * cfg.k > B.MAX_SLOTS:
            continue
        x = synth.make_hidden(cfg, n, rep, "cpu")
        idx, w = B.route(B.shape_of(cfg), gw, x.cuda(), ws=ws)
        ref = O.route(oshape(cfg), lay["gate_w"].numpy(), x.numpy(), tie_eps=TIE_EPS)
        ok = ref["flags"] == 0
        assert np.array_equal(idx.cpu().numpy()[ok], ref["idx"][ok]), (rep, n)
        assert int(ws.buf[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("n,wdt", [(5, "bf16"), (16, "bf16"), (64, "bf16"), (16, "f32")])
def test_dedup_around_the_folded_grid(n, wdt):
    """The dedup grid is folded in half where E >= 8k and ceil(U_max/2) >=
    2k: a workgroup runs distinct expert v and, when U > fold, v + fold.
    Routings with exactly U experts at k, fold - 1, fold, fold + 1 and U_max
    (narrow and LDS-staged wide tiles) give the per-slot output bit for bit
    and report U; one case is checked against the oracle."""
    cfg = small_config("fold", 512, 64, 6, 352, 2, wdt)
    lay = synth.make_layer(cfg, "cpu")
    host, lay_dev, shape = host_layer(lay), to_dev(lay), B.shape_of(cfg)
    u_max = min(cfg.E, n * cfg.k)
    fold = (u_max + 1) // 2
    assert cfg.E >= 8 * cfg.k and fold >= 2 * cfg.k       # the folded grid runs
    x = synth.make_hidden(cfg, n, 3, "cpu")
    x_dev = x.cuda()
    for U in sorted({cfg.k, fold - 1, fold, fold + 1, u_max}):
        idx, w = synth.crafted_routing(n, cfg.k, cfg.E, U, seed=U)
        idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
        nu = torch.zeros(1, dtype=torch.int32, device="cuda")
        y_dd = B.expert_pass_dedup(shape, lay_dev, x_dev, idx_d, w_d, n_unique=nu)
        y_ps = B.expert_pass_perslot(shape, lay_dev, x_dev, idx_d, w_d)
        torch.cuda.synchronize()
        assert int(nu.item()) == U, (n, U)
        assert torch.equal(y_dd, y_ps), (n, U)
        if U == fold + 1:
            y_ref = oracle_y(cfg, host, x.numpy(), idx, w)[0]
            assert rel_err(y_dd.cpu().numpy(), y_ref) <= OUT_RTOL[wdt], (n, U)


def test_one_workspace_shared_by_every_kind_of_call():
    """One workspace, zeroed once at allocation and never again, serves every
    kind of call in any order and size (routing, the three expert passes,
    the stack pass, the filter and both verification modes): each call on
    the shared workspace equals the same call on a fresh one, and the head
    (arrival counters) is zero after every call."""
    cfg = small_config("shared-ws", 512, 64, 6, 352, 2, "bf16")
    lay = synth.make_layer(cfg, "cpu")
    lay_dev = to_dev(lay)
    shape = B.shape_of(cfg)
    L = 3
    stack = {k: (None if v is None else torch.stack([v] * L).contiguous())
             for k, v in lay_dev.items()}
    stack["layout"] = "rows"
    ws = B.Workspace()
    rng = np.random.default_rng(5)

    def head_zero():
        torch.cuda.synchronize()
        return int(ws.buf[:256].count_nonzero()) == 0

    for rep, n in enumerate([16, 3, 9, 1, 24]):
        x = synth.make_hidden(cfg, n, rep, "cuda")
        idx_f, w_f = B.route(shape, lay_dev["gate_w"], x)
        y_f = B.expert_pass_dedup(shape, lay_dev, x, idx_f, w_f)
        y_s = B.expert_pass_dedup(shape, lay_dev, x, idx_f, w_f, ws=ws)
        assert head_zero()
        idx_s, w_s = B.route(shape, lay_dev["gate_w"], x, ws=ws)
        assert head_zero()
        gs = [0, n // 2, n] if n > 1 else [0, 1]
        yg_f = B.expert_pass_dedup_grouped(shape, lay_dev, x, idx_f, w_f, gs)
        yg_s = B.expert_pass_dedup_grouped(shape, lay_dev, x, idx_f, w_f, gs, ws=ws)
        assert head_zero()
        yp_f = B.expert_pass_perslot(shape, lay_dev, x, idx_f, w_f)
        yp_s = B.expert_pass_perslot(shape, lay_dev, x, idx_f, w_f, ws=ws)
        assert head_zero()
        sk_f = B.stack_pass(shape, stack, x, "dedup")
        sk_s = B.stack_pass(shape, stack, x, "dedup", ws=ws)
        assert head_zero()
        lg = torch.from_numpy(rng.standard_normal((2, 3, 3000 + 7 * rep)).astype(np.float32)).cuda()
        p_f = B.verify_probs(lg, 0.8, 0.9)
        p_s = B.verify_probs(lg, 0.8, 0.9, ws=ws)
        assert head_zero()
        xt = p_f[:, :2].argmax(dim=2).to(torch.int32)
        n_f, t_f = B.verify_gate(p_f, xt, mode=B.VERIFY_GREEDY)
        n_s, t_s = B.verify_gate(p_s, xt, mode=B.VERIFY_GREEDY, ws=ws)
        assert head_zero()
        u = torch.from_numpy(rng.random((2, 2)).astype(np.float32)).cuda()
        r = torch.from_numpy(rng.integers(-2**31, 2**31 - 1, 2).astype(np.int32)).cuda()
        q = p_f[:, :2].contiguous()
        m_f, o_f = B.verify_gate(p_f, xt, q=q, u=u, r=r, mode=B.VERIFY_SAMPLING)
        m_s, o_s = B.verify_gate(p_s, xt, q=q, u=u, r=r, mode=B.VERIFY_SAMPLING, ws=ws)
        assert head_zero()
        torch.cuda.synchronize()
        assert torch.equal(y_s, y_f) and torch.equal(idx_s, idx_f) and torch.equal(w_s, w_f)
        assert torch.equal(yg_s, yg_f) and torch.equal(yp_s, yp_f)
        assert all(torch.equal(a_, b_) for a_, b_ in zip(sk_s, sk_f))
        assert torch.equal(p_s, p_f) and torch.equal(n_s, n_f) and torch.equal(t_s, t_f)
        assert torch.equal(m_s, m_f) and torch.equal(o_s, o_f)


def test_runs_are_bitwise_deterministic():
    cfg = small_config("det", 512, 64, 6, 352, 2, "bf16")
    lay_dev = to_dev(synth.make_layer(cfg, "cpu"))
    x = synth.make_hidden(cfg, 16, 0, "cpu").cuda()
    outs = []
    for _ in range(3):
        idx, w = B.route(B.shape_of(cfg), lay_dev["gate_w"], x)
        y_ps, y_dd, U, _ = _run_both(cfg, lay_dev, x, idx, w)
        outs.append((idx.clone(), y_ps.clone(), y_dd.clone()))
    for o in outs[1:]:
        assert all(torch.equal(a_, b_) for a_, b_ in zip(o, outs[0]))


def test_mfma_column_position_does_not_change_results():
    """A token's output bits do not depend on which other tokens share its
    MFMA tile: each token alone equals the same token inside a 16-token pass."""
    cfg = small_config("colpos", 512, 4, 1, 256, 0, "bf16")
    lay_dev = to_dev(synth.make_layer(cfg, "cpu"))
    x = synth.make_hidden(cfg, 16, 0, "cpu").cuda()
    idx = torch.zeros((16, 1), dtype=torch.int32, device="cuda")
    w = torch.ones((16, 1), dtype=torch.float32, device="cuda")
    shape = B.shape_of(cfg)
    y_all = B.expert_pass_dedup(shape, lay_dev, x, idx, w)
    for t in (0, 5, 15):
        y_one = B.expert_pass_dedup(shape, lay_dev, x[t:t + 1].contiguous(), idx[:1], w[:1])
        torch.cuda.synchronize()
        assert torch.equal(y_one[0], y_all[t])


# ------------------------------------------------------------- full-size configs

def _host_experts(cfg, lay_dev, used):
    """Host bit patterns of the routed experts in `used` (others zero, never
    read) and of the shared experts."""
    hdt = np.uint16 if cfg.wdtype == "bf16" else np.float32
    host = {"w13": np.zeros((cfg.E,) + tuple(lay_dev["w13"].shape[1:]), hdt),
            "w2": np.zeros((cfg.E,) + tuple(lay_dev["w2"].shape[1:]), hdt)}
    for e in used:
        host["w13"][e] = synth.to_host_bits(lay_dev["w13"][e])
        host["w2"][e] = synth.to_host_bits(lay_dev["w2"][e])
    host["ws13"] = None if lay_dev["ws13"] is None else synth.to_host_bits(lay_dev["ws13"])
    host["ws2"] = None if lay_dev["ws2"] is None else synth.to_host_bits(lay_dev["ws2"])
    return host


def _full_pass(cfg, lay_dev, tiled, n, rep=0, tokens=None):
    """One verify pass of the workload end to end: the GPU routes and both
    GPU engines run on that routing; the oracle routes the same hidden
    states itself and runs its layer on its own routing.  Routing, U and
    the outputs are compared on every token (or the given tokens): tokens
    the oracle flags as near-ties are exempt from the index comparison and
    their outputs are checked against the oracle layer on the GPU's
    routing of that token, a valid top-k of the GPU's logits."""
    _say(f"[full] {cfg.name} n={n} rep={rep}")
    x_dev = synth.make_hidden(cfg, n, rep, "cuda")
    gate_np = lay_dev["gate_w"].cpu().numpy()
    x_np = x_dev.cpu().numpy()
    idx, w, ref, flagged = _check_route(cfg, lay_dev["gate_w"], x_dev, gate_np, x_np)
    y_ps, y_dd, U, _ = _run_both(cfg, tiled, x_dev, idx, w)
    assert torch.equal(y_ps, y_dd)
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    assert U == O.pass_bytes(oshape(cfg), gi)[3]
    assert B.pass_bytes(B.shape_of(cfg), gi) == O.pass_bytes(oshape(cfg), gi)
    ok = (ref["flags"] == 0)[:, None]
    idx_ref = np.where(ok, ref["idx"], gi).astype(np.int32)
    w_ref = np.where(ok, ref["w"], gw.astype(np.float64))
    toks = np.arange(x_np.shape[0]) if tokens is None else np.asarray(tokens)
    host = _host_experts(cfg, lay_dev, np.unique(idx_ref[toks]))
    y_ref, _, _, _ = oracle_y(cfg, host, x_np, idx_ref, w_ref, tokens=toks, threads=16)
    err = rel_err(y_ps.cpu().numpy()[toks], y_ref)
    _say(f"   {len(toks)} tokens: rel err {err:.3e}  U={U}  flagged={flagged}")
    assert err <= OUT_RTOL[cfg.wdtype]


def _full_layer(name):
    cfg = synth.CONFIGS[name]
    lay_dev = synth.make_layer(cfg, "cuda")
    tiled = B.pack_weights(B.shape_of(cfg), {k: lay_dev[k] for k in ("w13", "w2", "ws13", "ws2")})
    return cfg, lay_dev, tiled


def test_full_tiny():
    cfg, lay_dev, tiled = _full_layer("tiny")
    _full_pass(cfg, lay_dev, tiled, 4)


def test_full_v2lite_every_token():
    cfg, lay_dev, tiled = _full_layer("v2lite")
    for n in (1, 2, 4, 8, 16):
        _full_pass(cfg, lay_dev, tiled, n)
    del lay_dev, tiled
    torch.cuda.empty_cache()


def test_full_mixtral_every_token():
    cfg, lay_dev, tiled = _full_layer("mixtral")
    for n in (1, 4, 8):
        _full_pass(cfg, lay_dev, tiled, n)
    del lay_dev, tiled
    torch.cuda.empty_cache()


def test_full_v3_one_sequence_and_every_column_tile():
    """The V3-shaped pass of 4 sequences x 16 tokens: all of sequence 1
    (tokens 16..31) and tokens of the other 16-token column tiles."""
    cfg, lay_dev, tiled = _full_layer("v3")
    _full_pass(cfg, lay_dev, tiled, 16, tokens=list(range(16, 32)) + [0, 9, 32, 40, 47, 55, 63])
    del lay_dev, tiled
    torch.cuda.empty_cache()
