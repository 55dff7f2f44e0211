"""GPU calls at the largest sizes the C ABI accepts (the limits declared in
include/moe_verify.h), checked against the CPU oracle through the C ABI:
the layer with the most experts, top-k, shared experts and slots, the
verification round with the most sequences and drafted tokens and at the
largest vocabulary, the logits filter at the largest vocabulary and with
the most rows, and grouped deduplication with the most token groups."""
import numpy as np
import pytest
import torch

import oracle as O
from speculative_decode_verify_gate_amd import binding as B
from speculative_decode_verify_gate_amd import synth
from helpers import OUT_RTOL, host_layer, oracle_y, oshape, rel_err, small_config, to_dev
from test_gpu_parity import _check_record, _check_route, _run_both
from test_gpu_verify import _case, _check_nucleus, _run_gpu, _run_oracle

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("n", [1, 32])
def test_layer_with_the_most_experts_topk_shared_and_slots(n):
    # 256 experts, top-16, 4 shared experts; 32 tokens fill all 512 slots
    cfg = small_config("moe-max", 256, B.MAX_EXPERTS, B.MAX_TOPK, 128, B.MAX_SHARED, "bf16")
    assert 32 * cfg.k == B.MAX_SLOTS
    _say(f"[limits] layer E={cfg.E} k={cfg.k} S={cfg.S} n={n}")
    lay = synth.make_layer(cfg, "cpu")
    x = synth.make_hidden(cfg, n, 0, "cpu")
    host, x_np = host_layer(lay), x.numpy()
    lay_dev, x_dev = to_dev(lay), x.cuda()
    _, _, ref, flagged = _check_route(cfg, lay_dev["gate_w"], x_dev, host["gate_w"], x_np)
    idx_o = torch.from_numpy(ref["idx"]).cuda()
    w_o = torch.from_numpy(ref["w"].astype(np.float32)).cuda()
    y_ps, y_dd, U, ws = _run_both(cfg, lay_dev, x_dev, idx_o, w_o)
    y_ref, _, _, U_ref = oracle_y(cfg, host, x_np, ref["idx"], ref["w"].astype(np.float32))
    assert U == U_ref
    assert torch.equal(y_ps, y_dd)
    _check_record(cfg, ws, ref["idx"])
    err = rel_err(y_ps.cpu().numpy(), y_ref)
    _say(f"   rel err {err:.3e}  U={U}  flagged={flagged}")
    assert err <= OUT_RTOL["bf16"]
    assert B.pass_bytes(B.shape_of(cfg), ref["idx"]) == O.pass_bytes(oshape(cfg), ref["idx"])


@pytest.mark.parametrize("mode", [B.VERIFY_GREEDY, B.VERIFY_SAMPLING])
def test_round_with_the_most_sequences_and_drafted_tokens(mode):
    rng = np.random.default_rng(640 + mode)
    _say(f"[limits] round S={B.MAX_SEQ} gamma={B.MAX_DRAFT} mode={mode}")
    p, q, x, u, r = _case(rng, B.MAX_SEQ, B.MAX_DRAFT, 512, mode)
    n_g, t_g = _run_gpu(p, q, x, u, r, mode)
    n_o, t_o = _run_oracle(p, q, x, u, r, mode)
    np.testing.assert_array_equal(n_g, n_o)
    np.testing.assert_array_equal(t_g, t_o)


def test_filter_and_round_at_the_largest_vocabulary():
    V = B.MAX_VOCAB
    rng = np.random.default_rng(24)
    _say(f"[limits] filter + round at V={V}")
    vl = (rng.standard_normal((1, 2, V), dtype=np.float32) * 3.0)
    dl = vl[:, :1] + np.float32(0.5) * rng.standard_normal((1, 1, V), dtype=np.float32)
    p = B.verify_probs(torch.from_numpy(vl).cuda(), 0.7, 0.9)
    q = B.verify_probs(torch.from_numpy(dl).cuda(), 0.7, 0.9)
    pn, qn = p.cpu().numpy(), q.cpu().numpy()
    _check_nucleus(pn.reshape(2, V), vl.reshape(2, V), 0.7, 0.9)
    _check_nucleus(qn.reshape(1, V), dl.reshape(1, V), 0.7, 0.9)
    kept = np.flatnonzero(qn[0, 0])
    w = qn[0, 0, kept].astype(np.float64)
    for mode in (B.VERIFY_GREEDY, B.VERIFY_SAMPLING):
        for rep in range(3):
            x = np.array([[kept[rng.choice(kept.size, p=w / w.sum())]]], dtype=np.int32)
            u = rng.random((1, 1)).astype(np.float32)
            r = rng.integers(0, 2**32, 1, dtype=np.uint64)
            args = (pn, qn, x, u, r) if mode == B.VERIFY_SAMPLING else (pn, None, x, None, None)
            n_g, t_g = _run_gpu(*args, mode)
            n_o, t_o = _run_oracle(*args, mode)
            np.testing.assert_array_equal(n_g, n_o)
            np.testing.assert_array_equal(t_g, t_o)


def test_filter_with_the_most_rows():
    rows, V = 65535, 8
    rng = np.random.default_rng(65535)
    _say(f"[limits] filter rows={rows} V={V}")
    lg = (rng.standard_normal((rows, V)) * rng.uniform(0.5, 4.0, (rows, 1))).astype(np.float32)
    lg[:, 3] = lg[:, 5]                       # one exact tie in every row
    got = B.verify_probs(torch.from_numpy(lg).cuda(), 0.9, 0.8).cpu().numpy()
    _check_nucleus(got, lg, 0.9, 0.8)


def test_grouped_dedup_with_the_most_groups():
    # the most tokens, one group per token: the most groups; every group
    # holds k distinct experts and the output is the per-slot engine's
    cfg = small_config("groups-max", 256, 16, 2, 128, 1, "bf16")
    n = B.MAX_TOKENS
    assert n == B.MAX_GROUPS
    _say(f"[limits] grouped dedup G={n}")
    lay = to_dev(synth.make_layer(cfg, "cpu"))
    shape = B.shape_of(cfg)
    x = synth.make_hidden(cfg, n, 2, "cuda")
    idx, w = B.route(shape, lay["gate_w"], x)
    nun = torch.zeros(n, dtype=torch.int32, device="cuda")
    y_g = B.expert_pass_dedup_grouped(shape, lay, x, idx, w, list(range(n + 1)), n_unique=nun)
    y_ps = B.expert_pass_perslot(shape, lay, x, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(y_g, y_ps)
    assert bool((nun == cfg.k).all())
    # and grouped as 8 sequences of 8: U_g is the number of distinct
    # experts of each group, and the host byte count agrees
    gs = [8 * i for i in range(9)]
    nu8 = torch.zeros(8, dtype=torch.int32, device="cuda")
    y_8 = B.expert_pass_dedup_grouped(shape, lay, x, idx, w, gs, n_unique=nu8)
    torch.cuda.synchronize()
    assert torch.equal(y_8, y_ps)
    idx_np = idx.cpu().numpy()
    want = [len(set(idx_np[a:b].ravel().tolist())) for a, b in zip(gs[:-1], gs[1:])]
    assert list(nu8.cpu().numpy()) == want
    assert B.pass_bytes_grouped(shape, idx_np, gs)[1] == want
