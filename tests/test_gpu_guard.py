"""Every device call writes its declared outputs and nothing else: each output
is the middle of a larger allocation whose guard bytes on both sides hold a
canary pattern that must survive the call (C ABI conventions of
include/moe_verify.h)."""
import numpy as np
import pytest
import torch

from speculative_decode_verify_gate_amd import binding as B
from speculative_decode_verify_gate_amd import synth
from helpers import small_config

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side


class Guarded:
    """A tensor view with canary bytes before and after it."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((n + 2 * GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
        self.n = n
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(shape)

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.raw[:GUARD] == 0xA5).all()) and bool((self.raw[GUARD + self.n:] == 0xA5).all())


def test_route_and_passes_stay_inside_their_outputs():
    cfg = small_config("guard", 512, 64, 6, 352, 2, "bf16")
    lay = {k: (None if v is None else v.cuda()) for k, v in synth.make_layer(cfg, "cpu").items()}
    shape = B.shape_of(cfg)
    for n in (1, 16, 17, 64):
        x = synth.make_hidden(cfg, n, 0, "cuda")
        idx, w = Guarded((n, cfg.k), torch.int32), Guarded((n, cfg.k), torch.float32)
        logits, margin = Guarded((n, cfg.E), torch.float32), Guarded((n,), torch.float32)
        B.route(shape, lay["gate_w"], x, idx=idx.t, w=w.t, logits=logits.t, margin=margin.t,
                bias=synth.make_bias(cfg, "cuda"))
        assert all(g.intact() for g in (idx, w, logits, margin)), n
        for engine in ("perslot", "dedup", "grouped"):
            y = Guarded((n, cfg.d), torch.float32)
            nu = Guarded((2,), torch.int32)
            if engine == "perslot":
                B.expert_pass_perslot(shape, lay, x, idx.t, w.t, y=y.t)
            elif engine == "dedup":
                B.expert_pass_dedup(shape, lay, x, idx.t, w.t, y=y.t, n_unique=nu.t[:1])
            elif n > 1:
                B.expert_pass_dedup_grouped(shape, lay, x, idx.t, w.t, [0, n // 2, n], y=y.t,
                                            n_unique=nu.t)
            assert y.intact() and nu.intact(), (n, engine)


def test_stack_pass_stays_inside_its_outputs():
    cfg = small_config("guard-stack", 256, 16, 2, 128, 1, "bf16")
    L, n = 3, 9
    lays = [synth.make_layer(cfg, "cuda", layer=l) for l in range(L)]
    stack = {k: torch.stack([lay[k] for lay in lays]).contiguous()
             for k in ("gate_w", "w13", "w2", "ws13", "ws2")}
    x = synth.make_hidden(cfg, n, 0, "cuda")
    for engine in ("perslot", "dedup"):
        idx, w = Guarded((L, n, cfg.k), torch.int32), Guarded((L, n, cfg.k), torch.float32)
        y, nu = Guarded((L, n, cfg.d), torch.float32), Guarded((L,), torch.int32)
        B.stack_pass(B.shape_of(cfg), stack, x, engine, idx=idx.t, w=w.t, y=y.t, n_unique=nu.t)
        assert all(g.intact() for g in (idx, w, y, nu)), engine


def test_verify_round_stays_inside_its_outputs():
    rng = np.random.default_rng(2)
    S, gamma, V = 3, 5, 3000
    p = torch.from_numpy(rng.dirichlet(np.ones(V), (S, gamma + 1)).astype(np.float32)).cuda()
    q = torch.from_numpy(rng.dirichlet(np.ones(V), (S, gamma)).astype(np.float32)).cuda()
    x = torch.from_numpy(rng.integers(0, V, (S, gamma)).astype(np.int32)).cuda()
    u = torch.rand((S, gamma), device="cuda")
    r = torch.randint(-2**31, 2**31 - 1, (S,), device="cuda", dtype=torch.int32)
    for mode in (B.VERIFY_GREEDY, B.VERIFY_SAMPLING):
        na, out = Guarded((S,), torch.int32), Guarded((S, gamma + 1), torch.int32)
        B.verify_gate(p, x, q=q, u=u, r=r, mode=mode, n_accepted=na.t, out=out.t)
        assert na.intact() and out.intact(), mode


@pytest.mark.parametrize("V", [4099, 32000])
def test_filter_stays_inside_its_outputs(V):
    # single and paired calls, top_p < 1 (all four launches) and = 1, a
    # ragged vocabulary (scalar loads) and an aligned one (16-byte stores)
    rng = np.random.default_rng(V)
    lp = torch.from_numpy((rng.standard_normal((5, V)) * 3).astype(np.float32)).cuda()
    lq = torch.from_numpy((rng.standard_normal((3, V)) * 3).astype(np.float32)).cuda()
    for top_p in (0.9, 1.0):
        p = Guarded((5, V), torch.float32)
        B.verify_probs(lp, 0.7, top_p, out=p.t)
        assert p.intact(), ("single", top_p)
        p, q = Guarded((5, V), torch.float32), Guarded((3, V), torch.float32)
        B.verify_probs_pair(lp, lq, 0.7, top_p, out_p=p.t, out_q=q.t)
        assert p.intact() and q.intact(), ("pair", top_p)
