"""moe_stack_pass_noalloc against moe_stack_pass, through the C ABI: the
variant runs the same kernels on the library's static device workspace, so
its routing, U and layer outputs must equal the workspace entry point's bit
for bit.  Two calls in a row (the second on a smaller stack and fewer
tokens, so it runs on what the first left in the shared array), both
engines, then the caller-workspace entry point again."""
import numpy as np
import pytest
import torch

from speculative_decode_verify_gate_amd import binding as B
from speculative_decode_verify_gate_amd import synth
from helpers import small_config, to_dev

pytestmark = pytest.mark.gpu


def _stack(cfg, L):
    lays = [to_dev(synth.make_layer(cfg, "cpu", layer=l)) for l in range(L)]
    st = {k: (None if lays[0][k] is None else torch.stack([lay[k] for lay in lays]).contiguous())
          for k in ("gate_w", "w13", "w2", "ws13", "ws2")}
    st["layout"] = "rows"
    return st


def _both(shape, st, x, engine):
    L = st["gate_w"].shape[0]
    nu_a = torch.full((L,), -1, dtype=torch.int32, device="cuda")
    nu_b = torch.full((L,), -1, dtype=torch.int32, device="cuda")
    ref = B.stack_pass(shape, st, x, engine, n_unique=nu_a)
    got = B.stack_pass_noalloc(shape, st, x, engine, n_unique=nu_b)
    torch.cuda.synchronize()
    return ref, got, nu_a, nu_b


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_noalloc_equals_the_workspace_entry_point(wdt):
    cfg = small_config("noalloc", 512, 64, 6, 352, 2, wdt)
    shape = B.shape_of(cfg)
    big = _stack(cfg, 4)
    for call, (L, n) in enumerate([(4, 24), (2, 5)]):
        st = big if L == 4 else {k: (v[:L].contiguous() if torch.is_tensor(v) else v)
                                 for k, v in big.items()}
        x = synth.make_hidden(cfg, n, call, "cuda")
        for engine in ("dedup", "perslot"):
            print(f"[noalloc] {wdt} call {call} L={L} n={n} {engine}", flush=True)
            ref, got, nu_a, nu_b = _both(shape, st, x, engine)
            for a_, b_ in zip(ref, got):
                assert torch.equal(a_, b_), (call, engine)
            if engine == "dedup":
                assert torch.equal(nu_a, nu_b) and int(nu_b.min()) >= cfg.k
    # the caller-workspace entry point is unchanged afterwards
    x = synth.make_hidden(cfg, 16, 9, "cuda")
    ref = B.stack_pass(shape, big, x, "dedup")
    again = B.stack_pass(shape, big, x, "dedup")
    got = B.stack_pass_noalloc(shape, big, x, "dedup")
    torch.cuda.synchronize()
    for a_, b_, c_ in zip(ref, again, got):
        assert torch.equal(a_, b_) and torch.equal(a_, c_)
