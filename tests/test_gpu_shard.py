"""One GPU's share of a layer whose experts are split along d_ff over G GPUs
(rows of W1 and W3, the same columns of W2, routed and shared experts
alike; gate and tokens whole), at the real layer shapes, through the C ABI.
On the routing of the whole gate, the shares' passes add up to the whole
layer's pass (the down projection and the combine are linear; the
hidden-unit activations of a share are those of the whole layer, bit for
bit, since each depends only on its own rows), and each share requests
exactly 1/G of the bytes ("Deep Dive into Mixture of Experts", section
"2017: The Sparse-Gating Leap": the gate-weighted sum of expert outputs).
This is the part of a multi-GPU layer that one GPU can show; the summing
all-reduce itself is not run."""
import pytest
import torch

from speculative_decode_verify_gate_amd import binding as B
from speculative_decode_verify_gate_amd import synth

pytestmark = pytest.mark.gpu

# Only the down projection's summation order differs between the whole
# pass and the sum of the shares (the shares' partial sums are added last,
# in fp32): L-infinity relative error well inside this.
SHARE_RTOL = 1e-5


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name,G,n", [("v3", 8, 4), ("v3", 8, 8), ("v2lite", 4, 16),
                                      ("mixtral", 8, 4)])
def test_shares_add_up_to_the_layer(name, G, n):
    cfg = synth.CONFIGS[name]
    share = synth.share_config(cfg, G)
    _say(f"[shard] {name} G={G} n={n}: d_ff {cfg.f} -> {share.f}")
    lay = synth.make_layer(cfg, "cuda")
    x = synth.make_hidden(cfg, n, 0, "cuda")
    shape, s_shape = B.shape_of(cfg), B.shape_of(share)
    idx, w = B.route(shape, lay["gate_w"], x)
    y = B.expert_pass_dedup(shape, lay, x, idx, w)
    total = torch.zeros_like(y)
    for g in range(G):
        part = synth.shard_layer(lay, G, g)
        y_ps = B.expert_pass_perslot(s_shape, part, x, idx, w)
        y_dd = B.expert_pass_dedup(s_shape, part, x, idx, w)
        torch.cuda.synchronize()
        assert torch.equal(y_ps, y_dd), g
        total += y_dd
        del part
    torch.cuda.synchronize()
    err = float((total - y).abs().max() / y.abs().max())
    _say(f"   shares vs whole: rel err {err:.2e}")
    assert err <= SHARE_RTOL
    idx_h = idx.cpu()
    ps, dd, sh, U = B.pass_bytes(shape, idx_h)
    ps_g, dd_g, sh_g, U_g = B.pass_bytes(s_shape, idx_h)
    assert (ps_g * G, dd_g * G, sh_g * G, U_g) == (ps, dd, sh, U)
