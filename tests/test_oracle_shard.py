"""The d_ff sharding the multi-GPU layout relies on, on the CPU oracle:
every expert split along d_ff into G shares (rows of W1 and W3, the same
columns of W2, routed and shared experts alike) with the gate and the
tokens whole.  Each hidden unit's activation depends only on its own rows
of W1 and W3 and on the whole token, and the down projection and the
weighted combine are linear, so the layer's output is the sum of the
shares' outputs (fp64 oracle: to rounding), and each share requests 1/G of
the bytes ("Deep Dive into Mixture of Experts", section "2017: The
Sparse-Gating Leap": the output is the gate-weighted sum of expert outputs;
the SwiGLU expert is the reading the layer shapes use)."""
import numpy as np
import pytest

import oracle as O
from speculative_decode_verify_gate_amd import synth
from helpers import host_layer, oshape, small_config


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("G", [2, 4])
def test_layer_is_the_sum_of_its_dff_shares(wdt, G):
    cfg = small_config("shard", 64, 8, 2, 128, 1, wdt)
    lay = synth.make_layer(cfg, "cpu")
    x = synth.make_hidden(cfg, 6, 0, "cpu").numpy()
    host = host_layer(lay)
    s = oshape(cfg)
    r = O.route(s, host["gate_w"], x)
    y, rb, sb, U = O.layer(s, host["w13"], host["w2"], host["ws13"], host["ws2"], x, r["idx"],
                           r["w"])
    share = synth.share_config(cfg, G)
    assert share.f == cfg.f // G and share.expert_bytes * G == cfg.expert_bytes
    s_sh = oshape(share)
    total = np.zeros_like(y)
    for g in range(G):
        h = host_layer(synth.shard_layer(lay, G, g))
        yg, rbg, sbg, Ug = O.layer(s_sh, h["w13"], h["w2"], h["ws13"], h["ws2"], x, r["idx"],
                                   r["w"])
        assert (rbg * G, sbg * G, Ug) == (rb, sb, U)
        total += yg
    scale = np.max(np.abs(y))
    assert np.max(np.abs(total - y)) <= 1e-12 * scale
    # a share is a layer in its own right: the dedup formulation agrees
    yd = O.layer(s_sh, h["w13"], h["w2"], h["ws13"], h["ws2"], x, r["idx"], r["w"],
                 engine="dedup")[0]
    np.testing.assert_array_equal(yd, yg)


def test_share_config_needs_whole_32_wide_shares():
    assert synth.share_config(synth.CONFIGS["v3"], 8).f == 256
    assert synth.share_config(synth.CONFIGS["mixtral"], 8).f == 1792
    assert synth.share_config(synth.CONFIGS["v2lite"], 4).f == 352
    for name, G in (("v2lite", 8), ("v3", 3), ("tiny", 32)):
        with pytest.raises(ValueError):
            synth.share_config(synth.CONFIGS[name], G)
