"""GPU: the per-kernel timing of the library (moe_timing_enable / read) counts
each bracketed launch once, measures a positive time, and leaves every
output bit unchanged."""
import math

import pytest
import torch

from speculative_decode_verify_gate_amd import binding as B
from speculative_decode_verify_gate_amd import synth
from helpers import small_config

pytestmark = pytest.mark.gpu


def test_timing_counts_each_launch_and_changes_no_output():
    cfg = small_config("timing", 256, 32, 4, 128, 1, "bf16")
    shape = B.shape_of(cfg)
    lay = B.pack_weights(shape, synth.make_layer(cfg, "cuda"))
    x = synth.make_hidden(cfg, 12, 0, "cuda")
    ws = B.Workspace()
    idx, w = B.route(shape, lay["gate_w"], x, ws=ws)
    y0 = B.expert_pass_dedup(shape, lay, x, idx, w, ws=ws).clone()
    torch.cuda.synchronize()
    B.timing_read()  # start from zero
    B.timing_enable(("gate", "up", "down", "combine"))
    try:
        idx1, w1 = B.route(shape, lay["gate_w"], x, ws=ws)
        y1 = B.expert_pass_dedup(shape, lay, x, idx1, w1, ws=ws).clone()
        y2 = B.expert_pass_perslot(shape, lay, x, idx1, w1, ws=ws).clone()
        torch.cuda.synchronize()
        t = B.timing_read()
    finally:
        B.timing_enable(())
    assert torch.equal(idx1, idx) and torch.equal(w1, w)
    assert torch.equal(y1, y0) and torch.equal(y2, y0)
    for kind in ("up", "down", "combine"):
        ms, n = t[kind]
        assert n == 2 and math.isfinite(ms) and ms > 0, (kind, t[kind])
    assert t["gate"][1] >= 1 and t["gate"][0] > 0
    assert t["verify"] == (0.0, 0) and t["filter"] == (0.0, 0)
    # a read returns what accumulated since the previous one; disabled, nothing
    B.expert_pass_dedup(shape, lay, x, idx, w, ws=ws)
    torch.cuda.synchronize()
    assert all(v == (0.0, 0) for v in B.timing_read().values())
