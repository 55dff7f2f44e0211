"""Seeded synthetic inputs for the MoE verify-pass layer.

This module only draws inputs: layer shapes, N(0, 0.02) weights and AR(1)
hidden states.  It holds none of the layer's arithmetic and imports neither
the GPU library nor the CPU oracle; both are fed from here.

Workloads (the pages name model families but print no layer sizes; the sizes
below are the ones this project measures on):
  tiny      fp32 layer, d=256, 8 experts top-2, d_ff=512, n=4, rho=0.9
  mixtral   Mixtral-8x7B-shaped layer, d=4096, 8 experts top-2, d_ff=14336,
            bf16 weights, fp32 gate, rho=0.8, n=1..8
  v2lite    DeepSeek-V2-Lite-shaped layer, d=2048, 64 routed experts top-6 +
            2 shared, d_ff=1408, bf16, rho=0.85, n=1..16
  v2stack   the v2lite layer stacked 26 deep, rho in {0,.5,.8,.95,.99}
  v3        DeepSeek-V3-shaped layer, d=7168, 256 routed top-8 + 1 shared,
            d_ff=2048, bf16, 4 concurrent sequences of n=1..16, rho=0.9

Hidden states follow a stationary AR(1) chain per sequence:
h_0 ~ N(0, I), h_t = rho h_{t-1} + sqrt(1 - rho^2) eps_t, so consecutive
tokens of a pass are correlated and tend to pick the same experts.

Seeds: tensor ``tid`` of layer ``L`` uses seed*1000 + L*10 + tid; the hidden
states of (rho index i, pass size n, repetition r) use
seed*10**6 + i*10**4 + n*100 + r.  Values depend on the device the draw runs
on (torch's CPU and GPU generators differ); a caller that checks GPU results
on the CPU copies the drawn tensors across.
"""
from dataclasses import dataclass, field
import math
import numpy as np

import torch

WEIGHT_STD = 0.02
T_GATE, T_W13, T_W2, T_WS13, T_WS2, T_BIAS = 0, 1, 2, 3, 4, 5
# Scale of the synthetic per-expert routing bias: a fraction of the logit
# spread of a unit-variance token, WEIGHT_STD * sqrt(d).
BIAS_REL_STD = 0.25


@dataclass(frozen=True)
class LayerConfig:
    name: str
    d: int
    E: int
    k: int
    f: int
    S: int
    wdtype: str            # "bf16" or "f32"
    rho: float
    seed: int
    n_values: tuple
    n_seq: int = 1
    layers: int = 1
    rhos: tuple = field(default_factory=tuple)

    @property
    def torch_wdtype(self):
        return torch.bfloat16 if self.wdtype == "bf16" else torch.float32

    @property
    def wbytes(self):
        return 2 if self.wdtype == "bf16" else 4

    @property
    def expert_bytes(self):
        return 3 * self.d * self.f * self.wbytes

    def tokens(self, n):
        return self.n_seq * n


CONFIGS = {
    "tiny": LayerConfig("tiny", 256, 8, 2, 512, 0, "f32", 0.9, 1, (4,)),
    "mixtral": LayerConfig("mixtral", 4096, 8, 2, 14336, 0, "bf16", 0.8, 2,
                           tuple(range(1, 9))),
    "v2lite": LayerConfig("v2lite", 2048, 64, 6, 1408, 2, "bf16", 0.85, 3,
                          tuple(range(1, 17))),
    "v2stack": LayerConfig("v2stack", 2048, 64, 6, 1408, 2, "bf16", 0.85, 4,
                           tuple(range(1, 17)), layers=26,
                           rhos=(0.0, 0.5, 0.8, 0.95, 0.99)),
    "v3": LayerConfig("v3", 7168, 256, 8, 2048, 1, "bf16", 0.9, 5,
                      tuple(range(1, 17)), n_seq=4),
}


def share_config(cfg: LayerConfig, G: int) -> LayerConfig:
    """One GPU's share of the layer when every expert (routed and shared) is
    split along d_ff over G GPUs: the same d, E, k and S, d_ff / G.  The
    gate and the hidden states stay whole (replicated on every GPU).  The
    kernels need d_ff / G to be a multiple of 32."""
    if G < 1 or cfg.f % G or (cfg.f // G) % 32:
        raise ValueError(f"d_ff = {cfg.f} does not split into {G} shares of a multiple of 32")
    return LayerConfig(f"{cfg.name}_share{G}", cfg.d, cfg.E, cfg.k, cfg.f // G, cfg.S, cfg.wdtype,
                       cfg.rho, cfg.seed, cfg.n_values, cfg.n_seq, cfg.layers, cfg.rhos)


def shard_layer(lay, G: int, g: int):
    """Share g of G of a layer's weights (make_layer's dict): rows
    [g f/G, (g+1) f/G) of W1 and W3 and the same columns of W2, for the
    routed and the shared experts; the gate whole.  Copies, contiguous."""
    f = lay["w13"].shape[2]
    if f % G:
        raise ValueError("d_ff does not split into G shares")
    a, b = g * (f // G), (g + 1) * (f // G)
    out = {"gate_w": lay["gate_w"],
           "w13": lay["w13"][:, :, a:b, :].contiguous(),
           "w2": lay["w2"][:, :, a:b].contiguous(),
           "ws13": None, "ws2": None}
    if lay.get("ws13") is not None:
        out["ws13"] = lay["ws13"][:, :, a:b, :].contiguous()
        out["ws2"] = lay["ws2"][:, :, a:b].contiguous()
    return out


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal_weights(shape, seed, device, dtype, chunk_dim0=True):
    """N(0, WEIGHT_STD) drawn in fp32, then cast (round-to-nearest-even for
    bf16).  Drawn one leading slice at a time to bound temporary memory."""
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    if not chunk_dim0 or len(shape) == 1:
        out.copy_(torch.randn(shape, generator=g, device=device) * WEIGHT_STD)
        return out
    for i in range(shape[0]):
        out[i].copy_(torch.randn(shape[1:], generator=g, device=device) * WEIGHT_STD)
    return out


def make_gate(cfg: LayerConfig, device="cpu", layer: int = 0, E=None):
    """The gate of one layer alone: fp32 [E][d], the same draw as make_layer's."""
    E = cfg.E if E is None else E
    return _normal_weights((E, cfg.d), cfg.seed * 1000 + layer * 10 + T_GATE, device,
                           torch.float32, False)


def make_layer(cfg: LayerConfig, device="cpu", layer: int = 0, E=None):
    """Weights of one layer: dict with gate_w fp32 [E][d], w13 [E][2][f][d],
    w2 [E][d][f], ws13 [S][2][f][d] / ws2 [S][d][f] (None when S == 0)."""
    E = cfg.E if E is None else E
    base = cfg.seed * 1000 + layer * 10
    wdt = cfg.torch_wdtype
    lay = {
        "gate_w": make_gate(cfg, device, layer, E),
        "w13": _normal_weights((E, 2, cfg.f, cfg.d), base + T_W13, device, wdt),
        "w2": _normal_weights((E, cfg.d, cfg.f), base + T_W2, device, wdt),
        "ws13": None,
        "ws2": None,
    }
    if cfg.S > 0:
        lay["ws13"] = _normal_weights((cfg.S, 2, cfg.f, cfg.d), base + T_WS13, device, wdt)
        lay["ws2"] = _normal_weights((cfg.S, cfg.d, cfg.f), base + T_WS2, device, wdt)
    return lay


def make_bias(cfg: LayerConfig, device="cpu", layer: int = 0, scale=BIAS_REL_STD):
    """Per-expert routing bias fp32 [E] for the DeepSeek-style biased gate:
    N(0, (scale * WEIGHT_STD * sqrt(d))^2), i.e. a set fraction of the
    spread of the logits.  The pages give no bias values (the bias is tuned
    during training), so any fixed draw of comparable scale stands in."""
    g = _gen(cfg.seed * 1000 + layer * 10 + T_BIAS, device)
    std = scale * WEIGHT_STD * math.sqrt(cfg.d)
    return (torch.randn((cfg.E,), generator=g, device=device) * std).contiguous()


def sequence_groups(cfg: LayerConfig, n: int):
    """Token boundaries of the cfg.n_seq sequences in a pass of n tokens each
    (rows s*n .. s*n+n-1 are sequence s): [0, n, 2n, ..., n_seq*n]."""
    return [s * n for s in range(cfg.n_seq + 1)]


def ar1_chain(n, d, rho, gen, device):
    """n x d stationary AR(1) chain with unit marginal variance."""
    eps = torch.randn((n, d), generator=gen, device=device)
    h = torch.empty((n, d), dtype=torch.float32, device=device)
    if n == 0:
        return h
    h[0] = eps[0]
    c = math.sqrt(max(0.0, 1.0 - rho * rho))
    for t in range(1, n):
        h[t] = rho * h[t - 1] + c * eps[t]
    return h


def hidden_seed(cfg: LayerConfig, n: int, rep: int, rho_index: int = 0):
    return cfg.seed * 10**6 + rho_index * 10**4 + n * 100 + rep


def make_hidden(cfg: LayerConfig, n: int, rep: int = 0, device="cpu", rho=None,
                rho_index: int = 0):
    """Hidden states of one verify pass: fp32 [n_seq * n][d], sequence-major
    (tokens of sequence s are rows s*n .. s*n+n-1)."""
    rho = cfg.rho if rho is None else rho
    g = _gen(hidden_seed(cfg, n, rep, rho_index), device)
    chains = [ar1_chain(n, cfg.d, rho, g, device) for _ in range(cfg.n_seq)]
    return torch.cat(chains, dim=0).contiguous()


def to_host_bits(t):
    """Host numpy view of a weight tensor: uint16 bit patterns for bf16,
    float32 otherwise."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def crafted_routing(N: int, k: int, E: int, U: int, seed: int):
    """A routing of N tokens with exactly U distinct experts, for timing the
    dedup engine at a chosen byte share: U experts drawn without
    replacement, slot (t, j) takes expert number (t*k + j) mod U of them.
    Consecutive slots of a token are distinct because k <= U, and every one
    of the U experts is used because U <= N*k.  Weights are uniform 1/k.
    Returns (idx int32 [N][k], w float32 [N][k]) as numpy arrays."""
    if not (k <= U <= min(E, N * k)):
        raise ValueError(f"U={U} outside [k, min(E, N*k)] = [{k}, {min(E, N * k)}]")
    rng = np.random.default_rng(seed)
    experts = rng.permutation(E)[:U]
    slots = np.arange(N * k).reshape(N, k)
    idx = experts[slots % U].astype(np.int32)
    w = np.full((N, k), 1.0 / k, dtype=np.float32)
    return idx, w
