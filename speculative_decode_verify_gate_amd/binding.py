"""ctypes binding of libmoeverify.so (include/moe_verify.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the HIP stream, status codes become exceptions.  Every step of
the layer runs in the library's gfx950 kernels; there is no fallback, and
loading fails loudly when the library has not been built.  MOE_VERIFY_LIB,
if set, names another build of the same library to load instead (for
comparing two builds of the kernels in separate processes).
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_VERIFY_LIB") or os.path.join(_HERE, "libmoeverify.so")

MOE_F32, MOE_BF16 = 0, 1
MAX_TOKENS, MAX_TOPK, MAX_SLOTS, MAX_EXPERTS, MAX_SHARED = 64, 16, 512, 256, 4
KERNEL_KINDS = ("gate", "topk", "compact", "up", "down", "combine", "verify", "filter")
VERIFY_GREEDY, VERIFY_SAMPLING = 0, 1
MAX_SEQ, MAX_DRAFT, MAX_VOCAB = 64, 63, 1 << 24
FILTER_ONE_LAUNCH_ROWS, FILTER_ONE_LAUNCH_VOCAB = 128, 262144
MAX_GROUPS = 64
MAX_LAYERS = 64
ENGINE_PERSLOT, ENGINE_DEDUP = 0, 1

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


class Shape(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("d_ff", C.c_int32), ("n_shared", C.c_int32), ("wdtype", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [("w13", C.c_void_p), ("w2", C.c_void_p), ("ws13", C.c_void_p),
                ("ws2", C.c_void_p), ("layout", C.c_int32)]


class StackWeights(C.Structure):
    _fields_ = [("gate_w", C.c_void_p), ("bias", C.c_void_p), ("w13", C.c_void_p),
                ("w2", C.c_void_p), ("ws13", C.c_void_p), ("ws2", C.c_void_p),
                ("layout", C.c_int32)]


LAYOUTS = {"rows": 0, "tiled": 1}


def load():
    """Load the built library (never builds; never falls back)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m speculative_decode_verify_gate_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P, i32, sz = C.c_void_p, C.c_int32, C.POINTER(C.c_size_t)
    lib.moe_route.argtypes = [P, P, P, i32, P, P, P, P, P, sz, P]
    lib.moe_route_biased.argtypes = [P, P, P, P, i32, P, P, P, P, P, sz, P]
    lib.moe_expert_pass_dedup_grouped.argtypes = [P, P, P, i32, i32, P, P, P, P, P, P, sz, P]
    lib.moe_pass_bytes_grouped.argtypes = [P, P, i32, i32, P, P, P]
    lib.moe_stack_pass.argtypes = [P, i32, P, P, i32, i32, P, P, P, P, P, sz, P]
    lib.moe_stack_pass_noalloc.argtypes = [P, i32, P, P, i32, i32, P, P, P, P, P]
    lib.moe_expert_pass_perslot.argtypes = [P, P, P, i32, P, P, P, P, sz, P]
    lib.moe_expert_pass_dedup.argtypes = [P, P, P, i32, P, P, P, P, P, sz, P]
    lib.moe_pass_bytes.argtypes = [P, P, i32, P, P, P, P]
    lib.moe_pack_weights.argtypes = [P, i32, P, P, P, P, P]
    lib.moe_status_string.argtypes = [C.c_int]
    lib.moe_status_string.restype = C.c_char_p
    lib.moe_filter_spin_limit.argtypes = [C.c_uint32]
    lib.moe_timing_enable.argtypes = [C.c_int]
    lib.moe_timing_read.argtypes = [P, P]
    lib.moe_verify_gate.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, P, sz, P]
    lib.moe_verify_probs.argtypes = [i32, i32, P, C.c_float, C.c_float, P, P, sz, P]
    lib.moe_verify_probs_pair.argtypes = [i32, P, P, i32, P, P, i32, C.c_float, C.c_float, P,
                                          sz, P]
    for fn in ("moe_route", "moe_route_biased", "moe_expert_pass_perslot",
               "moe_expert_pass_dedup", "moe_expert_pass_dedup_grouped", "moe_pass_bytes",
               "moe_pass_bytes_grouped", "moe_stack_pass", "moe_stack_pass_noalloc",
               "moe_pack_weights",
               "moe_timing_enable",
               "moe_timing_read", "moe_verify_gate", "moe_verify_probs",
               "moe_verify_probs_pair"):
        getattr(lib, fn).restype = C.c_int
    _lib = lib
    return lib


_NEED = {}


def _shape_key(shape):
    return (shape.d_model, shape.n_experts, shape.top_k, shape.d_ff, shape.n_shared,
            shape.wdtype)


def _need(fn, shape, n, query):
    """Workspace bytes of a call, asked once per (call, shape, token count)."""
    key = (fn, _shape_key(shape), n)
    if key not in _NEED:
        need = C.c_size_t(0)
        _check(fn, query(C.byref(need)))
        _NEED[key] = need.value
    return _NEED[key]


def _check(fn, rc):
    if rc != 0:
        raise MoeError(fn, rc, load().moe_status_string(rc).decode())


def make_shape(d_model, n_experts, top_k, d_ff, n_shared=0, wdtype="bf16"):
    wd = {"bf16": MOE_BF16, "f32": MOE_F32, MOE_BF16: MOE_BF16, MOE_F32: MOE_F32}[wdtype]
    return Shape(d_model, n_experts, top_k, d_ff, n_shared, wd)


def shape_of(cfg):
    """Shape of a synth.LayerConfig."""
    return make_shape(cfg.d, cfg.E, cfg.k, cfg.f, cfg.S, cfg.wdtype)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t, dtype, name):
    if t is None:
        return None
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on the GPU "
                         f"(got {t.dtype} on {t.device}, contiguous={t.is_contiguous()})")
    return t


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class Workspace:
    """A grow-only device byte buffer reused across calls (256-byte aligned,
    zero-filled when allocated).

    The library keeps arrival counters in the first 256 bytes of every
    workspace and returns them to zero after each call; no call writes
    anything else there.  The zero fill at allocation is therefore the
    only initialisation any sequence of calls needs."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
        return self.buf


def _weights(shape, w):
    wdt = torch.bfloat16 if shape.wdtype == MOE_BF16 else torch.float32
    keep = [_dev(w["w13"], wdt, "w13"), _dev(w["w2"], wdt, "w2"),
            _dev(w.get("ws13"), wdt, "ws13"), _dev(w.get("ws2"), wdt, "ws2")]
    ptrs = [None if t is None else t.data_ptr() for t in keep]
    return keep, Weights(*ptrs, LAYOUTS[w.get("layout", "rows")])


def pack_weights(shape, weights):
    """Copy of a row-major weight dict in MOE_LAYOUT_TILED (new device
    tensors of the same shapes; the gate is shared, not copied)."""
    lib = load()
    out = dict(weights)
    out["layout"] = "tiled"
    for a, b in (("w13", "w2"), ("ws13", "ws2")):
        if weights.get(a) is None:
            continue
        src13, src2 = weights[a], weights[b]
        dst13, dst2 = torch.empty_like(src13), torch.empty_like(src2)
        _check("moe_pack_weights", lib.moe_pack_weights(
            C.byref(shape), src13.shape[0], _ptr(src13), _ptr(src2), _ptr(dst13), _ptr(dst2),
            _stream()))
        out[a], out[b] = dst13, dst2
    return out


def route(shape, gate_w, x, *, bias=None, idx=None, w=None, logits=None, margin=None,
          ws=None):
    """Gate logits, top-k and softmax over the k.  Returns (idx int32 [N][k],
    w fp32 [N][k]); logits [N][E] and margin [N] are filled when given.  With
    bias (fp32 [E]) the DeepSeek-style biased routing (moe_route_biased)."""
    lib = load()
    gate_w = _dev(gate_w, torch.float32, "gate_w")
    x = _dev(x, torch.float32, "x")
    bias = _dev(bias, torch.float32, "bias")
    if bias is not None and tuple(bias.shape) != (shape.n_experts,):
        raise ValueError(f"bias must be [{shape.n_experts}]")
    n = x.shape[0]
    if idx is None:
        idx = torch.empty((n, shape.top_k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((n, shape.top_k), dtype=torch.float32, device=x.device)
    _dev(idx, torch.int32, "idx"), _dev(w, torch.float32, "w")
    _dev(logits, torch.float32, "logits"), _dev(margin, torch.float32, "margin")
    need = _need("moe_route", shape, n, lambda nb: lib.moe_route(
        C.byref(shape), _ptr(gate_w), _ptr(x), n, None, _ptr(idx), _ptr(w), None, None, nb,
        None))
    ws = ws or Workspace(x.device)
    buf = ws.get(need)
    have = C.c_size_t(buf.numel())
    _check("moe_route_biased", lib.moe_route_biased(
        C.byref(shape), _ptr(gate_w), _ptr(bias), _ptr(x), n, _ptr(logits), _ptr(idx), _ptr(w),
        _ptr(margin), _ptr(buf), C.byref(have), _stream()))
    return idx, w


def _expert_pass(fn, shape, weights, x, idx, w, y, ws, n_unique=None, groups=None):
    lib = load()
    keep, cw = _weights(shape, weights)
    x = _dev(x, torch.float32, "x")
    idx = _dev(idx, torch.int32, "idx")
    w = _dev(w, torch.float32, "w")
    n = x.shape[0]
    if y is None:
        y = torch.empty((n, shape.d_model), dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    # grouped pass: (G, host int32 group_start) after the token count
    pre = [] if groups is None else [len(groups) - 1, (C.c_int32 * len(groups))(*groups)]
    extra = [] if n_unique is False else [None]
    need = _need((fn, None if groups is None else len(groups)), shape, n,
                 lambda nb: getattr(lib, fn)(
                     C.byref(shape), C.byref(cw), _ptr(x), n, *pre, _ptr(idx), _ptr(w), _ptr(y),
                     *extra, None, nb, None))
    ws = ws or Workspace(x.device)
    buf = ws.get(need)
    have = C.c_size_t(buf.numel())
    extra = [] if n_unique is False else [_ptr(n_unique)]
    _check(fn, getattr(lib, fn)(C.byref(shape), C.byref(cw), _ptr(x), n, *pre, _ptr(idx),
                                _ptr(w), _ptr(y), *extra, _ptr(buf), C.byref(have), _stream()))
    del keep
    return y


def expert_pass_perslot(shape, weights, x, idx, w, *, y=None, ws=None):
    """Per-slot engine.  weights: dict with w13, w2 (and ws13, ws2 when the
    shape has shared experts).  Returns y fp32 [N][d]."""
    return _expert_pass("moe_expert_pass_perslot", shape, weights, x, idx, w, y, ws,
                        n_unique=False)


def expert_pass_dedup(shape, weights, x, idx, w, *, y=None, n_unique=None, ws=None):
    """Deduplicating engine; n_unique (int32 [1] on the GPU) receives U."""
    _dev(n_unique, torch.int32, "n_unique")
    return _expert_pass("moe_expert_pass_dedup", shape, weights, x, idx, w, y, ws,
                        n_unique=n_unique)


def _group_list(group_start, n):
    gs = [int(v) for v in group_start]
    if len(gs) < 2 or len(gs) - 1 > MAX_GROUPS:
        raise ValueError(f"group_start needs 2 .. {MAX_GROUPS + 1} boundaries")
    if gs[0] != 0 or gs[-1] != n or any(b <= a for a, b in zip(gs, gs[1:])):
        raise ValueError(f"group_start must rise strictly from 0 to {n}")
    return gs


def expert_pass_dedup_grouped(shape, weights, x, idx, w, group_start, *, y=None,
                              n_unique=None, ws=None):
    """Deduplicating engine inside token groups: group g is tokens
    group_start[g] .. group_start[g+1]-1 (a host sequence).  n_unique (int32
    [G] on the GPU) receives U_g."""
    _dev(n_unique, torch.int32, "n_unique")
    gs = _group_list(group_start, x.shape[0])
    if n_unique is not None and n_unique.numel() < len(gs) - 1:
        raise ValueError("n_unique needs one entry per group")
    return _expert_pass("moe_expert_pass_dedup_grouped", shape, weights, x, idx, w, y, ws,
                        n_unique=n_unique, groups=gs)


def _stack_args(shape, stack, x, engine, idx, w, y, n_unique):
    eng = {"perslot": ENGINE_PERSLOT, "dedup": ENGINE_DEDUP}[engine]
    wdt = torch.bfloat16 if shape.wdtype == MOE_BF16 else torch.float32
    gate_w = _dev(stack["gate_w"], torch.float32, "gate_w")
    L = gate_w.shape[0]
    bias = _dev(stack.get("bias"), torch.float32, "bias")
    keep = [gate_w, bias] + [_dev(stack.get(k), wdt, k) for k in ("w13", "w2", "ws13", "ws2")]
    for t, want in ((keep[2], (L, shape.n_experts, 2, shape.d_ff, shape.d_model)),
                    (keep[3], (L, shape.n_experts, shape.d_model, shape.d_ff)),
                    (gate_w, (L, shape.n_experts, shape.d_model))):
        if tuple(t.shape) != want:
            raise ValueError(f"stack array of shape {tuple(t.shape)}, expected {want}")
    if bias is not None and tuple(bias.shape) != (L, shape.n_experts):
        raise ValueError(f"bias must be [{L}][{shape.n_experts}]")
    cw = StackWeights(*[None if t is None else t.data_ptr() for t in keep],
                      LAYOUTS[stack.get("layout", "rows")])
    x = _dev(x, torch.float32, "x")
    n = x.shape[0]
    dev = x.device
    idx = torch.empty((L, n, shape.top_k), dtype=torch.int32, device=dev) if idx is None else idx
    w = torch.empty((L, n, shape.top_k), dtype=torch.float32, device=dev) if w is None else w
    y = torch.empty((L, n, shape.d_model), dtype=torch.float32, device=dev) if y is None else y
    _dev(idx, torch.int32, "idx"), _dev(w, torch.float32, "w"), _dev(y, torch.float32, "y")
    _dev(n_unique, torch.int32, "n_unique")
    return keep, cw, eng, L, x, n, idx, w, y


def stack_pass(shape, stack, x, engine, *, idx=None, w=None, y=None, n_unique=None, ws=None):
    """One pass of the same tokens x through every layer of a stack, fused
    (moe_stack_pass).  stack: dict with gate_w fp32 [L][E][d], optional bias
    fp32 [L][E], w13 [L][E][2][f][d], w2 [L][E][d][f] (ws13 / ws2 [L][S]...
    with shared experts) and layout.  engine: "perslot" or "dedup".
    Returns (idx int32 [L][N][k], w fp32 [L][N][k], y fp32 [L][N][d]);
    n_unique (int32 [L] on the GPU) receives U per layer."""
    lib = load()
    keep, cw, eng, L, x, n, idx, w, y = _stack_args(shape, stack, x, engine, idx, w, y, n_unique)
    key = ("moe_stack_pass", L, eng)
    need = _need(key, shape, n, lambda nb: lib.moe_stack_pass(
        C.byref(shape), L, C.byref(cw), _ptr(x), n, eng, _ptr(idx), _ptr(w), _ptr(y), None,
        None, nb, None))
    ws = ws or Workspace(x.device)
    buf = ws.get(need)
    have = C.c_size_t(buf.numel())
    _check("moe_stack_pass", lib.moe_stack_pass(
        C.byref(shape), L, C.byref(cw), _ptr(x), n, eng, _ptr(idx), _ptr(w), _ptr(y),
        _ptr(n_unique), _ptr(buf), C.byref(have), _stream()))
    del keep
    return idx, w, y


def stack_pass_noalloc(shape, stack, x, engine, *, idx=None, w=None, y=None, n_unique=None):
    """stack_pass on the library's static device workspace
    (moe_stack_pass_noalloc): the call allocates nothing on the device
    (outputs not given are allocated here, by torch, before the call)."""
    lib = load()
    keep, cw, eng, L, x, n, idx, w, y = _stack_args(shape, stack, x, engine, idx, w, y, n_unique)
    _check("moe_stack_pass_noalloc", lib.moe_stack_pass_noalloc(
        C.byref(shape), L, C.byref(cw), _ptr(x), n, eng, _ptr(idx), _ptr(w), _ptr(y),
        _ptr(n_unique), _stream()))
    del keep
    return idx, w, y


def pass_bytes_grouped(shape, idx_host, group_start):
    """Requested routed bytes of a grouped dedup pass and U per group:
    (dedup_bytes, [U_g])."""
    lib = load()
    t = torch.as_tensor(idx_host).to(torch.int32).contiguous()
    if t.is_cuda:
        raise ValueError("pass_bytes_grouped takes a host routing trace")
    gs = _group_list(group_start, t.shape[0])
    G = len(gs) - 1
    out = C.c_uint64(0)
    u = (C.c_int32 * G)()
    _check("moe_pass_bytes_grouped", lib.moe_pass_bytes_grouped(
        C.byref(shape), C.c_void_p(t.data_ptr()), t.shape[0], G, (C.c_int32 * (G + 1))(*gs),
        C.byref(out), u))
    return int(out.value), [int(v) for v in u]


def pass_bytes(shape, idx_host):
    """Requested bytes of a pass from a host routing trace:
    (perslot, dedup, shared, n_unique)."""
    lib = load()
    t = torch.as_tensor(idx_host).to(torch.int32).contiguous()
    if t.is_cuda:
        raise ValueError("pass_bytes takes a host routing trace")
    out = (C.c_uint64 * 3)()
    u = C.c_int32(0)
    base = C.addressof(out)
    _check("moe_pass_bytes", lib.moe_pass_bytes(C.byref(shape), C.c_void_p(t.data_ptr()),
                                                t.shape[0], C.c_void_p(base),
                                                C.c_void_p(base + 8), C.c_void_p(base + 16),
                                                C.byref(u)))
    return int(out[0]), int(out[1]), int(out[2]), int(u.value)


def verify_gate(p, x, *, q=None, u=None, r=None, mode=VERIFY_SAMPLING, n_accepted=None,
                out=None, ws=None):
    """One verification round per sequence.  p fp32 [S][gamma+1][V], x int32
    [S][gamma], q fp32 [S][gamma][V], u fp32 [S][gamma], r int32 [S] holding
    uint32 bit patterns (sampling).  Returns (n_accepted int32 [S], tokens
    int32 [S][gamma+1])."""
    lib = load()
    p = _dev(p, torch.float32, "p")
    S, G1, V = p.shape
    gamma = G1 - 1
    x = _dev(x, torch.int32, "x")
    if tuple(x.shape) != (S, gamma):
        raise ValueError(f"x must be [{S}][{gamma}]")
    if mode == VERIFY_SAMPLING:
        q, u, r = _dev(q, torch.float32, "q"), _dev(u, torch.float32, "u"), _dev(r, torch.int32, "r")
        if q is None or u is None or r is None:
            raise ValueError("sampling needs q, u and r")
        if tuple(q.shape) != (S, gamma, V) or tuple(u.shape) != (S, gamma) or tuple(r.shape) != (S,):
            raise ValueError("q, u, r have the wrong shapes")
    else:
        q = u = r = None
    if n_accepted is None:
        n_accepted = torch.empty((S,), dtype=torch.int32, device=p.device)
    if out is None:
        out = torch.empty((S, gamma + 1), dtype=torch.int32, device=p.device)
    _dev(n_accepted, torch.int32, "n_accepted"), _dev(out, torch.int32, "out")
    key = ("verify", S, gamma, V)
    if key not in _NEED:
        nb = C.c_size_t(0)
        _check("moe_verify_gate", lib.moe_verify_gate(S, gamma, V, mode, _ptr(p), _ptr(q), _ptr(x),
                                                      _ptr(u), _ptr(r), _ptr(n_accepted),
                                                      _ptr(out), None, C.byref(nb), None))
        _NEED[key] = nb.value
    ws = ws or Workspace(p.device)
    buf = ws.get(_NEED[key])
    have = C.c_size_t(buf.numel())
    _check("moe_verify_gate", lib.moe_verify_gate(S, gamma, V, mode, _ptr(p), _ptr(q), _ptr(x),
                                                  _ptr(u), _ptr(r), _ptr(n_accepted), _ptr(out),
                                                  _ptr(buf), C.byref(have), _stream()))
    return n_accepted, out


def verify_probs(logits, temperature, top_p=1.0, *, out=None, ws=None):
    """softmax(logits / temperature) then top-p filtering, per row of an fp32
    [..., V] tensor on the GPU (moe_verify_probs).  Returns the filtered
    probabilities, same shape."""
    lib = load()
    logits = _dev(logits, torch.float32, "logits")
    V = logits.shape[-1]
    rows = logits.numel() // V
    if out is None:
        out = torch.empty_like(logits)
    _dev(out, torch.float32, "out")
    if out.shape != logits.shape:
        raise ValueError("out must have the shape of logits")
    key = ("filter", rows, V)
    if key not in _NEED:
        nb = C.c_size_t(0)
        _check("moe_verify_probs", lib.moe_verify_probs(rows, V, _ptr(logits), float(temperature),
                                                        float(top_p), _ptr(out), None,
                                                        C.byref(nb), None))
        _NEED[key] = nb.value
    ws = ws or Workspace(logits.device)
    buf = ws.get(_NEED[key])
    have = C.c_size_t(buf.numel())
    _check("moe_verify_probs", lib.moe_verify_probs(rows, V, _ptr(logits), float(temperature),
                                                    float(top_p), _ptr(out), _ptr(buf),
                                                    C.byref(have), _stream()))
    return out


def verify_probs_pair(logits_p, logits_q, temperature, top_p=1.0, *, out_p=None, out_q=None,
                      ws=None):
    """The filtering of verify_probs for the verifier's logits [..., V] and
    the draft's [..., V] (same V) in one launch sequence
    (moe_verify_probs_pair).  Returns (p, q), each bit for bit what
    verify_probs gives for its rows."""
    lib = load()
    logits_p = _dev(logits_p, torch.float32, "logits_p")
    logits_q = _dev(logits_q, torch.float32, "logits_q")
    V = logits_p.shape[-1]
    if logits_q.shape[-1] != V:
        raise ValueError("logits_p and logits_q must have the same vocabulary")
    rows_p, rows_q = logits_p.numel() // V, logits_q.numel() // V
    out_p = torch.empty_like(logits_p) if out_p is None else out_p
    out_q = torch.empty_like(logits_q) if out_q is None else out_q
    _dev(out_p, torch.float32, "out_p")
    _dev(out_q, torch.float32, "out_q")
    if out_p.shape != logits_p.shape or out_q.shape != logits_q.shape:
        raise ValueError("outputs must have the shapes of their logits")
    key = ("filter", rows_p + rows_q, V)
    if key not in _NEED:
        nb = C.c_size_t(0)
        _check("moe_verify_probs_pair",
               lib.moe_verify_probs_pair(rows_p, _ptr(logits_p), _ptr(out_p), rows_q,
                                         _ptr(logits_q), _ptr(out_q), V, float(temperature),
                                         float(top_p), None, C.byref(nb), None))
        _NEED[key] = nb.value
    ws = ws or Workspace(logits_p.device)
    buf = ws.get(_NEED[key])
    have = C.c_size_t(buf.numel())
    _check("moe_verify_probs_pair",
           lib.moe_verify_probs_pair(rows_p, _ptr(logits_p), _ptr(out_p), rows_q, _ptr(logits_q),
                                     _ptr(out_q), V, float(temperature), float(top_p), _ptr(buf),
                                     C.byref(have), _stream()))
    return out_p, out_q


def filter_spin_limit(polls=0):
    """Polls after which a one-launch filter workgroup stops waiting at a row
    barrier and writes NaN over its chunks (moe_filter_spin_limit; 0: the
    default).  For tests of that failure path."""
    _check("moe_filter_spin_limit", load().moe_filter_spin_limit(int(polls)))


def timing_enable(kinds=KERNEL_KINDS):
    """Bracket the launches of the given kernel kinds with HIP events
    (an empty sequence disables timing)."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS.index(k)
    _check("moe_timing_enable", load().moe_timing_enable(mask))


def timing_read():
    """{kind: (total_ms, launches)} accumulated since the last read."""
    ms = (C.c_double * len(KERNEL_KINDS))()
    cnt = (C.c_int64 * len(KERNEL_KINDS))()
    _check("moe_timing_read", load().moe_timing_read(C.addressof(ms), C.addressof(cnt)))
    return {k: (ms[i], int(cnt[i])) for i, k in enumerate(KERNEL_KINDS)}
