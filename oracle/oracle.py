"""ctypes marshalling for liboracle.so (test infrastructure only).

Every function takes host numpy arrays and returns numpy arrays.  bf16 weights
are numpy uint16 arrays holding the raw bit patterns.  No arithmetic of the
method happens here.
"""
import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

F32 = 0
BF16 = 1
FLAG_BOUNDARY = 1
FLAG_ORDER = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class _Shape(C.Structure):
    _fields_ = [("d", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("f", C.c_int32), ("S", C.c_int32), ("wdtype", C.c_int32)]


class _Weights(C.Structure):
    _fields_ = [("w13", C.c_void_p), ("w2", C.c_void_p),
                ("ws13", C.c_void_p), ("ws2", C.c_void_p)]


@dataclass(frozen=True)
class Shape:
    d: int
    E: int
    k: int
    f: int
    S: int = 0
    wdtype: int = BF16

    def c(self):
        return _Shape(self.d, self.E, self.k, self.f, self.S, self.wdtype)


def load():
    """Load (building first if absent) and return the oracle library."""
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        lib = C.CDLL(path)
        P = C.c_void_p
        i32 = C.c_int32
        lib.oracle_bf16_rne.argtypes = [C.c_float]
        lib.oracle_bf16_rne.restype = C.c_uint16
        lib.oracle_bf16_rne_f64.argtypes = [C.c_double]
        lib.oracle_bf16_rne_f64.restype = C.c_uint16
        lib.oracle_gate_logits.argtypes = [P, P, P, i32, P]
        lib.oracle_route.argtypes = [P, P, P, i32, C.c_double, P, P, P, P, P]
        lib.oracle_route_biased.argtypes = [P, P, P, P, i32, C.c_double, P, P, P, P, P]
        lib.oracle_layer_grouped.argtypes = [P, P, P, i32, i32, P, P, P, i32, P, P, P]
        lib.oracle_expert.argtypes = [P, P, P, P, P, P]
        lib.oracle_layer.argtypes = [P, P, P, i32, P, P, i32, i32, P, P, P]
        lib.oracle_dense_mixture.argtypes = [P, P, P, P, i32, P]
        lib.oracle_pass_bytes.argtypes = [P, P, i32, P, P, P, P]
        lib.oracle_compact.argtypes = [P, P, i32, P, P, P, P, P]
        lib.oracle_sample_index.argtypes = [P, i32, C.c_uint32]
        lib.oracle_sample_index.restype = i32
        lib.oracle_verify_gate.argtypes = [i32, i32, i32, P, P, P, P, C.c_uint32, P, P]
        lib.oracle_filter_probs.argtypes = [i32, P, C.c_double, C.c_double, P, P]
        lib.oracle_filter_probs.restype = C.c_int
        for fn in ("oracle_gate_logits", "oracle_route", "oracle_route_biased", "oracle_expert",
                   "oracle_layer", "oracle_layer_grouped", "oracle_dense_mixture",
                   "oracle_pass_bytes", "oracle_compact"):
            getattr(lib, fn).restype = C.c_int
        _LIB = lib
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _wt(shape, a):
    if a is None:
        return None
    dt = np.uint16 if shape.wdtype == BF16 else np.float32
    return np.ascontiguousarray(a, dtype=dt)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


def expert_bytes(shape: Shape) -> int:
    return 3 * shape.d * shape.f * (2 if shape.wdtype == BF16 else 4)


def bf16_rne(x):
    """bf16 bit patterns of fp32 values, nearest-even (elementwise, slow)."""
    lib = load()
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    of = out.reshape(-1)
    for i in range(flat.size):
        of[i] = lib.oracle_bf16_rne(float(flat[i]))
    return out


def bf16_rne_f64(x):
    """bf16 bit patterns of fp64 values rounded in one step, nearest-even
    (elementwise, slow)."""
    lib = load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    of = out.reshape(-1)
    for i in range(flat.size):
        of[i] = lib.oracle_bf16_rne_f64(float(flat[i]))
    return out


def gate_logits(shape: Shape, gate_w, x):
    lib = load()
    gate_w, x = _f32(gate_w), _f32(x)
    n = x.shape[0]
    out = np.empty((n, shape.E), dtype=np.float64)
    _check(lib.oracle_gate_logits(C.byref(shape.c()), _p(gate_w), _p(x), n, _p(out)),
           "oracle_gate_logits")
    return out


def route(shape: Shape, gate_w, x, tie_eps=1e-4, bias=None):
    """Returns dict(logits fp64 [N][E], idx int32 [N][k], w fp64 [N][k],
    margin fp64 [N], flags uint8 [N]).  With bias [E], the DeepSeek-style
    biased routing (oracle_route_biased)."""
    lib = load()
    gate_w, x = _f32(gate_w), _f32(x)
    n = x.shape[0]
    logits = np.empty((n, shape.E), dtype=np.float64)
    idx = np.empty((n, shape.k), dtype=np.int32)
    w = np.empty((n, shape.k), dtype=np.float64)
    margin = np.empty((n,), dtype=np.float64)
    flags = np.empty((n,), dtype=np.uint8)
    outs = (_p(logits), _p(idx), _p(w), _p(margin), _p(flags))
    if bias is None:
        _check(lib.oracle_route(C.byref(shape.c()), _p(gate_w), _p(x), n, float(tie_eps), *outs),
               "oracle_route")
    else:
        b = _f32(bias).reshape(shape.E)
        _check(lib.oracle_route_biased(C.byref(shape.c()), _p(gate_w), _p(b), _p(x), n,
                                       float(tie_eps), *outs), "oracle_route_biased")
    return dict(logits=logits, idx=idx, w=w, margin=margin, flags=flags)


def expert(shape: Shape, W1, W3, W2, x):
    """One SwiGLU expert on one token x [d]."""
    lib = load()
    W1, W3, W2 = _wt(shape, W1), _wt(shape, W3), _wt(shape, W2)
    x = _f32(x)
    out = np.empty((shape.d,), dtype=np.float64)
    _check(lib.oracle_expert(C.byref(shape.c()), _p(W1), _p(W3), _p(W2), _p(x), _p(out)),
           "oracle_expert")
    return out


def _weights(shape, w13, w2, ws13, ws2):
    arrs = [_wt(shape, w13), _wt(shape, w2), _wt(shape, ws13), _wt(shape, ws2)]
    return arrs, _Weights(*[None if a is None else a.ctypes.data for a in arrs])


def layer(shape: Shape, w13, w2, ws13, ws2, x, idx, w, engine="perslot", n_threads=1):
    """Returns (y fp64 [N][d], routed_bytes, shared_bytes, n_unique)."""
    lib = load()
    keep, cw = _weights(shape, w13, w2, ws13, ws2)
    x = _f32(x)
    idx = _i32(idx)
    w = np.ascontiguousarray(w, dtype=np.float64)
    n = x.shape[0]
    y = np.empty((n, shape.d), dtype=np.float64)
    b = np.zeros((2,), dtype=np.uint64)
    u = np.zeros((1,), dtype=np.int32)
    eng = {"perslot": 0, "dedup": 1}[engine]
    _check(lib.oracle_layer(C.byref(shape.c()), C.byref(cw), _p(x), n, _p(idx), _p(w), eng,
                            int(n_threads), _p(y), _p(b), _p(u)), "oracle_layer")
    del keep
    return y, int(b[0]), int(b[1]), int(u[0])


def layer_grouped(shape: Shape, w13, w2, ws13, ws2, x, idx, w, group_start, n_threads=1):
    """Dedup inside token groups.  Returns (y fp64 [N][d], routed_bytes,
    shared_bytes, n_unique per group [G])."""
    lib = load()
    keep, cw = _weights(shape, w13, w2, ws13, ws2)
    x = _f32(x)
    idx = _i32(idx)
    w = np.ascontiguousarray(w, dtype=np.float64)
    gs = _i32(group_start)
    G = gs.size - 1
    n = x.shape[0]
    y = np.empty((n, shape.d), dtype=np.float64)
    b = np.zeros((2,), dtype=np.uint64)
    u = np.zeros((max(G, 1),), dtype=np.int32)
    _check(lib.oracle_layer_grouped(C.byref(shape.c()), C.byref(cw), _p(x), n, G, _p(gs),
                                    _p(idx), _p(w), int(n_threads), _p(y), _p(b), _p(u)),
           "oracle_layer_grouped")
    del keep
    return y, int(b[0]), int(b[1]), u[:G].copy()


def dense_mixture(shape: Shape, gate_w, w13, w2, ws13, ws2, x):
    lib = load()
    keep, cw = _weights(shape, w13, w2, ws13, ws2)
    gate_w, x = _f32(gate_w), _f32(x)
    n = x.shape[0]
    y = np.empty((n, shape.d), dtype=np.float64)
    _check(lib.oracle_dense_mixture(C.byref(shape.c()), _p(gate_w), C.byref(cw), _p(x), n,
                                    _p(y)), "oracle_dense_mixture")
    del keep
    return y


def pass_bytes(shape: Shape, idx):
    """Returns (perslot_bytes, dedup_bytes, shared_bytes, n_unique)."""
    lib = load()
    idx = _i32(idx)
    n = idx.shape[0]
    out = np.zeros((3,), dtype=np.uint64)
    u = np.zeros((1,), dtype=np.int32)
    o = out.ctypes.data
    _check(lib.oracle_pass_bytes(C.byref(shape.c()), _p(idx), n, C.c_void_p(o),
                                 C.c_void_p(o + 8), C.c_void_p(o + 16), _p(u)),
           "oracle_pass_bytes")
    return int(out[0]), int(out[1]), int(out[2]), int(u[0])


def compact(shape: Shape, idx):
    """Returns dict(counts [E], offs [E+1], list [N*k], uniq [U], n_unique)."""
    lib = load()
    idx = _i32(idx)
    n = idx.shape[0]
    E = shape.E
    counts = np.empty((E,), dtype=np.int32)
    offs = np.empty((E + 1,), dtype=np.int32)
    lst = np.empty((n * shape.k,), dtype=np.int32)
    uniq = np.empty((E,), dtype=np.int32)
    u = np.zeros((1,), dtype=np.int32)
    _check(lib.oracle_compact(C.byref(shape.c()), _p(idx), n, _p(counts), _p(offs), _p(lst),
                              _p(uniq), _p(u)), "oracle_compact")
    U = int(u[0])
    return dict(counts=counts, offs=offs, list=lst, uniq=uniq[:U].copy(), n_unique=U)


GREEDY = 0
SAMPLING = 1


def sample_index(weights, r):
    """Inverse-CDF index over floor(w * 2^40) weights with 32-bit uniform r
    (-1 if every weight quantizes to zero)."""
    w = np.ascontiguousarray(weights, dtype=np.float32)
    return int(load().oracle_sample_index(w.ctypes.data, w.size, int(r) & 0xFFFFFFFF))


def verify_gate(p, x, *, q=None, u=None, r=0, mode=SAMPLING):
    """One verification round for one sequence: p [gamma+1][V], q [gamma][V],
    x [gamma], u [gamma], r uint32.  Returns (n_accepted, tokens [gamma+1])."""
    p = np.ascontiguousarray(p, dtype=np.float32)
    gamma = p.shape[0] - 1
    V = p.shape[1]
    x = np.ascontiguousarray(x, dtype=np.int32).reshape(gamma)
    qa = None if q is None else np.ascontiguousarray(q, dtype=np.float32)
    ua = None if u is None else np.ascontiguousarray(u, dtype=np.float32).reshape(gamma)
    n = np.zeros(1, np.int32)
    t = np.zeros(gamma + 1, np.int32)
    rc = load().oracle_verify_gate(gamma, V, mode, p.ctypes.data,
                                   None if qa is None else qa.ctypes.data, x.ctypes.data,
                                   None if ua is None else ua.ctypes.data,
                                   int(r) & 0xFFFFFFFF, n.ctypes.data, t.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_verify_gate: bad arguments")
    return int(n[0]), t


def filter_probs(logits, temperature, top_p):
    """softmax(logits / temperature) then top-p filtering, per row of a
    [..., V] array.  Returns (probs fp64, boundary gap per row)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    V = lg.shape[-1]
    rows = lg.reshape(-1, V)
    out = np.empty(rows.shape, dtype=np.float64)
    gaps = np.empty(rows.shape[0], dtype=np.float64)
    lib = load()
    for i in range(rows.shape[0]):
        g = np.zeros(1, np.float64)
        _check(lib.oracle_filter_probs(V, rows[i].ctypes.data, float(temperature), float(top_p),
                                       out[i].ctypes.data, g.ctypes.data), "oracle_filter_probs")
        gaps[i] = g[0]
    return out.reshape(lg.shape), gaps.reshape(lg.shape[:-1])
