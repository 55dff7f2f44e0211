"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every function include/moe_verify.h declares, arguments are
validated before anything is launched, workspace queries answer without
launching, and the host byte accounting matches the oracle bit for bit."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from speculative_decode_verify_gate_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_verify.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    names = _declared()
    for fn in ("moe_route", "moe_expert_pass_perslot", "moe_expert_pass_dedup",
               "moe_pass_bytes", "moe_route_biased", "moe_expert_pass_dedup_grouped",
               "moe_pass_bytes_grouped", "moe_verify_gate"):
        assert fn in names


def test_binding_limits_are_the_header_limits():
    text = open(HEADER).read()
    defs = {}
    for name, val in re.findall(r"^#define (MOE_\w+) (\(?[0-9 <]+\)?)", text, re.M):
        defs[name] = eval(val, {})  # integers and shifts only
    for name in ("MAX_TOKENS", "MAX_TOPK", "MAX_SLOTS", "MAX_EXPERTS", "MAX_SHARED",
                 "MAX_SEQ", "MAX_DRAFT", "MAX_VOCAB", "MAX_GROUPS", "MAX_LAYERS",
                 "FILTER_ONE_LAUNCH_ROWS", "FILTER_ONE_LAUNCH_VOCAB"):
        assert getattr(B, name) == defs["MOE_" + name], name


def test_library_exports_every_declared_symbol():
    lib = B.load()
    for fn in _declared():
        assert hasattr(lib, fn), fn


def _shape(**kw):
    base = dict(d_model=2048, n_experts=64, top_k=6, d_ff=1408, n_shared=2, wdtype="bf16")
    base.update(kw)
    return B.make_shape(**base)


FAKE = C.c_void_p(0x100000)   # never dereferenced: every case fails validation first


def _route(shape, n=4, gate=FAKE, x=FAKE, idx=FAKE, w=FAKE, ws=FAKE, nbytes=1 << 30):
    sz = C.c_size_t(nbytes)
    return B.load().moe_route(C.byref(shape), gate, x, n, None, idx, w, None, ws,
                              C.byref(sz), None), sz.value


@pytest.mark.parametrize("bad,code", [
    (dict(top_k=0), -1), (dict(top_k=65), -1), (dict(n_experts=300, top_k=6), -1),
    (dict(n_shared=5), -1), (dict(wdtype=7), -1), (dict(d_model=2040), -2),
    (dict(d_ff=1400), -2), (dict(top_k=17, n_experts=64), -1),
])
def test_bad_shapes_are_rejected(bad, code):
    shape = _shape(**{k: v for k, v in bad.items() if k != "wdtype"})
    if "wdtype" in bad:
        shape.wdtype = bad["wdtype"]
    assert _route(shape)[0] == code


def test_bad_token_counts_and_pointers_are_rejected():
    s = _shape()
    assert _route(s, n=0)[0] == -1
    assert _route(s, n=65)[0] == -1
    assert _route(_shape(top_k=16, n_experts=64), n=33)[0] == -1   # 528 slots > 512
    assert _route(s, gate=None)[0] == -1
    assert _route(s, idx=None)[0] == -1
    assert _route(s, ws=C.c_void_p(0x100010))[0] == -1              # misaligned workspace
    assert _route(s, nbytes=16)[0] == -3                             # workspace too small


def test_workspace_queries_answer_without_launching():
    for n in (1, 16, 64):
        s = _shape(n_experts=256, top_k=8, d_model=7168, d_ff=2048, n_shared=1)
        rc, need = _route(s, n=n, ws=None, nbytes=0)
        assert rc == 0 and need >= 4 * n * 256 * (7168 // 256)
        lib = B.load()
        cw = B.Weights(0x100000, 0x100000, 0x100000, 0x100000)
        for fn, extra in (("moe_expert_pass_perslot", []), ("moe_expert_pass_dedup", [None])):
            sz = C.c_size_t(0)
            rc = getattr(lib, fn)(C.byref(s), C.byref(cw), FAKE, n, FAKE, FAKE, FAKE, *extra,
                                  None, C.byref(sz), None)
            assert rc == 0
            rows = n * 8 + n * 1
            assert sz.value >= rows * 2048 * 2 + rows * 7168 * 4
            if fn.endswith("dedup"):
                assert sz.value >= rows * 2048 * 2 + rows * 7168 * 4 + 4 * (3 * 256 + 2 + n * 8)


def test_expert_pass_rejects_missing_shared_weights():
    lib = B.load()
    s = _shape()
    sz = C.c_size_t(0)
    cw = B.Weights(0x100000, 0x100000, None, None)
    rc = lib.moe_expert_pass_perslot(C.byref(s), C.byref(cw), FAKE, 4, FAKE, FAKE, FAKE,
                                     None, C.byref(sz), None)
    assert rc == -1
    s0 = _shape(n_shared=0)
    cw2 = B.Weights(0x100000, 0x100000, 0x100000, None)
    rc = lib.moe_expert_pass_perslot(C.byref(s0), C.byref(cw2), FAKE, 4, FAKE, FAKE, FAKE,
                                     None, C.byref(sz), None)
    assert rc == -1


def test_pass_bytes_matches_oracle_bit_exact():
    rng = np.random.default_rng(0)
    for (d, E, k, f, S, wd) in [(256, 8, 2, 512, 0, "f32"), (4096, 8, 2, 14336, 0, "bf16"),
                                (2048, 64, 6, 1408, 2, "bf16"), (7168, 256, 8, 2048, 1, "bf16")]:
        s = B.make_shape(d, E, k, f, S, wd)
        so = O.Shape(d, E, k, f, S, O.BF16 if wd == "bf16" else O.F32)
        for n in (1, 2, 7, 16, 64):
            if n * k > 512:
                continue
            idx = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
            assert B.pass_bytes(s, idx) == O.pass_bytes(so, idx)
    with pytest.raises(B.MoeError):
        B.pass_bytes(B.make_shape(256, 8, 2, 512), np.array([[0, 8]], dtype=np.int32))


def test_status_strings():
    lib = B.load()
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(-3) == b"workspace too small"


def test_bad_layout_and_pack_arguments_are_rejected():
    lib = B.load()
    s = _shape()
    sz = C.c_size_t(0)
    cw = B.Weights(0x100000, 0x100000, 0x100000, 0x100000, 7)
    rc = lib.moe_expert_pass_perslot(C.byref(s), C.byref(cw), FAKE, 4, FAKE, FAKE, FAKE,
                                     None, C.byref(sz), None)
    assert rc == -1
    # overlapping source and destination
    rc = lib.moe_pack_weights(C.byref(s), 2, C.c_void_p(0x100000), None,
                              C.c_void_p(0x100000 + 4096), None, None)
    assert rc == -1
    # a source without a destination
    rc = lib.moe_pack_weights(C.byref(s), 2, C.c_void_p(0x100000), None, None, None, None)
    assert rc == -1
    assert lib.moe_pack_weights(C.byref(s), -1, None, None, None, None, None) == -1
    # nothing to do is fine and launches nothing
    assert lib.moe_pack_weights(C.byref(s), 3, None, None, None, None, None) == 0


def _verify(n_seq=2, gamma=4, V=1000, mode=1, p=FAKE, q=FAKE, x=FAKE, u=FAKE, r=FAKE,
            n=FAKE, out=FAKE, ws=None, nbytes=0):
    nb = C.c_size_t(nbytes)
    return B.load().moe_verify_gate(n_seq, gamma, V, mode, p, q, x, u, r, n, out, ws,
                                    C.byref(nb), None), nb.value


def test_verify_gate_validation_and_workspace_query():
    ok, need = _verify()
    assert ok == 0
    # 256 bytes of counters + S * chunks(V) * (gamma + 1) uint64, 256-aligned
    chunks = (1000 + 2047) // 2048
    assert need == 256 + ((2 * chunks * 5 * 8 + 255) // 256) * 256
    ok, need_big = _verify(n_seq=64, gamma=63, V=152064)
    assert ok == 0 and need_big == 256 + ((64 * 75 * 64 * 8 + 255) // 256) * 256
    bad = [dict(n_seq=0), dict(n_seq=65), dict(gamma=-1), dict(gamma=64), dict(V=0),
           dict(V=(1 << 24) + 1), dict(mode=2), dict(p=None), dict(n=None), dict(out=None),
           dict(x=None), dict(q=None), dict(u=None), dict(r=None)]
    for kw in bad:
        rc, _ = _verify(**kw)
        assert rc == -1, kw
    # greedy needs neither q, u nor r; gamma 0 needs no draft tokens
    assert _verify(mode=0, q=None, u=None, r=None)[0] == 0
    assert _verify(gamma=0, x=None, q=None, u=None)[0] == 0
    # a workspace smaller than needed
    rc, _ = _verify(ws=FAKE, nbytes=need - 1)
    assert rc == -3


def _grouped(shape, n, G, gs, ws=None, nbytes=0, idx=FAKE):
    lib = B.load()
    cw = B.Weights(0x100000, 0x100000, 0x100000, 0x100000)
    sz = C.c_size_t(nbytes)
    arr = None if gs is None else (C.c_int32 * len(gs))(*gs)
    rc = lib.moe_expert_pass_dedup_grouped(C.byref(shape), C.byref(cw), FAKE, n, G, arr, idx,
                                           FAKE, FAKE, None, ws, C.byref(sz), None)
    return rc, sz.value


def test_grouped_dedup_validation_and_workspace():
    s = _shape(n_experts=256, top_k=8, d_model=7168, d_ff=2048, n_shared=1)
    n = 64
    rc1, one = _grouped(s, n, 1, [0, n])
    assert rc1 == 0
    sz = C.c_size_t(0)
    cw = B.Weights(0x100000, 0x100000, 0x100000, 0x100000)
    assert B.load().moe_expert_pass_dedup(C.byref(s), C.byref(cw), FAKE, n, FAKE, FAKE, FAKE,
                                          None, None, C.byref(sz), None) == 0
    assert one == sz.value                      # one group: the dedup workspace
    rec = ((4 * (3 * 256 + 2 + n * 8)) + 255) // 256 * 256
    rc4, four = _grouped(s, n, 4, [0, 16, 32, 48, 64])
    assert rc4 == 0 and four == one + 3 * rec   # one compaction record per group
    for G, gs in [(0, [0]), (2, [0, 64, 64]), (2, [1, 30, 64]), (2, [0, 30, 63]),
                  (3, [0, 40, 20, 64]), (65, list(range(66))), (2, None)]:
        assert _grouped(s, n, G, gs)[0] == -1, gs
    assert _grouped(s, n, 4, [0, 16, 32, 48, 64], ws=FAKE, nbytes=four - 1)[0] == -3


def test_grouped_pass_bytes_matches_oracle():
    rng = np.random.default_rng(3)
    for (d, E, k, f, S, wd) in [(256, 8, 2, 512, 0, "f32"), (7168, 256, 8, 2048, 1, "bf16"),
                                (2048, 64, 6, 1408, 2, "bf16")]:
        s = B.make_shape(d, E, k, f, S, wd)
        so = O.Shape(d, E, k, f, S, O.BF16 if wd == "bf16" else O.F32)
        for n, gs in [(4, [0, 4]), (4, [0, 1, 2, 3, 4]), (16, [0, 4, 8, 12, 16]),
                      (13, [0, 5, 6, 13]), (64, [0, 16, 32, 48, 64])]:
            if n * k > 512:
                continue
            idx = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
            got_b, got_u = B.pass_bytes_grouped(s, idx, gs)
            # oracle: the plain byte count of each group's own routing
            ref = [O.pass_bytes(so, idx[gs[g]:gs[g + 1]]) for g in range(len(gs) - 1)]
            assert got_u == [r[3] for r in ref]
            assert got_b == sum(r[1] for r in ref)
            assert B.pass_bytes(s, idx)[1] <= got_b <= B.pass_bytes(s, idx)[0]
    with pytest.raises(ValueError):
        B.pass_bytes_grouped(B.make_shape(256, 8, 2, 512), np.zeros((4, 2), np.int32), [0, 2, 3])


def _stack(shape, L=3, n=4, engine=0, w=True, ws=None, nbytes=0, gate=FAKE):
    lib = B.load()
    sw = B.StackWeights(gate.value if gate is not None else None, None, 0x100000, 0x100000,
                        0x100000, 0x100000, 0) if w else None
    sz = C.c_size_t(nbytes)
    rc = lib.moe_stack_pass(C.byref(shape), L, None if sw is None else C.byref(sw), FAKE, n,
                            engine, FAKE, FAKE, FAKE, None, ws, C.byref(sz), None)
    return rc, sz.value


def test_stack_pass_validation_and_workspace():
    s = _shape()
    lib = B.load()
    rc, need3 = _stack(s, L=3, n=16, engine=1)
    assert rc == 0
    # the head (256 bytes of counters), L layers of routing partials, then
    # the expert part (L compaction records, activation and output rows); a
    # single-layer expert pass has the same head in front of its part
    r1 = C.c_size_t(0)
    assert lib.moe_route(C.byref(s), FAKE, FAKE, 16, None, FAKE, FAKE, None, None,
                         C.byref(r1), None) == 0
    e1 = C.c_size_t(0)
    cw = B.Weights(0x100000, 0x100000, 0x100000, 0x100000)
    assert lib.moe_expert_pass_dedup(C.byref(s), C.byref(cw), FAKE, 16, FAKE, FAKE, FAKE, None,
                                     None, C.byref(e1), None) == 0
    parts = (r1.value - 256)
    assert need3 == 256 + 3 * parts + 3 * (e1.value - 256)
    rc, need_ps = _stack(s, L=3, n=16, engine=0)
    assert rc == 0 and need_ps < need3          # no compaction records
    for kw in (dict(L=0), dict(L=65), dict(engine=2), dict(w=False), dict(gate=None),
               dict(n=0), dict(n=65)):
        assert _stack(s, **kw)[0] == -1, kw
    assert _stack(s, L=3, n=16, engine=1, ws=FAKE, nbytes=need3 - 1)[0] == -3


def test_verify_probs_validation():
    lib = B.load()
    ok = dict(rows=2, V=1000, lg=FAKE, T=0.7, p=0.9, out=C.c_void_p(0x900000))
    bad = [dict(rows=0), dict(V=0), dict(V=(1 << 24) + 1), dict(lg=None), dict(out=None),
           dict(T=0.0), dict(T=-1.0), dict(T=float("inf")), dict(T=float("nan")), dict(p=0.0),
           dict(p=1.5), dict(p=float("nan")), dict(out=C.c_void_p(0x100000 + 4000))]  # overlap
    nb = C.c_size_t(0)
    for kw in bad:
        a = dict(ok, **kw)
        rc = lib.moe_verify_probs(a["rows"], a["V"], a["lg"], a["T"], a["p"], a["out"], None,
                                  C.byref(nb), None)
        assert rc == -1, kw
    # workspace query: chunk statistics, first-level histogram, candidate list, row state
    assert lib.moe_verify_probs(36, 102400, FAKE, 0.7, 0.9, C.c_void_p(0x10000000), None, C.byref(nb),
                                None) == 0
    chunks = (102400 + 4095) // 4096
    assert nb.value >= 36 * (chunks * 8 + 256 * 8 + 102400 * 8 + 64 + 16)
    assert lib.moe_verify_probs(65536, 16, FAKE, 0.7, 0.9, C.c_void_p(0x10000000), None,
                                C.byref(nb), None) == -2


def test_verify_probs_pair_validation():
    """The paired filter checks each row set as the single call does, and
    that no output overlaps an input or the other output; its workspace is
    the single call's for all rows."""
    lib = B.load()
    V = 1000
    n = 2 * V * 4
    ok = dict(rp=2, lp=FAKE, op=C.c_void_p(0x900000), rq=2, lq=C.c_void_p(0x200000),
              oq=C.c_void_p(0xA00000), V=V, T=0.7, p=0.9)
    bad = [dict(rp=0), dict(rq=0), dict(rq=-1), dict(lp=None), dict(op=None), dict(lq=None),
           dict(oq=None), dict(V=0), dict(T=0.0), dict(p=1.5),
           dict(op=C.c_void_p(0x100000 + 4000)),            # p's output over p's logits
           dict(oq=C.c_void_p(0x200000 + n - 4)),           # q's output over q's logits
           dict(op=C.c_void_p(0x200000 + 8)),               # p's output over q's logits
           dict(oq=C.c_void_p(0x100000 + 8)),               # q's output over p's logits
           dict(oq=C.c_void_p(0x900000 + n - 4))]           # the outputs overlap
    nb = C.c_size_t(0)

    def call(a, ws=None, nbytes=None):
        return lib.moe_verify_probs_pair(a["rp"], a["lp"], a["op"], a["rq"], a["lq"], a["oq"],
                                         a["V"], a["T"], a["p"], ws,
                                         C.byref(nb if nbytes is None else nbytes), None)
    for kw in bad:
        assert call(dict(ok, **kw)) == -1, kw
    # the two logits arrays may overlap (read only)
    assert call(dict(ok, lq=C.c_void_p(0x100000 + 8))) == 0
    single = C.c_size_t(0)
    assert lib.moe_verify_probs(36 + 32, 102400, FAKE, 0.7, 0.9, C.c_void_p(0x10000000), None,
                                C.byref(single), None) == 0
    pair = C.c_size_t(0)
    assert call(dict(ok, rp=36, rq=32, V=102400, op=C.c_void_p(0x10000000),
                     lq=C.c_void_p(0x20000000), oq=C.c_void_p(0x30000000)), nbytes=pair) == 0
    assert pair.value == single.value
    assert call(dict(ok, rp=40000, rq=25536, V=16, op=C.c_void_p(0x10000000),
                     lq=C.c_void_p(0x20000000), oq=C.c_void_p(0x30000000)), nbytes=pair) == -2


def test_binding_workspace_is_zero_filled_and_grow_only():
    """The binding's Workspace needs no bookkeeping between calls: the head
    that holds arrival counters is zero at allocation and every call leaves
    it zero.  It grows (zero-filled again) and never shrinks."""
    ws = B.Workspace("cpu")
    buf = ws.get(1024)
    assert buf.numel() == 1024 and int(buf.sum()) == 0
    buf[300] = 9                              # data beyond the head survives
    assert int(ws.get(512)[300]) == 9 and ws.get(512).numel() == 1024
    grown = ws.get(4096)
    assert grown.numel() == 4096 and int(grown.sum()) == 0


def test_every_workspace_reserves_the_counter_head():
    """Every device call's workspace starts with the 256-byte counter head:
    the expert passes, the grouped pass and the filter, which keep no
    counters, still ask for it and place their data after it."""
    lib = B.load()
    s = B.make_shape(512, 64, 6, 352, 2, "bf16")
    nb = C.c_size_t(0)
    n, k, E, f, d, S = 16, 6, 64, 352, 512, 2
    rec = ((3 * E + 2 + n * k) * 4 + 255) // 256 * 256
    rows = n * k + S * n
    a = (rows * f * 2 + 255) // 256 * 256
    o = (rows * d * 4 + 255) // 256 * 256
    W = B.Weights(0x100000, 0x200000, 0x300000, 0x400000, 0)
    assert lib.moe_expert_pass_dedup(C.byref(s), C.byref(W), FAKE, n, FAKE, FAKE, FAKE, None,
                                     None, C.byref(nb), None) == 0
    assert nb.value == 256 + rec + a + o
    assert lib.moe_expert_pass_perslot(C.byref(s), C.byref(W), FAKE, n, FAKE, FAKE, FAKE, None,
                                       C.byref(nb), None) == 0
    assert nb.value == 256 + a + o
    gs = (C.c_int32 * 3)(0, 5, 16)
    assert lib.moe_expert_pass_dedup_grouped(C.byref(s), C.byref(W), FAKE, n, 2, gs, FAKE, FAKE,
                                             FAKE, None, None, C.byref(nb), None) == 0
    assert nb.value == 256 + 2 * rec + a + o
    assert lib.moe_verify_probs(2, 1000, FAKE, 0.7, 0.9, C.c_void_p(0x10000000), None,
                                C.byref(nb), None) == 0
    assert nb.value >= 256 + 2 * 1000 * 8


def test_noalloc_rejects_a_pass_beyond_its_array():
    """moe_stack_pass_noalloc validates and sizes a pass before any device
    work: the V3-shaped layer stacked 8 deep at 64 tokens needs more than
    the static array (MOE_ERR_WORKSPACE), a bad engine is rejected."""
    lib = B.load()
    shape = B.make_shape(7168, 256, 8, 2048, 1, "bf16")
    sw = B.StackWeights(0x100000, None, 0x200000, 0x300000, 0x400000, 0x500000, 1)
    p = C.c_void_p(0x600000)
    assert lib.moe_stack_pass_noalloc(C.byref(shape), 8, C.byref(sw), p, 64, 1, p, p, p, None,
                                      None) == -3
    assert lib.moe_stack_pass_noalloc(C.byref(shape), 1, C.byref(sw), p, 64, 2, p, p, p, None,
                                      None) == -1
    nb = C.c_size_t(0)
    assert lib.moe_stack_pass(C.byref(shape), 1, C.byref(sw), p, 64, 1, p, p, p, None, None,
                              C.byref(nb), None) == 0
    assert nb.value < 64 << 20      # one V3-shaped layer at 64 tokens fits
