#!/usr/bin/env python3
"""Benchmark: µs and effective HBM GB/s per n-token MoE verify pass, per-slot
vs dedup, on one MI355X.

Workload (default): the DeepSeek-V2-Lite-shaped MoE layer (d_model 2048, 64
routed experts top-6 + 2 shared, SwiGLU d_ff 1408, bf16 weights, fp32 gate),
hidden states an AR(1) chain with rho 0.85, verify passes of n = 1..16
tokens.  Weights and inputs are seeded synthetic draws made on the GPU.

A step is one verify pass of n tokens (default n = 16) through the whole
path for both engines: gate + top-k + softmax, then the per-slot expert pass;
gate + top-k + softmax, then the dedup expert pass (compaction, expert FFNs,
shared experts, combine).  Each engine call streams a different layer from a
rotation of weight sets larger than the on-chip caches, so no call finds the
previous call's experts cached.  `value` is the step's algorithmic bytes
(gate + requested expert bytes of both engines) over its time, inputs
resident in HBM.

The last stdout line is the compact headline (under 4 KB): the value, the
roofline of the dominant kernel (the W1/W3 + SwiGLU kernel of the dedup
engine, whose bytes all come from HBM; per engine the up and down kernels,
each timed with HIP events on the launch stream), the n = 1..16 sweep (µs
and requested GB/s per engine, mean U, r(n)), the measured and predicted
crossovers and how a bandwidth error moves them, the saving checks, and the
CPU oracle timed on this host as a reported baseline.  The full record
(per-pass percentiles, calibration fits, draft-length tables, verification
round, fused stack) goes to the --details file.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from speculative_decode_verify_gate_amd import binding as B  # noqa: E402
from speculative_decode_verify_gate_amd import draftlen  # noqa: E402
from speculative_decode_verify_gate_amd import stepmodel  # noqa: E402
from speculative_decode_verify_gate_amd import synth  # noqa: E402

METRIC = "µs & effective HBM GB/s per n-token MoE verify pass, per-slot vs dedup"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Engines:
    """Route + expert pass for both engines with reusable workspaces."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.shape = B.shape_of(cfg)
        self.ws_route = B.Workspace()
        self.ws_ps = B.Workspace()
        self.ws_dd = B.Workspace()
        self.nu = torch.zeros((1,), dtype=torch.int32, device="cuda")

    def route(self, lay, x):
        return B.route(self.shape, lay["gate_w"], x, ws=self.ws_route)

    def perslot(self, lay, x, idx, w, y):
        return B.expert_pass_perslot(self.shape, lay, x, idx, w, y=y, ws=self.ws_ps)

    def dedup(self, lay, x, idx, w, y):
        return B.expert_pass_dedup(self.shape, lay, x, idx, w, y=y, n_unique=self.nu,
                                   ws=self.ws_dd)


def make_stack(cfg, shape, n_layers):
    """The weight sets, stored back to back as one stack ([L][...] arrays,
    MFMA-tiled, packed once) and as per-layer views of it."""
    wdt = cfg.torch_wdtype
    E, S, d, f = cfg.E, cfg.S, cfg.d, cfg.f
    stack = {"gate_w": torch.empty((n_layers, E, d), dtype=torch.float32, device="cuda"),
             "w13": torch.empty((n_layers, E, 2, f, d), dtype=wdt, device="cuda"),
             "w2": torch.empty((n_layers, E, d, f), dtype=wdt, device="cuda"),
             "ws13": torch.empty((n_layers, S, 2, f, d), dtype=wdt, device="cuda") if S else None,
             "ws2": torch.empty((n_layers, S, d, f), dtype=wdt, device="cuda") if S else None,
             "layout": "tiled"}
    for L in range(n_layers):
        rows = synth.make_layer(cfg, "cuda", layer=L)
        packed = B.pack_weights(shape, rows)
        for k in ("gate_w", "w13", "w2", "ws13", "ws2"):
            if stack[k] is not None:
                stack[k][L].copy_(packed[k])
        torch.cuda.synchronize()
        del rows, packed
        log(f"[bench] weights {L + 1}/{n_layers} drawn and packed")
    layers = [{k: (None if stack[k] is None else stack[k][L])
               for k in ("gate_w", "w13", "w2", "ws13", "ws2")} | {"layout": "tiled"}
              for L in range(n_layers)]
    return stack, layers


def fused_stack_leg(cfg, stack, n_values, reps, rho=None, rho_index=0):
    """The whole stack in one fused call per engine (moe_stack_pass: one
    routing launch for every layer's gate, one up, down and combine launch
    over every layer's instances), per n: median of `reps` calls on fresh
    hidden states.  Returns {n: {engine: (stack_us, U per layer)}}."""
    shape = B.shape_of(cfg)
    nL = stack["gate_w"].shape[0]
    out = {}
    ws = {"perslot": B.Workspace(), "dedup": B.Workspace()}
    for n in n_values:
        N = cfg.tokens(n)
        xs = [synth.make_hidden(cfg, n, rep, "cuda", rho=rho, rho_index=rho_index)
              for rep in range(reps)]
        idx = torch.empty((nL, N, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((nL, N, cfg.k), dtype=torch.float32, device="cuda")
        y = torch.empty((nL, N, cfg.d), dtype=torch.float32, device="cuda")
        nu = torch.zeros((reps, nL), dtype=torch.int32, device="cuda")
        for name in ("perslot", "dedup"):   # warm the workspaces
            B.stack_pass(shape, stack, xs[0], name, idx=idx, w=w, y=y, ws=ws[name])
        torch.cuda.synchronize()
        evs = {"perslot": [], "dedup": []}
        hold_gpu(0.05 * reps)
        for rep in range(reps):
            for name in ("perslot", "dedup"):
                e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                e0.record()
                B.stack_pass(shape, stack, xs[rep], name, idx=idx, w=w, y=y,
                             n_unique=nu[rep] if name == "dedup" else None, ws=ws[name])
                e1.record()
                evs[name].append((e0, e1))
        torch.cuda.synchronize()
        out[n] = {name: float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs[name]]))
                  for name in evs}
        out[n]["U"] = nu.cpu().numpy().astype(np.float64)
    return out


def hold_gpu(ms):
    """Keep the current stream busy for about `ms` milliseconds (a spin
    kernel), so that work queued behind it starts back to back."""
    torch.cuda._sleep(int(max(ms, 1.0) * 2.4e6))


def expert_bytes(cfg):
    return 3 * cfg.d * cfg.f * cfg.wbytes


def gate_bytes(cfg):
    return cfg.d * cfg.E * 4


def unique_count(idx_host, E):
    v = idx_host.reshape(-1)
    v = v[(v >= 0) & (v < E)]
    return int(np.unique(v).size)


SHORT_PASS_US = 50.0   # passes shorter than this get at least SHORT_PASS_REPS repetitions
SHORT_PASS_REPS = 200


class SweepLog:
    """Finished sweep points as JSON lines keyed by (leg, workload, rho, n,
    passes): a run given the same file (--resume) takes the points it finds
    there instead of measuring them again and appends the ones it measures,
    so an interrupted sweep continues where it stopped.  A line cut short by
    the interruption is ignored."""

    def __init__(self, path):
        self.path = path
        self.done = {}
        if path and os.path.exists(path):
            with open(path) as f:
                for line in f:
                    try:
                        d = json.loads(line)
                        self.done[self._k(d["key"])] = d["record"]
                    except (json.JSONDecodeError, KeyError, TypeError):
                        continue

    @staticmethod
    def _k(key):
        return json.dumps(key, sort_keys=True)

    def get(self, key):
        return self.done.get(self._k(key))

    def put(self, key, rec):
        if not self.path:
            return
        self.done[self._k(key)] = rec
        os.makedirs(os.path.dirname(os.path.abspath(self.path)), exist_ok=True)
        with open(self.path, "a+b") as f:
            # a line cut short by an interruption gets its end first, so the
            # new record starts a line of its own
            if f.seek(0, os.SEEK_END) > 0:
                f.seek(-1, os.SEEK_END)
                if f.read(1) != b"\n":
                    f.write(b"\n")
            f.write((json.dumps({"key": key, "record": rec}) + "\n").encode())
            f.flush()
            os.fsync(f.fileno())


def run_sweep(cfg, eng, layers, xs, n_values, reps, top_up=True, points=None):
    """Per n: reps passes per engine (topped up to SHORT_PASS_REPS when an
    engine's median pass is under SHORT_PASS_US), each on the next layer of
    the rotation, each on its own hidden states.  Returns per-n records;
    with `points` (a SweepLog), n already there is taken from it."""
    out = []
    nL = len(layers)
    turn = 0
    Be = expert_bytes(cfg)

    def batch(n, y, reps_range):
        nonlocal turn
        ev = []
        # keep the GPU busy while the host queues the whole batch, so that no
        # event pair measures host launch latency
        hold_gpu(0.3 * len(reps_range))
        for rep in reps_range:
            if (n, rep) not in xs:
                xs[(n, rep)] = synth.make_hidden(cfg, n, rep, "cuda")
            x = xs[(n, rep)]
            rec = {}
            for name in ("perslot", "dedup"):
                lay = layers[turn % nL]
                turn += 1
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record()
                idx, w = eng.route(lay, x)
                e1.record()
                getattr(eng, name)(lay, x, idx, w, y)
                e2.record()
                rec[name] = (e0, e1, e2, idx)
            ev.append(rec)
        torch.cuda.synchronize()
        return ev

    for n in n_values:
        N = cfg.tokens(n)
        key = {"leg": "sweep", "workload": cfg.name, "rho": cfg.rho, "n": n, "passes": reps}
        done = points.get(key) if points else None
        if done is not None:
            out.append(done)
            log(f"  n={n:2d} taken from the sweep log")
            continue
        y = torch.empty((N, cfg.d), dtype=torch.float32, device="cuda")
        ev = batch(n, y, range(reps))
        short = min(float(np.median([rec[name][1].elapsed_time(rec[name][2]) * 1e3 for rec in ev]))
                    for name in ("perslot", "dedup")) < SHORT_PASS_US
        if top_up and short and reps < SHORT_PASS_REPS:
            ev += batch(n, y, range(reps, SHORT_PASS_REPS))
        torch.cuda.synchronize()
        t = {"perslot": [], "dedup": []}
        tr = {"perslot": [], "dedup": []}
        tt = {"perslot": [], "dedup": []}
        U = {"perslot": [], "dedup": []}
        for rec in ev:
            for name, (e0, e1, e2, idx) in rec.items():
                tr[name].append(e0.elapsed_time(e1) * 1e3)
                tt[name].append(e0.elapsed_time(e2) * 1e3)
                t[name].append(e1.elapsed_time(e2) * 1e3)
                U[name].append(unique_count(idx.cpu().numpy(), cfg.E))
        k, S = cfg.k, cfg.S
        r = {"n": n, "tokens": N, "passes": len(ev)}
        for name in ("perslot", "dedup"):
            us = float(np.median(t[name]))
            routed = (N * k * Be) if name == "perslot" else float(np.mean(U[name])) * Be
            req = routed + S * Be
            r[name] = {"us": round(us, 2), "us_p10": round(float(np.percentile(t[name], 10)), 2),
                       "us_p90": round(float(np.percentile(t[name], 90)), 2),
                       "route_us": round(float(np.median(tr[name])), 2),
                       "total_us": round(float(np.median(tt[name])), 2),
                       "requested_MB": round(req / 1e6, 3),
                       "GBs": round(req / us / 1e3, 1),
                       "req_frac": round(req / us / 1e3 / HBM_PEAK_GBS, 3),
                       "routed_GBs": round(routed / us / 1e3, 1)}
        u_bar = float(np.mean(U["dedup"])) / (N * k)
        r["u_bar"] = round(u_bar, 4)
        r["U_mean"] = round(float(np.mean(U["dedup"])), 2)
        r["U_median"] = float(np.median(U["dedup"]))
        # r(n): effective routed-byte bandwidth of dedup over that of per-slot
        r["r"] = round(r["dedup"]["routed_GBs"] / r["perslot"]["routed_GBs"], 4)
        r["dedup_faster"] = r["dedup"]["us"] < r["perslot"]["us"]
        if points:
            points.put(key, r)
        out.append(r)
        log(f"  n={n:2d} perslot {r['perslot']['us']:8.1f} us {r['perslot']['GBs']:7.0f} GB/s | "
            f"dedup {r['dedup']['us']:8.1f} us {r['dedup']['GBs']:7.0f} GB/s | "
            f"u={u_bar:.3f} r={r['r']:.3f}")
    return out


def calibrate(cfg, eng, layers, xs, xreps, sweep, reps):
    """One-layer calibration of the step-time model t = B / BW + t0.
    Per-slot: B = N k B_e at every n, timed on the standard routing trace
    (the sweep).  Dedup: at every n, crafted routings with exactly U
    distinct experts for U spread over k .. min(E, N k), B = U B_e.  Shared
    experts and the gate are the same in both engines and land in t0.
    The per-slot engine is also timed on the same crafted routings, for the
    trace-aware fit t = U B_e / BW_first + (N k - U) B_e / BW_repeat + t0.
    Returns the fits and, per n, r(n) = BW_dd(n) / BW_ps."""
    Be = expert_bytes(cfg)
    k, E = cfg.k, cfg.E
    ns = [r["n"] for r in sweep]
    fit_ps = stepmodel.fit_line([cfg.tokens(n) * k * Be for n in ns],
                                [r["perslot"]["us"] for r in sweep])
    nL = len(layers)
    turn = 0
    points = []
    ps_points = []  # (first-read bytes, repeat bytes, us) of per-slot on crafted routings
    per_n = {}
    for n in ns:
        N = cfg.tokens(n)
        y = torch.empty((N, cfg.d), dtype=torch.float32, device="cuda")
        grid = sorted({int(round(u)) for u in np.linspace(k, min(E, N * k), 6)})
        meas = []
        for gi, U in enumerate(grid):
            idx_np, w_np = synth.crafted_routing(N, k, E, U, seed=cfg.seed * 10**4 + n * 100 + gi)
            idx = torch.from_numpy(idx_np).cuda()
            w = torch.from_numpy(w_np).cuda()
            evs = {"dedup": [], "perslot": []}
            hold_gpu(0.2 * reps)
            for rep in range(reps):
                for name in ("dedup", "perslot"):
                    lay = layers[turn % nL]
                    turn += 1
                    e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                    e0.record()
                    getattr(eng, name)(lay, xs[(n, rep % xreps)], idx, w, y)
                    e1.record()
                    evs[name].append((e0, e1))
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs["dedup"]]))
            us_ps = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs["perslot"]]))
            meas.append((U, us, us_ps))
            points.append((n, U * Be, us))
            ps_points.append((U * Be, (N * k - U) * Be, us_ps))
        rec = {"U": [m[0] for m in meas], "us": [round(m[1], 2) for m in meas],
               "perslot_us": [round(m[2], 2) for m in meas]}
        if len(grid) >= 2:
            f = stepmodel.fit_line([m[0] * Be for m in meas], [m[1] for m in meas])
            r, r_sd = stepmodel.bandwidth_ratio(f, fit_ps)
            rec.update({"fit": f.as_dict(), "r": round(r, 4), "r_sd": round(r_sd, 4)})
            rec["_fit"] = f
        per_n[n] = rec
        log(f"  calib n={n:2d} U={rec['U']} us={rec['us']}"
            + (f" r={rec['r']:.3f}" if "r" in rec else ""))
    fit_dd = stepmodel.fit_line([p[1] for p in points], [p[2] for p in points])
    r_all, r_all_sd = stepmodel.bandwidth_ratio(fit_dd, fit_ps)
    plane = stepmodel.fit_plane(*zip(*ps_points))
    log(f"  per-slot on crafted routings: {plane.as_dict()}")
    return {"perslot": fit_ps, "dedup_pooled": fit_dd, "r_pooled": (r_all, r_all_sd),
            "perslot_trace": plane, "per_n": per_n}


def predict_from_calibration(cfg, calib, n, u_bar):
    """Model prediction at pass size n and byte share u: (r(n), its standard
    error, saving us, its first-order standard error, the standard deviation
    of a measured saving about it).  Uses the per-n dedup fit where one
    exists, else the pooled one."""
    N = cfg.tokens(n)
    b_ps = N * cfg.k * expert_bytes(cfg)
    rec = calib["per_n"].get(n, {})
    f_dd = rec.get("_fit", calib["dedup_pooled"])
    r, r_sd = stepmodel.bandwidth_ratio(f_dd, calib["perslot"])
    sav, sav_sd = stepmodel.predicted_saving(calib["perslot"], f_dd, b_ps, u_bar * b_ps)
    iv_sd = stepmodel.saving_interval_sd(calib["perslot"], f_dd, b_ps, u_bar * b_ps)
    trace = stepmodel.predicted_saving_trace(calib["perslot_trace"], f_dd, u_bar * b_ps,
                                             (1.0 - u_bar) * b_ps)
    return r, r_sd, sav, sav_sd, iv_sd, trace


def saving_check(rec, measured, sav, sav_sd, iv_sd, trace):
    """Record the predicted saving (the line model, and the trace-aware one
    that prices repeated per-slot reads separately), their errors and
    whether the measured saving lies within two standard deviations of the
    line model's parameter error (the calibration's own bound), and within
    two of the wider interval that adds each fit's residual scatter."""
    rec["predicted_saving_us"], rec["predicted_saving_sd_us"] = round(sav, 2), round(sav_sd, 2)
    rec["saving_within_param_2sd"] = bool(abs(measured - sav) <= 2 * sav_sd)
    rec["saving_interval_sd_us"] = round(iv_sd, 2)
    rec["saving_within_2sd"] = bool(abs(measured - sav) <= 2 * iv_sd)
    t_sav, t_sd, t_iv = trace
    rec["trace_predicted_saving_us"], rec["trace_saving_interval_sd_us"] = round(t_sav, 2), round(t_iv, 2)
    rec["trace_saving_within_2sd"] = bool(abs(measured - t_sav) <= 2 * t_iv)


def draft_length_table(sweep, draft_fracs=(0.05, 0.2), alphas=None):
    """Best draft length per acceptance rate from the measured single-layer
    verify-pass times t(n) (route + expert pass, medians of the sweep), for
    each engine and for the faster of the two at every n.  The draft's time
    per token is a fraction of t(1)."""
    alphas = alphas or [0.3, 0.5, 0.6, 0.7, 0.8, 0.85, 0.9, 0.95, 0.98]
    t = {name: {r["n"]: r[name]["us"] + r[name]["route_us"] for r in sweep}
         for name in ("perslot", "dedup")}
    t["faster"] = {n: min(t["perslot"][n], t["dedup"][n]) for n in t["perslot"]}
    gmax = max(t["perslot"]) - 1
    out = {"model": "best gamma maximises E[k] / (t(gamma+1) + gamma t_draft) over "
                    f"0..{gmax}; gamma 0 is plain decoding at 1 / t(1); "
                    "E[k] = (1 - alpha^(gamma+1)) / (1 - alpha)",
           "alphas": alphas, "by_draft_cost": []}
    for frac in draft_fracs:
        td = frac * t["perslot"][1]
        rec = {"t_draft_over_t1": frac, "t_draft_us": round(td, 2)}
        for name, tn in t.items():
            gs = draftlen.staircase(alphas, tn, td, gmax)
            rec[f"best_gamma_{name}"] = gs
            rec[f"speedup_{name}"] = [round(draftlen.round_rate(a, g, tn, td) * tn[1], 3)
                                      for a, g in zip(alphas, gs)]
        out["by_draft_cost"].append(rec)
    return out


def verify_gate_leg(vocabs=(102400, 129280), n_seq=4, gamma=8, reps=200, temperature=0.7,
                    top_p=0.9):
    """The verification round after the verify pass, from the models' logits:
    the verifier's and the draft's distributions (moe_verify_probs_pair:
    softmax of logits / temperature, top-p filtering, at the page's
    settings, both row sets in one launch sequence; and the verifier's
    alone, moe_verify_probs, since a draft's rows are filtered while it
    drafts), then the round
    (moe_verify_gate), each timed per call, for n_seq sequences with
    gamma drafted tokens on seeded synthetic logits.  Bytes counted: the
    filter reads and writes every row once ((2 gamma + 1) rows per sequence);
    greedy reads every row of p (n_seq (gamma+1) V fp32); sampling reads
    the row it draws from twice over the vocabulary, p and q at the first
    rejection (2 n_seq V fp32) -- the acceptance tests' scalars are not
    counted."""
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    out = []

    def timed_us(fn):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        evs = []
        hold_gpu(0.1 * reps)
        for _ in range(reps):
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))

    for V in vocabs:
        vlog = torch.randn((n_seq, gamma + 1, V), generator=g, device="cuda") * 3.0
        dlog = (vlog[:, :gamma] + 0.5 * torch.randn((n_seq, gamma, V), generator=g,
                                                     device="cuda")).contiguous()
        p = B.verify_probs(vlog, temperature, top_p)
        q = B.verify_probs(dlog, temperature, top_p)
        x = torch.multinomial(q.reshape(-1, V), 1, generator=g).reshape(n_seq, gamma)
        x = x.to(torch.int32).contiguous()
        u = torch.rand((n_seq, gamma), generator=g, device="cuda")
        r = torch.randint(-2**31, 2**31 - 1, (n_seq,), generator=g, device="cuda",
                          dtype=torch.int32)
        rec = {"vocab": V, "n_seq": n_seq, "gamma": gamma, "temperature": temperature,
               "top_p": top_p}
        rows = n_seq * (2 * gamma + 1)
        # both distributions through one launch sequence (the same settings)
        fws = B.Workspace()
        fu = timed_us(lambda: B.verify_probs_pair(vlog, dlog, temperature, top_p, out_p=p,
                                                  out_q=q, ws=fws))
        rec["filter_us"] = round(fu, 2)
        rec["filter_GBs"] = round(2 * rows * V * 4 / fu / 1e3, 1)
        # the verifier's rows alone (the draft's are filtered while drafting)
        pu = timed_us(lambda: B.verify_probs(vlog, temperature, top_p, out=p, ws=fws))
        rec["filter_p_us"] = round(pu, 2)
        rec["filter_p_GBs"] = round(2 * n_seq * (gamma + 1) * V * 4 / pu / 1e3, 1)
        for mode, name in ((B.VERIFY_GREEDY, "greedy"), (B.VERIFY_SAMPLING, "sampling")):
            ws = B.Workspace()
            us = timed_us(lambda: B.verify_gate(p, x, q=q, u=u, r=r, mode=mode, ws=ws))
            nbytes = (n_seq * (gamma + 1) * V * 4) if name == "greedy" else (2 * n_seq * V * 4)
            rec[f"{name}_us"] = round(us, 2)
            rec[f"{name}_GBs"] = round(nbytes / us / 1e3, 1)
        out.append(rec)
        log(f"  verify V={V}: filter p+q {rec['filter_us']} us, p {rec['filter_p_us']} us, "
            f"greedy {rec['greedy_us']} us, sampling {rec['sampling_us']} us")
    return out


XGMI_LINK_GBS = 153.0  # one MI355X xGMI link, each direction


def shard_doc(whole, share, G, sweep, n_layers):
    """The share sweep as a document: per n, one GPU's share pass (measured)
    and, beside it, the per-link bandwidth bound of the ring all-reduce that
    would sum the G shares' fp32 outputs, 2 (G - 1) / G x N d 4 bytes over
    one xGMI link (a lower bound: latency and RCCL's launch are not in it).
    Nothing here runs on a second GPU."""
    by_n = []
    for r in sweep:
        ar = r["tokens"] * whole.d * 4
        ring_us = 2 * (G - 1) / G * ar / (XGMI_LINK_GBS * 1e3)
        rec = dict(r)
        rec["allreduce_MB"] = round(ar / 1e6, 4)
        rec["allreduce_ring_us_bound"] = round(ring_us, 2)
        rec["G_gpu_pass_us_lower_bound"] = {
            name: round(r[name]["us"] + ring_us, 2) for name in ("perslot", "dedup")}
        by_n.append(rec)
    return {"kind": "one GPU's share of a d_ff-sharded layer",
            "workload": f"{whole.name}-shaped layer, every expert (routed and shared) split "
                        f"along d_ff over {G} GPUs: one share of d_ff {share.f} "
                        f"({share.expert_bytes} bytes per expert), gate and tokens whole; "
                        f"{whole.n_seq} sequence(s) x n = {min(share.n_values)}.."
                        f"{max(share.n_values)} tokens; {n_layers} weight sets rotated",
            "G": G, "d_ff": whole.f, "share_d_ff": share.f,
            "xgmi_link_GBs": XGMI_LINK_GBS,
            "note": "us and GB/s are one GPU's share pass (route + expert pass timed "
                    "apart; requested bytes of the share); the all-reduce figure is a "
                    "bandwidth bound, not a measurement",
            "by_n": by_n}


def calibration_json(calib):
    return {"model": "t_us = bytes / BW + t0 (routed expert bytes; shared experts and "
                     "gate in t0)",
            "perslot": calib["perslot"].as_dict(),
            "perslot_trace": dict(calib["perslot_trace"].as_dict(),
                                  model="t_us = U B_e / BW_first + (N k - U) B_e / BW_repeat + t0, "
                                        "per-slot on the crafted routings"),
            "dedup_pooled": calib["dedup_pooled"].as_dict(),
            "r_pooled": round(calib["r_pooled"][0], 4),
            "r_pooled_sd": round(calib["r_pooled"][1], 4),
            "dedup_by_n": {str(n): {k: v for k, v in rec.items() if k != "_fit"}
                           for n, rec in calib["per_n"].items()}}


def rho_point(cfg, eng, layers, stack, reps, rho, ri, n):
    """The measurements of one (rho, n) of the stack sweep: median stack-pass
    times (route only, route + per-slot, route + dedup), the mean U of the
    dedup layer passes, and the fused stack calls."""
    nL = len(layers)
    Be = expert_bytes(cfg)
    N = cfg.tokens(n)
    y = torch.empty((N, cfg.d), dtype=torch.float32, device="cuda")
    nu = torch.zeros((reps * nL,), dtype=torch.int32, device="cuda")
    xs = [synth.make_hidden(cfg, n, rep, "cuda", rho=rho, rho_index=ri) for rep in range(reps)]
    t = {"route": [], "perslot": [], "dedup": []}
    evs = []
    for rep in range(reps):
        x = xs[rep]
        row = {}
        for name in ("route", "perslot", "dedup"):
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            # the host queues the whole stack pass while the GPU waits
            hold_gpu(0.1 * nL)
            e0.record()
            for L in range(nL):
                idx, w = eng.route(layers[L], x)
                if name == "perslot":
                    eng.perslot(layers[L], x, idx, w, y)
                elif name == "dedup":
                    B.expert_pass_dedup(eng.shape, layers[L], x, idx, w, y=y,
                                        n_unique=nu[rep * nL + L:rep * nL + L + 1],
                                        ws=eng.ws_dd)
            e1.record()
            row[name] = (e0, e1)
        evs.append(row)
    torch.cuda.synchronize()
    for row in evs:
        for name, (e0, e1) in row.items():
            t[name].append(e0.elapsed_time(e1) * 1e3)
    U = nu.cpu().numpy().astype(np.float64)
    fz = fused_stack_leg(cfg, stack, [n], reps, rho=rho, rho_index=ri)[n]
    fused = {"perslot_stack_us": round(fz["perslot"], 1),
             "dedup_stack_us": round(fz["dedup"], 1),
             "perslot_layer_us": round(fz["perslot"] / nL, 2),
             "dedup_layer_us": round(fz["dedup"] / nL, 2),
             "U_mean": round(float(fz["U"].mean()), 2),
             "perslot_GBs": round((N * cfg.k + cfg.S) * Be * nL / fz["perslot"] / 1e3, 1),
             "dedup_GBs": round((fz["U"].mean() + cfg.S) * Be * nL / fz["dedup"] / 1e3, 1)}
    return {"u_bar": float(U.mean()) / (N * cfg.k), "U_mean": round(float(U.mean()), 2),
            "stack_us": {k: float(np.median(v)) for k, v in t.items()}, "fused": fused}


def rho_sweep(cfg, eng, layers, stack, calib, reps, points=None):
    """The layer stack at each rho: per (rho, n), `reps` stack passes per
    engine, each pass running every layer on the same hidden states (route
    + expert pass per layer).  A route-only stack pass is timed too, so the
    expert-pass share is the difference.  U is read from the dedup engine's
    device counter of every layer pass.  The same passes are then timed as
    one fused stack call per engine (moe_stack_pass).  With `points` (a
    SweepLog), the measurements of a (rho, n) already there are taken from
    it; what follows from the calibration is computed again."""
    nL = len(layers)
    Be = expert_bytes(cfg)
    out = []
    ns = list(cfg.n_values)
    for ri, rho in enumerate(cfg.rhos):
        recs = []
        for n in ns:
            N = cfg.tokens(n)
            key = {"leg": "rho", "workload": cfg.name, "rho": rho, "n": n, "passes": reps,
                   "layers": nL}
            m = points.get(key) if points else None
            if m is None:
                m = rho_point(cfg, eng, layers, stack, reps, rho, ri, n)
                if points:
                    points.put(key, m)
            else:
                log(f"  rho={rho:.2f} n={n:2d} taken from the sweep log")
            u_bar, med, rec_fused = m["u_bar"], m["stack_us"], m["fused"]
            ps = (med["perslot"] - med["route"]) / nL
            dd = (med["dedup"] - med["route"]) / nL
            r, r_sd, sav, sav_sd, iv_sd, trace = predict_from_calibration(cfg, calib, n, u_bar)
            rec = {"n": n, "u_bar": round(u_bar, 4), "U_mean": m["U_mean"],
                   "stack_us": {k: round(v, 1) for k, v in med.items()},
                   "perslot_layer_us": round(ps, 2), "dedup_layer_us": round(dd, 2),
                   "perslot_GBs": round((N * cfg.k + cfg.S) * Be / ps / 1e3, 1),
                   "dedup_GBs": round((m["U_mean"] + cfg.S) * Be / dd / 1e3, 1),
                   "saving_us": round(ps - dd, 2),
                   "r": round(r, 4), "r_sd": round(r_sd, 4),
                   "dedup_faster": dd < ps, "u_lt_r": u_bar < r,
                   "fused": rec_fused}
            saving_check(rec, ps - dd, sav, sav_sd, iv_sd, trace)
            recs.append(rec)
            log(f"  rho={rho:.2f} n={n:2d} u={u_bar:.3f} r={r:.3f} per-layer ps {ps:7.1f} "
                f"dd {dd:7.1f} us, saving {ps - dd:6.1f} (pred {sav:6.1f} +- {iv_sd:.1f}); "
                f"fused stack per layer ps {rec_fused['perslot_layer_us']:7.1f} "
                f"dd {rec_fused['dedup_layer_us']:7.1f} us (with routing)")
        out.append({"rho": rho, "passes_per_n": reps, "layers": nL, "by_n": recs,
                    "saving_within_2sd": f"{sum(r['saving_within_2sd'] for r in recs)} of {len(recs)}",
                    "trace_saving_within_2sd":
                        f"{sum(r['trace_saving_within_2sd'] for r in recs)} of {len(recs)}",
                    "crossover": {"measured": stepmodel.first_n(ns, [r["dedup_faster"] for r in recs]),
                                  "predicted_u_lt_r": stepmodel.first_n(ns, [r["u_lt_r"] for r in recs])}})
    return out


def variants_leg(cfg, eng, layers, n_values, reps):
    """The layer variants on the same passes.  Per n and repetition, three
    engine calls on the next layers of the rotation -- per-slot, dedup over
    the union of the sequences' tokens, and dedup per sequence (one token
    group per sequence, moe_expert_pass_dedup_grouped) -- each after its
    own plain route, and one DeepSeek-style biased route (per-expert bias,
    moe_route_biased) timed alone.  U of every dedup pass is read from the
    engines' device outputs."""
    nL = len(layers)
    Be = expert_bytes(cfg)
    bias = [synth.make_bias(cfg, "cuda", layer=L) for L in range(nL)]
    out = []
    turn = 0
    names = ("perslot", "union", "perseq")
    for n in n_values:
        N = cfg.tokens(n)
        gs = synth.sequence_groups(cfg, n)
        G = len(gs) - 1
        y = torch.empty((N, cfg.d), dtype=torch.float32, device="cuda")
        nu_u = torch.zeros((reps,), dtype=torch.int32, device="cuda")
        nu_g = torch.zeros((reps, G), dtype=torch.int32, device="cuda")
        ws_g = B.Workspace()
        xs = [synth.make_hidden(cfg, n, rep, "cuda") for rep in range(reps)]
        idx_b = []
        evs = []
        hold_gpu(0.5 * reps)
        for rep in range(reps):
            x = xs[rep]
            row = {}
            for name in names:
                lay = layers[turn % nL]
                turn += 1
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record()
                idx, w = eng.route(lay, x)
                e1.record()
                if name == "perslot":
                    eng.perslot(lay, x, idx, w, y)
                elif name == "union":
                    B.expert_pass_dedup(eng.shape, lay, x, idx, w, y=y,
                                        n_unique=nu_u[rep:rep + 1], ws=eng.ws_dd)
                else:
                    B.expert_pass_dedup_grouped(eng.shape, lay, x, idx, w, gs, y=y,
                                                n_unique=nu_g[rep], ws=ws_g)
                e2.record()
                row[name] = (e0, e1, e2)
            L = turn % nL
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            ib, _ = B.route(eng.shape, layers[L]["gate_w"], x, bias=bias[L], ws=eng.ws_route)
            e1.record()
            row["route_bias"] = (e0, e1)
            idx_b.append(ib)
            evs.append(row)
        torch.cuda.synchronize()
        t = {k: [] for k in names + ("route", "route_bias")}
        for row in evs:
            for name in names:
                e0, e1, e2 = row[name]
                t["route"].append(e0.elapsed_time(e1) * 1e3)
                t[name].append(e1.elapsed_time(e2) * 1e3)
            t["route_bias"].append(row["route_bias"][0].elapsed_time(row["route_bias"][1]) * 1e3)
        med = {k: float(np.median(v)) for k, v in t.items()}
        U_u = float(nu_u.cpu().numpy().mean())
        U_g = nu_g.cpu().numpy().astype(np.float64)
        U_b = float(np.mean([unique_count(i.cpu().numpy(), cfg.E) for i in idx_b]))
        routed = {"perslot": N * cfg.k * Be, "union": U_u * Be, "perseq": U_g.sum(axis=1).mean() * Be}
        rec = {"n": n, "tokens": N, "sequences": G,
               "U_union": round(U_u, 2), "U_per_sequence_sum": round(float(U_g.sum(axis=1).mean()), 2),
               "U_per_sequence_mean": round(float(U_g.mean()), 2),
               "U_union_biased_route": round(U_b, 2),
               "route_us": round(med["route"], 2), "route_bias_us": round(med["route_bias"], 2)}
        for name in names:
            req = routed[name] + cfg.S * Be
            rec[name] = {"us": round(med[name], 2), "GBs": round(req / med[name] / 1e3, 1),
                         "req_frac": round(req / med[name] / 1e3 / HBM_PEAK_GBS, 3)}
        rec["union_saving_over_perseq_us"] = round(med["perseq"] - med["union"], 2)
        out.append(rec)
        log(f"  n={n:2d} x{G}: perslot {med['perslot']:8.1f} union {med['union']:8.1f} "
            f"perseq {med['perseq']:8.1f} us | U {U_u:.1f} vs sum {rec['U_per_sequence_sum']:.1f}"
            f" | route {med['route']:.1f} biased {med['route_bias']:.1f} us")
    return out


def timed_steps(cfg, eng, layers, x, steps, warmup, kernel_events=(),
                engines=("perslot", "dedup")):
    """The headline step at one pass size: K timed steps after W warmups,
    bracketed by device synchronisation; a step is route + expert pass for
    each of `engines`.  With kernel_events, the library brackets launches of
    those kernel kinds with HIP events on the launch stream; otherwise
    nothing is recorded inside the timed region."""
    nL = len(layers)
    N = x.shape[0]
    y = torch.empty((N, cfg.d), dtype=torch.float32, device="cuda")
    turn = 0
    idxs = {name: [] for name in engines}

    def one_step(keep):
        nonlocal turn
        for name in engines:
            lay = layers[turn % nL]
            turn += 1
            idx, w = eng.route(lay, x)
            getattr(eng, name)(lay, x, idx, w, y)
            if keep:
                idxs[name].append(idx)

    for _ in range(warmup):
        one_step(False)
    torch.cuda.synchronize()
    B.timing_read()            # drop anything recorded before
    if kernel_events:
        B.timing_enable(kernel_events)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    B.timing_enable(())
    kt = B.timing_read()
    U = {k: [unique_count(i.cpu().numpy(), cfg.E) for i in v] for k, v in idxs.items()}
    return wall, kt, U


def timeline_leg(cfg, eng, layers, n_values, steps, warmup):
    """Per pass size and engine: W warmup steps, then K steps of route +
    expert pass queued while a spin kernel holds the GPU, so that a kernel
    trace of the run shows each launch's duration and the gaps between
    launches as the GPU sees them (no host launch latency).  Cases run in
    the order n, then per-slot before dedup; the wall time per step is
    reported beside them."""
    nL = len(layers)
    out = []
    turn = 0
    for n in n_values:
        N = cfg.tokens(n)
        x = synth.make_hidden(cfg, n, 99, "cuda")
        y = torch.empty((N, cfg.d), dtype=torch.float32, device="cuda")
        for name in ("perslot", "dedup"):
            log(f"[timeline] n={n} {name}: {warmup} warmup + {steps} steps")
            for _ in range(warmup):
                lay = layers[turn % nL]
                turn += 1
                idx, w = eng.route(lay, x)
                getattr(eng, name)(lay, x, idx, w, y)
            torch.cuda.synchronize()
            hold_gpu(0.25 * steps)
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            idxs = []
            for _ in range(steps):
                lay = layers[turn % nL]
                turn += 1
                idx, w = eng.route(lay, x)
                getattr(eng, name)(lay, x, idx, w, y)
                idxs.append(idx)
            e1.record()
            torch.cuda.synchronize()
            U = [unique_count(i.cpu().numpy(), cfg.E) for i in idxs]
            out.append({"n": n, "tokens": N, "engine": name,
                        "us_per_step": round(e0.elapsed_time(e1) * 1e3 / steps, 2),
                        "U_mean": round(float(np.mean(U)), 2)})
    return {"kind": "timeline", "workload": f"{cfg.name}-shaped layer, route + expert pass",
            "steps": steps, "warmup": warmup, "by_case": out}


def host_info():
    """What the CPU baseline ran on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}


def oracle_pass(cfg, n, seconds, threads, rep=0):
    """The CPU oracle (as written, not tuned) on one verify pass of n tokens
    per sequence (route + dedup layer, fp64) with the row-major weights of
    layer 0, repeated for about `seconds` (at least once).  Returns (seconds
    per pass, passes, requested bytes of the pass)."""
    import oracle as O

    layer = synth.make_layer(cfg, "cuda", layer=0)
    s = O.Shape(cfg.d, cfg.E, cfg.k, cfg.f, cfg.S, O.BF16 if cfg.wdtype == "bf16" else O.F32)
    x_np = synth.make_hidden(cfg, n, rep, "cuda").cpu().numpy()
    gate = layer["gate_w"].cpu().numpy()
    r = O.route(s, gate, x_np)
    used = np.unique(r["idx"])
    hdt = np.uint16 if cfg.wdtype == "bf16" else np.float32
    host_w13 = np.zeros((cfg.E,) + tuple(layer["w13"].shape[1:]), hdt)
    host_w2 = np.zeros((cfg.E,) + tuple(layer["w2"].shape[1:]), hdt)
    for e in used:
        host_w13[e] = synth.to_host_bits(layer["w13"][e])
        host_w2[e] = synth.to_host_bits(layer["w2"][e])
    ws13, ws2 = synth.to_host_bits(layer["ws13"]), synth.to_host_bits(layer["ws2"])
    del layer
    torch.cuda.empty_cache()
    passes = 0
    U = 0
    t0 = time.perf_counter()
    while True:
        r = O.route(s, gate, x_np)
        _, rb, sb, U = O.layer(s, host_w13, host_w2, ws13, ws2, x_np, r["idx"], r["w"],
                               engine="dedup", n_threads=threads)
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / passes
    return dt, passes, gate_bytes(cfg) + (U + cfg.S) * expert_bytes(cfg)


def cpu_baseline(cfg, n, seconds):
    """The oracle timed on this host on the bench step's pass: all host
    threads (up to 16) for about `seconds`, and one pass single-threaded."""
    threads = min(16, len(os.sched_getaffinity(0)))
    dt, passes, req = oracle_pass(cfg, n, seconds, threads, rep=99)
    dt1, _, _ = oracle_pass(cfg, n, 0.0, 1, rep=99)
    return {"value": round(req / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "us_per_pass": round(dt * 1e6, 1),
            "single_thread_us_per_pass": round(dt1 * 1e6, 1),
            "host": host_info(),
            "sample": f"{passes} oracle pass(es) of the n={n} {cfg.name} verify pass "
                      f"(route + dedup layer, fp64), {threads} threads, {dt * passes:.1f} s; "
                      f"then one pass on 1 thread"}


def cpu_sweep(seconds):
    """The oracle on every workload at a few pass sizes (all host threads up
    to 16, about `seconds` per point, at least one pass)."""
    threads = min(16, len(os.sched_getaffinity(0)))
    points = {"tiny": (4,), "mixtral": (1, 4, 8), "v2lite": (1, 4, 8, 16), "v3": (1, 16)}
    out = []
    for name, ns in points.items():
        cfg = synth.CONFIGS[name]
        for n in ns:
            dt, passes, req = oracle_pass(cfg, n, seconds, threads)
            out.append({"workload": name, "n": n, "tokens": cfg.tokens(n),
                        "us_per_pass": round(dt * 1e6, 1), "GBs": round(req / dt / 1e9, 3),
                        "passes": passes})
            log(f"  cpu {name} n={n}: {dt * 1e3:.1f} ms per pass")
    return {"kind": "oracle sweep", "threads": threads, "host": host_info(), "points": out}


def traffic_record(kernel, engine, workload):
    """HBM bytes per launch of one kernel of one engine from committed
    rocprofv3 counter runs, if they were taken on the current kernel source;
    else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{engine}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256()
    for f in rec.get("source_files", []):
        sha.update(open(os.path.join(ROOT, f), "rb").read())
    if rec.get("source_sha256") != sha.hexdigest():
        return None
    return rec


def engine_kernels(cfg, eng, layers, x, steps, warmup, engine):
    """The up (W1/W3 + SwiGLU) and down (W2) kernels of one engine, timed
    live: K steps of route + that engine's pass, the library bracketing the
    two kernels' launches with HIP events on the launch stream.  Algorithmic
    bytes per launch: instances streamed (N k + S per-slot, U + S dedup) x
    the bytes of one instance's matrices (2 d f s_w up, d f s_w down)."""
    _, kt, U = timed_steps(cfg, eng, layers, x, steps, warmup, kernel_events=("up", "down"),
                           engines=(engine,))
    N = x.shape[0]
    units = [(N * cfg.k if engine == "perslot" else u) + cfg.S for u in U[engine]]
    out = {}
    for kind, unit in (("up", 2 * cfg.d * cfg.f * cfg.wbytes), ("down", cfg.d * cfg.f * cfg.wbytes)):
        ms, launches = kt[kind]
        launches = max(1, launches)
        algo = sum(units) * unit / launches
        avg_us = ms * 1e3 / launches
        achieved = algo / (avg_us * 1e-6) / 1e9 if avg_us > 0 else None
        tr = traffic_record(f"expert_{kind}", engine, cfg.name)
        out[kind] = {"achieved": None if achieved is None else round(achieved, 1),
                     "frac": None if achieved is None else round(achieved / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(avg_us, 2), "launches": launches,
                     "algorithmic_bytes_per_launch": int(algo), "unit_bytes": unit,
                     "instances_per_launch": round(sum(units) / launches, 2),
                     "traffic": None if tr is None else tr.get("bytes_per_launch"),
                     "traffic_frac_of_algorithmic": None if tr is None else
                     round(tr.get("bytes_per_launch") / algo, 3),
                     # the counters' bytes beyond L2 over the same launch time
                     "traffic_GBs": None if tr is None or not avg_us > 0 else
                     round(tr.get("bytes_per_launch") / (avg_us * 1e-6) / 1e9, 1)}
    return out


def bandwidth_sensitivity(cfg, calib, sweep, z=2.0):
    """How an error in the calibrated bandwidths moves each result: the
    predicted crossovers and the best draft length, recomputed with each
    engine's bandwidth moved by z standard errors in the direction that
    favours it and in the direction that disfavours it.  Model pass time per
    engine: t(n) = route(n) + B(n) / BW + t0 with B_ps = N k B_e and B_dd =
    u(n) N k B_e (shared experts in t0)."""
    Be = expert_bytes(cfg)
    ns = [r["n"] for r in sweep]
    fps, fdd = calib["perslot"], calib["dedup_pooled"]

    def model(bw_ps, bw_dd):
        ps, dd = stepmodel.with_bandwidth(fps, bw_ps), stepmodel.with_bandwidth(fdd, bw_dd)
        t = {"perslot": {}, "dedup": {}}
        saving = []
        for r in sweep:
            b_ps = cfg.tokens(r["n"]) * cfg.k * Be
            tp = ps.predict(b_ps)[0]
            td = dd.predict(r["u_bar"] * b_ps)[0]
            t["perslot"][r["n"]] = tp + r["perslot"]["route_us"]
            t["dedup"][r["n"]] = td + r["dedup"]["route_us"]
            saving.append(tp - td)
        return t, saving

    cases = {"nominal": (fps.bw_GBs, fdd.bw_GBs),
             "dedup_favoured": (fps.bw_GBs - z * fps.bw_sd_GBs, fdd.bw_GBs + z * fdd.bw_sd_GBs),
             "perslot_favoured": (fps.bw_GBs + z * fps.bw_sd_GBs, fdd.bw_GBs - z * fdd.bw_sd_GBs)}
    alphas = [0.3, 0.5, 0.6, 0.7, 0.8, 0.85, 0.9, 0.95, 0.98]
    gmax = max(ns) - 1
    out = {"z": z, "bw_ps_GBs": [round(fps.bw_GBs, 1), round(fps.bw_sd_GBs, 1)],
           "bw_dd_GBs": [round(fdd.bw_GBs, 1), round(fdd.bw_sd_GBs, 1)], "cases": {}}
    stairs = {}
    for name, (bp, bd) in cases.items():
        t, saving = model(bp, bd)
        # r(n) of the per-n calibration, moved by z of its own standard error
        shift = {"nominal": 0.0, "dedup_favoured": z, "perslot_favoured": -z}[name]
        r = [x["r"] + shift * x["r_sd"] for x in sweep]
        td = 0.05 * t["perslot"][1]
        stairs[name] = {e: draftlen.staircase(alphas, t[e], td, gmax) for e in ("perslot", "dedup")}
        out["cases"][name] = {
            "r_pooled": round(bd / bp, 4),
            "crossover_u_lt_r": stepmodel.first_n(ns, [x["u_bar"] < rr for x, rr in zip(sweep, r)]),
            "crossover_model_saving": stepmodel.first_n(ns, [sv > 0 for sv in saving]),
            "best_gamma": stairs[name]}
    out["alphas"] = alphas
    out["t_draft_over_t1"] = 0.05
    out["best_gamma_max_shift"] = {
        e: max(abs(a - b) for name in cases for a, b in zip(stairs[name][e], stairs["nominal"][e]))
        for e in ("perslot", "dedup")}
    return out


def compact_sweep(sweep):
    """Per-n record of the sweep for the headline: us and requested GB/s per
    engine, mean U and r(n)."""
    return [{"n": r["n"], "ps_us": r["perslot"]["us"], "ps_GBs": round(r["perslot"]["GBs"]),
             "dd_us": r["dedup"]["us"], "dd_GBs": round(r["dedup"]["GBs"]), "U": r["U_mean"],
             "r": r["r"]} for r in sweep]


def write_details(path, doc):
    """The full record of a run (sweep, calibration, draft lengths,
    verification round, kernels, CPU baseline) as one JSON file, when a
    path is given."""
    if not path:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(doc, f, indent=1)
        log(f"[bench] details written to {path}")
    except OSError as e:
        log(f"[bench] could not write {path}: {e}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="v2lite", choices=sorted(synth.CONFIGS))
    ap.add_argument("--n", type=int, default=None, help="pass size of the timed step")
    ap.add_argument("--layers", type=int, default=None, help="weight sets in the rotation")
    ap.add_argument("--reps", type=int, default=50,
                    help="passes per n and engine in the sweep (at least %d for passes "
                         "under %g us)" % (SHORT_PASS_REPS, SHORT_PASS_US))
    ap.add_argument("--calib-reps", type=int, default=16,
                    help="passes per (n, U) point of the dedup calibration")
    ap.add_argument("--verify-only", action="store_true",
                    help="only time the verification round (moe_verify_gate) and print "
                         "its JSON")
    ap.add_argument("--rho-sweep", action="store_true",
                    help="instead of the bench line: the routing-overlap sweep over the "
                         "26-layer V2-Lite stack (one JSON document)")
    ap.add_argument("--variants", action="store_true",
                    help="instead of the bench line: per-slot vs union dedup vs "
                         "per-sequence dedup, and plain vs biased routing, over the "
                         "config's pass sizes (one JSON document)")
    ap.add_argument("--variant-reps", type=int, default=12,
                    help="passes per n and engine in the variants leg")
    ap.add_argument("--stack-reps", type=int, default=32,
                    help="stack passes per (rho, n) in the rho sweep")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sweep", action="store_true",
                    help="only time the CPU oracle on every workload at a few pass sizes "
                         "(one JSON document)")
    ap.add_argument("--engine", default="both", choices=("both", "perslot", "dedup"),
                    help="engines of the timed steps (one engine isolates its kernels for "
                         "a profiler run)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused-stack leg after the timed steps")
    ap.add_argument("--resume", default=None,
                    help="sweep log (JSON lines): points of the n sweep and of the rho sweep "
                         "found there are not measured again, measured ones are appended")
    ap.add_argument("--details", default=None,
                    help="file for the full record of the run (the last stdout line is "
                         "the compact headline); none is written without it")
    ap.add_argument("--timeline", default=None,
                    help="comma-separated pass sizes: instead of the bench line, K steps of "
                         "route + pass per engine at each size, queued while the GPU is held, "
                         "for a kernel-trace timeline (one JSON document)")
    ap.add_argument("--shard", type=int, default=None,
                    help="instead of the bench line: the n sweep on one GPU's share of the "
                         "config's layer with every expert split along d_ff over SHARD GPUs "
                         "(gate and tokens whole), with the summing all-reduce's per-link "
                         "bandwidth bound beside it (one JSON document)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (for scaling HBM "
                         "byte counters) and print its byte counts")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer is not sharded across GPUs; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "launches": 5,
                          "read_bytes_per_launch": nbytes, "write_bytes_per_launch": nbytes}))
        return

    if args.cpu_sweep:
        print(json.dumps(cpu_sweep(min(args.cpu_seconds, 3.0))), flush=True)
        return

    if args.verify_only:
        print(json.dumps({"verify_gate": verify_gate_leg()}), flush=True)
        return

    cfg = synth.CONFIGS["v2stack" if args.rho_sweep else args.config]
    whole = cfg
    if args.shard:
        cfg = synth.share_config(cfg, args.shard)
    n_head = args.n or max(cfg.n_values)
    layer_bytes = (cfg.E + cfg.S) * expert_bytes(cfg)
    n_layers = args.layers or (cfg.layers if args.rho_sweep else
                               max(2, min(8, int(8e9 // layer_bytes))))
    log(f"[bench] {cfg.name}: {n_layers} weight sets of {layer_bytes / 1e9:.2f} GB, "
        f"timed step n={n_head}")
    shape = B.shape_of(cfg)
    stack, layers = make_stack(cfg, shape, n_layers)
    eng = Engines(cfg)

    if args.timeline:
        print(json.dumps(timeline_leg(cfg, eng, layers, [int(v) for v in args.timeline.split(",")],
                                      args.steps, args.warmup)), flush=True)
        return

    if args.variants:
        log("[bench] variants warmup")
        variants_leg(cfg, eng, layers, cfg.n_values[:1], 2)
        log("[bench] variants")
        doc = {"kind": "layer variants",
               "workload": f"{cfg.name}-shaped layer, {cfg.n_seq} sequence(s) x n = "
                           f"{min(cfg.n_values)}..{max(cfg.n_values)} tokens per pass, "
                           f"{n_layers} weight sets rotated",
               "by_n": variants_leg(cfg, eng, layers, cfg.n_values, args.variant_reps)}
        print(json.dumps(doc), flush=True)
        return

    if args.shard:
        xs = {}
        log("[bench] share sweep warmup")
        run_sweep(cfg, eng, layers, xs, cfg.n_values[:2], 5, top_up=False)
        log(f"[bench] share sweep: d_ff {whole.f} / {args.shard} = {cfg.f}")
        points = SweepLog(args.resume) if args.resume else None
        sweep = run_sweep(cfg, eng, layers, xs, cfg.n_values, args.reps, points=points)
        doc = shard_doc(whole, cfg, args.shard, sweep, n_layers)
        write_details(args.details, doc)
        print(json.dumps(doc), flush=True)
        return

    sweep = calib = None
    if not args.no_sweep or args.rho_sweep:
        xs = {(n, rep): synth.make_hidden(cfg, n, rep, "cuda")
              for n in cfg.n_values for rep in range(args.reps)}
        log("[bench] sweep warmup")
        run_sweep(cfg, eng, layers, xs, cfg.n_values[:2], 5, top_up=False)  # 10 passes per engine
        log("[bench] sweep")
        points = SweepLog(args.resume) if args.resume else None
        sweep = run_sweep(cfg, eng, layers, xs, cfg.n_values, args.reps, points=points)
        log("[bench] dedup calibration on crafted routings")
        calib = calibrate(cfg, eng, layers, xs, args.reps, sweep, args.calib_reps)
        for r in sweep:
            # the measured saving is a difference of median pass times, and
            # both engines' times grow with U, so the prediction it is held
            # against takes the passes' median U (a step when experts are few
            # and large); u_bar stays the mean, as its definition requires
            u_med = r["U_median"] / (cfg.tokens(r["n"]) * cfg.k)
            rr, rr_sd, sav, sav_sd, iv_sd, trace = predict_from_calibration(cfg, calib, r["n"], u_med)
            r["r_trace"] = r.pop("r")
            r["r"], r["r_sd"] = round(rr, 4), round(rr_sd, 4)
            r["saving_us"] = round(r["perslot"]["us"] - r["dedup"]["us"], 2)
            saving_check(r, r["saving_us"], sav, sav_sd, iv_sd, trace)
        del xs

    if args.rho_sweep:
        log(f"[bench] rho sweep over {n_layers} layers")
        doc = {"kind": "routing-overlap sweep",
               "workload": f"{cfg.name}: V2-Lite-shaped layer stacked {n_layers} deep "
                           f"({n_layers * layer_bytes / 1e9:.1f} GB of weights), "
                           f"n = 1..{max(cfg.n_values)}",
               "single_layer_sweep": sweep, "calibration": calibration_json(calib),
               "bandwidth_sensitivity": bandwidth_sensitivity(cfg, calib, sweep),
               "by_rho": rho_sweep(cfg, eng, layers, stack, calib, args.stack_reps,
                                   points=points)}
        write_details(args.details, doc)
        print(json.dumps(rho_summary(doc)), flush=True)
        return

    engines = ("perslot", "dedup") if args.engine == "both" else (args.engine,)
    x = synth.make_hidden(cfg, n_head, 99, "cuda")
    log(f"[bench] timed steps ({'+'.join(engines)}): {args.warmup} warmup + {args.steps}")
    wall, _, U_list = timed_steps(cfg, eng, layers, x, args.steps, args.warmup, engines=engines)
    N = cfg.tokens(n_head)
    Be = expert_bytes(cfg)
    step_bytes = 0.0
    if "perslot" in engines:
        step_bytes += gate_bytes(cfg) + (N * cfg.k + cfg.S) * Be
    if "dedup" in engines:
        step_bytes += float(np.mean([gate_bytes(cfg) + (u + cfg.S) * Be for u in U_list["dedup"]]))
    ms_step = wall / args.steps * 1e3
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # Dominant kernels, per engine: W1/W3 + SwiGLU (up) and W2 (down), each
    # engine timed live in a timed region of its own in which the library
    # brackets only those kernels with HIP events on the launch stream.
    kern = {}
    for name in engines:
        log(f"[bench] {name} steps with up/down kernel events")
        kern[name] = engine_kernels(cfg, eng, layers, x, args.steps, args.warmup, name)
    main_eng = "dedup" if "dedup" in engines else engines[0]
    up = kern[main_eng]["up"]
    roofline = {"bound": "hbm", "kernel": f"expert_up (W1/W3 + SwiGLU), {main_eng} engine",
                "achieved": up["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": up["frac"], "traffic": up["traffic"],
                "avg_launch_us": up["avg_launch_us"],
                "algorithmic_bytes_per_launch": up["algorithmic_bytes_per_launch"],
                "per_engine": {e: {k: {kk: v[kk] for kk in ("achieved", "frac", "avg_launch_us",
                                                              "traffic", "traffic_GBs")}
                                   for k, v in kern[e].items()} for e in engines}}

    fused = None
    if not args.no_fused:
        # The same rotation as one fused stack call per engine (all layers on
        # the step's tokens): per-layer time including routing.
        log("[bench] fused stack over the rotation")
        fz = fused_stack_leg(cfg, stack, [n_head], 16)[n_head]
        fused = {"layers": n_layers, "tokens": N,
                 "perslot_stack_us": round(fz["perslot"], 1),
                 "dedup_stack_us": round(fz["dedup"], 1),
                 "perslot_us_per_layer": round(fz["perslot"] / n_layers, 2),
                 "dedup_us_per_layer": round(fz["dedup"] / n_layers, 2),
                 "U_mean": round(float(fz["U"].mean()), 2)}

    config = {"workload": f"{cfg.name}-shaped MoE layer, one verify pass of n={n_head}"
                          f" tokens{' x %d sequences' % cfg.n_seq if cfg.n_seq > 1 else ''}"
                          f", {' and '.join(engines)} engine{'s' if len(engines) > 1 else ''}",
              "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k, "d_ff": cfg.f,
              "shared_experts": cfg.S, "weights": cfg.wdtype, "rho": cfg.rho,
              "tokens": N, "weight_sets_rotated": n_layers}
    head = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.wdtype == "bf16" else "f32",
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
    }
    details = {"headline": head, "kernels": kern, "fused_stack": fused,
               "step_bytes": int(step_bytes)}
    if sweep is not None:
        ns = [r["n"] for r in sweep]
        cross = {"measured": stepmodel.first_n(ns, [r["dedup_faster"] for r in sweep]),
                 "predicted_u_lt_r": stepmodel.first_n(ns, [r["u_bar"] < r["r"] for r in sweep]),
                 "predicted_model_saving_gt_0": stepmodel.first_n(
                     ns, [r["predicted_saving_us"] > 0 for r in sweep])}
        sens = bandwidth_sensitivity(cfg, calib, sweep)
        checks = {"within_param_2sd": f"{sum(r['saving_within_param_2sd'] for r in sweep)} of {len(sweep)}",
                  "within_interval_2sd": f"{sum(r['saving_within_2sd'] for r in sweep)} of {len(sweep)}",
                  "trace_model_within_interval_2sd":
                      f"{sum(r['trace_saving_within_2sd'] for r in sweep)} of {len(sweep)}"}
        head["crossover"] = cross
        head["bw_error_moves"] = {
            "crossover_u_lt_r": [sens["cases"][c]["crossover_u_lt_r"]
                                 for c in ("perslot_favoured", "nominal", "dedup_favoured")],
            "crossover_model": [sens["cases"][c]["crossover_model_saving"]
                                for c in ("perslot_favoured", "nominal", "dedup_favoured")],
            "best_gamma_max_shift": sens["best_gamma_max_shift"]}
        head["saving_check"] = checks
        head["sweep"] = compact_sweep(sweep)
        details.update({"sweep": sweep, "calibration": calibration_json(calib),
                        "draft_length": draft_length_table(sweep), "crossover": cross,
                        "saving_check": checks, "bandwidth_sensitivity": sens})
    if not args.no_sweep:
        log("[bench] verification round")
        details["verify_gate"] = verify_gate_leg()
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (~{args.cpu_seconds:.0f} s)")
        del layers, stack
        torch.cuda.empty_cache()
        cb = cpu_baseline(cfg, n_head, args.cpu_seconds)
        details["cpu_baseline"] = cb
        head["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample",
                                                   "us_per_pass")}
    head["details"] = os.path.relpath(args.details, ROOT) if args.details else None
    write_details(args.details, details)
    line = json.dumps(head)
    if len(line) > 4000 and "sweep" in head:
        # keep the headline short enough for a log tail: drop r(n) per entry
        for r in head["sweep"]:
            r.pop("r", None)
        line = json.dumps(head)
    print(line, flush=True)


def rho_summary(doc):
    """Compact record of the routing-overlap sweep: per rho, crossovers,
    saving-check counts and per n the byte share, per-layer pass times, the
    measured and predicted saving and the fused stack's per-layer times."""
    out = {"kind": doc["kind"], "workload": doc["workload"],
           "calibration": {k: doc["calibration"][k] for k in ("perslot", "dedup_pooled",
                                                               "perslot_trace", "r_pooled")},
           "bandwidth_sensitivity": {k: doc["bandwidth_sensitivity"][k]
                                     for k in ("z", "bw_ps_GBs", "bw_dd_GBs", "best_gamma_max_shift")},
           "by_rho": []}
    for rr in doc["by_rho"]:
        recs = rr["by_n"]
        out["by_rho"].append({
            "rho": rr["rho"], "crossover": rr["crossover"],
            "saving_within_param_2sd": f"{sum(r['saving_within_param_2sd'] for r in recs)} of {len(recs)}",
            "saving_within_2sd": rr["saving_within_2sd"],
            "trace_saving_within_2sd": rr["trace_saving_within_2sd"],
            "by_n": [{"n": r["n"], "u": r["u_bar"], "U": r["U_mean"], "r": r["r"],
                      "ps_layer_us": r["perslot_layer_us"], "dd_layer_us": r["dedup_layer_us"],
                      "saving_us": r["saving_us"], "pred_us": r["predicted_saving_us"],
                      "pred_sd_us": r["predicted_saving_sd_us"],
                      "interval_sd_us": r["saving_interval_sd_us"],
                      "trace_pred_us": r["trace_predicted_saving_us"],
                      "fused_ps_layer_us": r["fused"]["perslot_layer_us"],
                      "fused_dd_layer_us": r["fused"]["dedup_layer_us"]} for r in recs]})
    return out


if __name__ == "__main__":
    main()
