"""Benchmark of the BitLinear W1.58A8 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

Workload (the headline): decode at batch 1 through one layer of the
100B-class model -- q, o 8192x8192; k, v 1024x8192; up 28672x8192 with
ReLU^2; down 8192x28672 -- with seeded synthetic data: ternary weights
from N(0, 0.02^2) fp32, bf16 Student-t (nu = 3) activations, bf16 outputs.

One step = the whole per-call hot path of that layer, in layer order: one
fused decode launch (bitlinear_forward_fused: per-token absmax int8
quantization of the input in the kernel prologue, the ternary x int8 GEMV,
the gamma/s dequant, ReLU^2 on up) per group of products sharing an input --
q/k/v, then o, up, down.  Weights are packed before timing (as at model
load) into 4 layer copies (620 MB, past 2 x (256 MB Infinity Cache + 32 MB
L2)); consecutive steps use consecutive copies, so every step streams its
weights from HBM.  Steps are replayed from HIP graphs, timed with events on
the stream the kernels run on.

value = algorithmic bytes of a step / step time (GB/s): for each product
N*K/4 (packed W) + 4 (gamma) + 2*M*N (bf16 y), plus each distinct bf16
input once, 2*M*K (x~ never leaves the chip).

Also on the same line:
  roofline      the step's dominant launches, the fused up and down GEMVs,
                each timed alone over >= ceil(2 x 288 MiB / its bytes)
                rotating weight copies: (bytes_up + bytes_down) / (t_up +
                t_down), t = median over 25 graph replays; traffic from the
                committed FETCH_SIZE / WRITE_SIZE summary of the same
                launches (null if the kernel sources changed since);
  gemv_plain    the same two products through bitlinear_forward (x~ given);
  c5            the layer at 1, 16 and 512 tokens: each product alone
                (GB/s, TOPS), the layer with one quant per input + one
                forward per product (q/k/v also in one forward_multi call),
                and at 16 tokens the fused steps;
  prefill       the 2048-token prefill GEMMs (2048x2560 -> 6912 with ReLU^2,
                2048x6912 -> 2560): 2*M*N*K / kernel time, TOPS;
  c2            batch-1 decode at 2B-class shapes: the six products in one
                fused launch, and each product's plain GEMV;
  stack_c3      the 2B-class set as a 30-layer stack (388 MB packed, two
                stack copies alternating), one fused launch per input group,
                us per pass at 1/8/32/64 tokens;
  cpu_baseline  the CPU oracle on the same decode step, on one core and on
                every core the process may use.
Per-launch times are median and minimum over >= 20 replays.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0          # dense int8 MFMA, 5.0 POPS
CACHE_BYTES = (256 + 32) << 20   # Infinity Cache + 8 x 4 MB L2
SIMDS = 256 * 4                  # 256 CUs x 4 SIMDs
XCDS = 8
CLOCK_GHZ = 2.4                  # MI355X peak engine clock
REPS = 25                        # timed graph replays per measurement
GRAPH_STEPS = 8                  # decode steps per captured graph
LAYER_GROUPS = (("q", "k", "v"), ("o",), ("up",), ("down",))


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def copies_for(nbytes: float) -> int:
    """Distinct copies a timed loop must cycle through so that the bytes
    between two uses of one copy exceed twice the on-chip caches."""
    return max(2, math.ceil(2 * CACHE_BYTES / nbytes))


# --------------------------------------------------------------- helpers --
def gemv_bytes(m, n, k):
    """A plain forward: packed W, x~, s, gamma, bf16 y."""
    return n * k / 4 + m * k + 4 * m + 4 + 2 * m * n


def fused_bytes(m, n, k):
    """A fused product without its input: packed W, gamma, bf16 y."""
    return n * k / 4 + 4 + 2 * m * n


def quant_bytes(m, k):
    return 2 * m * k + m * k + 4 * m


def stats(ts):
    return {"median": round(statistics.median(ts), 3), "min": round(min(ts), 3), "reps": len(ts)}


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # once outside capture, on the same stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def replay_times(torch, g, per_graph, reps=REPS, warm=2):
    """Per-unit GPU time (us) of each of `reps` replays of graph g, which
    holds `per_graph` units; events on the stream the replays run on."""
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        g.replay()
        en.record()
        torch.cuda.synchronize()
        out.append(st.elapsed_time(en) * 1e3 / per_graph)
    return out


def time_launches(torch, launch, count, per_graph=None, reps=REPS):
    """Per-launch us (median, min over reps) of launch(i), i cycling through
    `count` variants (weight copies), `per_graph` launches per graph."""
    per_graph = per_graph or max(count, 16)
    g = capture(torch, lambda: [launch(i % count) for i in range(per_graph)])
    ts = replay_times(torch, g, per_graph, reps)
    del g
    return stats(ts)


# ------------------------------------------------------------ the weights --
class Weights:
    """Packed weights of a workload's matrices; matrix `name` has
    copies[name] device copies (copy 0 is the packed original)."""

    def __init__(self, B, torch, wl, names=None, copies=None, min_copies=1, codes=False):
        import datagen
        self.wl = wl
        self.names = list(names or wl.matrices.keys())
        self.mats, self.codes = {}, {}
        for name in self.names:
            n, k, relu2, group = wl.matrices[name]
            w = datagen.workload_weights(wl, name)
            wd = torch.from_numpy(w).cuda()
            packed, gamma = B.pack_weights(wd)
            del wd
            if codes:                                   # for the CPU baseline
                import oracle as O
                g = O.absmean_gamma(w)
                self.codes[name] = (O.ternary_codes(w, g), g)
            del w
            c = copies if copies is not None else copies_for(B.packed_bytes(n, k))
            c = max(c, min_copies)
            self.mats[name] = dict(n=n, k=k, relu2=relu2, group=group, gamma=gamma,
                                   packed=[packed] + [packed.clone() for _ in range(c - 1)])
        torch.cuda.synchronize()

    def copies(self, name):
        return len(self.mats[name]["packed"])


class Inputs:
    """bf16 activations of every input group at m tokens, their x~ and s, and
    bf16 outputs of every product."""

    def __init__(self, B, torch, W, m):
        import datagen
        self.m = m
        self.x, self.xq, self.s = {}, {}, {}
        for g in W.wl.groups():
            bits, _ = datagen.activations(W.wl, g, m)
            x = torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
            self.x[g] = x
            self.xq[g], self.s[g] = B.quant_act(x)
        self.y = {nm: torch.empty((m, d["n"]), dtype=torch.bfloat16, device="cuda")
                  for nm, d in W.mats.items()}


def fused_call(B, W, X, names, copy, ws):
    ops = []
    for nm in names:
        d = W.mats[nm]
        ops.append(dict(x=X.x[d["group"]], packed=d["packed"][copy % len(d["packed"])],
                        gamma=d["gamma"], n=d["n"], k=d["k"], y=X.y[nm], relu2=d["relu2"]))
    return B.FusedStep(ops, workspace=ws)


def forward_call(B, W, X, name, copy, ws):
    d = W.mats[name]
    g = d["group"]
    return lambda: B.forward(X.xq[g], X.s[g], d["packed"][copy % len(d["packed"])], d["gamma"],
                             d["n"], d["k"], relu2=d["relu2"], y=X.y[name], workspace=ws)


def step_bytes_fused(W, m, names=None):
    names = names or W.names
    b = sum(fused_bytes(m, W.mats[n]["n"], W.mats[n]["k"]) for n in names)
    groups = {W.mats[n]["group"]: W.mats[n]["k"] for n in names}
    return b + sum(2 * m * k for k in groups.values())


# ------------------------------------------------------- headline: c5 m=1 --
def run_headline(B, torch, W, args):
    """The c5 decode step at one token: one fused launch per input group."""
    X = Inputs(B, torch, W, 1)
    ws = B.Workspace()
    layers = copies_for(sum(B.packed_bytes(d["n"], d["k"]) for d in W.mats.values()))
    steps = [[fused_call(B, W, X, grp, l, ws) for grp in LAYER_GROUPS] for l in range(layers)]
    for st in steps:
        for c in st:
            ws.get(c.nbytes)

    def run_step(l):
        for c in steps[l % layers]:
            c()

    # the fused step against quant_act + forward per product, bit for bit
    run_step(0)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in X.y.items()}
    for nm in W.names:
        forward_call(B, W, X, nm, 0, ws)()
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k].view(torch.int16), X.y[k].view(torch.int16)), k

    # one graph of GRAPH_STEPS consecutive steps (layer copies in rotation,
    # GRAPH_STEPS a multiple of the copy count), one-step graphs per copy for
    # a remainder
    assert GRAPH_STEPS % layers == 0
    big = capture(torch, lambda: [run_step(i) for i in range(GRAPH_STEPS)])
    singles = [capture(torch, lambda l=l: run_step(l)) for l in range(layers)]
    big.replay()
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k].view(torch.int16), X.y[k].view(torch.int16)), k
    for i in range(max(1, args.warmup // GRAPH_STEPS)):
        big.replay()
    torch.cuda.synchronize()
    nbig, rest = divmod(args.steps, GRAPH_STEPS)
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for i in range(nbig):
        big.replay()
    for i in range(rest):
        singles[i % layers].replay()
    en.record()
    torch.cuda.synchronize()
    ms = st.elapsed_time(en) / args.steps
    per_rep = replay_times(torch, big, GRAPH_STEPS)
    sbytes = step_bytes_fused(W, 1)
    del big, singles

    # the dominant launches alone: fused up and down, and their plain GEMVs
    legs = {}
    for nm in ("up", "down"):
        d = W.mats[nm]
        cps = W.copies(nm)
        calls = [fused_call(B, W, X, (nm,), c, ws) for c in range(cps)]
        t = time_launches(torch, lambda c: calls[c](), cps, 2 * cps)
        tp = time_launches(torch, lambda c: forward_call(B, W, X, nm, c, ws)(), cps, 2 * cps)
        legs[nm] = {"copies": cps, "fused_us": t, "plain_us": tp,
                    "fused_bytes": int(fused_bytes(1, d["n"], d["k"]) + 2 * d["k"]),
                    "plain_bytes": int(gemv_bytes(1, d["n"], d["k"]))}
        del calls
    b_f = legs["up"]["fused_bytes"] + legs["down"]["fused_bytes"]
    t_f = legs["up"]["fused_us"]["median"] + legs["down"]["fused_us"]["median"]
    b_p = legs["up"]["plain_bytes"] + legs["down"]["plain_bytes"]
    t_p = legs["up"]["plain_us"]["median"] + legs["down"]["plain_us"]["median"]
    achieved = b_f / (t_f * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
            "kernel": "gemv_stream_fused_kernel at one token on the 100B-class up (28672x8192, "
                      "ReLU^2) and down (8192x28672) products: activation quant + GEMV + dequant",
            "bytes_per_launch_pair": b_f, "us_per_launch_pair": round(t_f, 3), "legs": legs}
    plain = {"kernel": "gemv_stream_kernel (bitlinear_forward, x~ given) on the same two products",
             "achieved": round(b_p / (t_p * 1e-6) / 1e9, 1), "unit": "GB/s",
             "frac": round(b_p / (t_p * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "bytes_per_launch_pair": b_p, "us_per_launch_pair": round(t_p, 3)}
    value = sbytes / (ms * 1e-3) / 1e9
    return value, ms, sbytes, layers, stats(per_rep), roof, plain


# ------------------------------------------------------------- c5 extras --
def run_c5(B, torch, W):
    out = {}
    layers = copies_for(sum(B.packed_bytes(d["n"], d["k"]) for d in W.mats.values()))
    for m in (1, 16, 512):
        X = Inputs(B, torch, W, m)
        ws = B.Workspace()
        for d in W.mats.values():
            ws.get(B.forward_workspace_bytes(m, d["n"], d["k"]))
        per = {}
        for nm in W.names:
            d = W.mats[nm]
            cps = W.copies(nm)
            t = time_launches(torch, lambda c, nm=nm: forward_call(B, W, X, nm, c, ws)(), cps,
                              max(2 * cps, 16) if cps < 64 else cps)
            us = t["median"]
            per[nm] = {"shape": f"{m}x{d['k']}->{d['n']}", "copies": cps, "us": t,
                       "GBs": round(gemv_bytes(m, d["n"], d["k"]) / (us * 1e-6) / 1e9, 1),
                       "TOPS": round(2.0 * m * d["n"] * d["k"] / (us * 1e-6) / 1e12, 2)}

        def layer(l):
            for g in X.x:
                x = X.x[g]
                B._check("quant", B.lib.bitlinear_quant_act(
                    x.data_ptr(), B.BL_BF16, m, x.shape[1], B.EPS_DEFAULT, X.xq[g].data_ptr(),
                    X.s[g].data_ptr(), B._stream()))
            for nm in W.names:
                forward_call(B, W, X, nm, l, ws)()

        def layer_multi(l):
            for g in X.x:
                x = X.x[g]
                B._check("quant", B.lib.bitlinear_quant_act(
                    x.data_ptr(), B.BL_BF16, m, x.shape[1], B.EPS_DEFAULT, X.xq[g].data_ptr(),
                    X.s[g].data_ptr(), B._stream()))
            ops = [dict(packed=W.mats[nm]["packed"][l], gamma=W.mats[nm]["gamma"],
                        n=W.mats[nm]["n"], y=X.y[nm]) for nm in ("q", "k", "v")]
            B.forward_multi(X.xq["attn_in"], X.s["attn_in"], 8192, ops, workspace=ws)
            for nm in ("o", "up", "down"):
                forward_call(B, W, X, nm, l, ws)()

        ops = 2.0 * m * sum(d["n"] * d["k"] for d in W.mats.values())
        lb = sum(gemv_bytes(m, d["n"], d["k"]) for d in W.mats.values()) + \
            sum(quant_bytes(m, x.shape[1]) for x in X.x.values())
        tl = time_launches(torch, layer, layers, 2 * layers)
        tm = time_launches(torch, layer_multi, layers, 2 * layers)
        res = {"layer_us": tl, "layer_GBs": round(lb / (tl["median"] * 1e-6) / 1e9, 1),
               "layer_TOPS": round(ops / (tl["median"] * 1e-6) / 1e12, 2),
               "layer_qkv_multi_us": tm,
               "layer_qkv_multi_TOPS": round(ops / (tm["median"] * 1e-6) / 1e12, 2),
               "per_matrix": per}
        if m == 16:
            steps = [[fused_call(B, W, X, grp, l, ws) for grp in LAYER_GROUPS] for l in range(layers)]
            tf = time_launches(torch, lambda l: [c() for c in steps[l]], layers, 2 * layers)
            res["layer_fused_us"] = tf
            res["layer_fused_GBs"] = round(step_bytes_fused(W, m) / (tf["median"] * 1e-6) / 1e9, 1)
            del steps
        out[str(m)] = res
        log(f"c5 m={m}: layer {tl['median']:.1f} us")
        del X
        torch.cuda.empty_cache()
    return {"workload": "one 100B-class layer (q,o 8192x8192; k,v 1024x8192; up 28672x8192 "
                        "+ReLU^2; down 8192x28672); each product timed over its own rotating "
                        f"copies, the layer over {layers} layer copies",
            "per_batch": out}


def run_prefill(B, torch):
    import datagen
    wl = datagen.WORKLOADS["c4"]
    out = {}
    tot_ops, tot_us = 0.0, 0.0
    m = 2048
    W = Weights(B, torch, wl, copies=1)
    X = Inputs(B, torch, W, m)
    for name in ("up", "down"):
        d = W.mats[name]
        n, k = d["n"], d["k"]
        t = time_launches(torch, lambda c: forward_call(B, W, X, name, 0, None)(), 1, 20)
        x = X.x[d["group"]]
        tq = time_launches(torch, lambda c: B.quant_act(x), 1, 20)
        ops = 2.0 * m * n * k
        tops = ops / (t["median"] * 1e-6) / 1e12
        out[name] = {"shape": f"{m}x{k}->{n}", "us": t, "TOPS": round(tops, 1),
                     "frac": round(tops / INT8_PEAK_TOPS, 4), "act_quant_us": tq}
        tot_ops += ops
        tot_us += t["median"]
    tops = tot_ops / (tot_us * 1e-6) / 1e12
    del W, X
    torch.cuda.empty_cache()
    return {"workload": "2048-token prefill: 2048x2560 -> 6912 (+ReLU^2), 2048x6912 -> 2560",
            "TOPS": round(tops, 1), "unit": "TOPS", "peak": INT8_PEAK_TOPS,
            "frac": round(tops / INT8_PEAK_TOPS, 4), "per_matrix": out}


def run_c2(B, torch):
    import datagen
    wl = datagen.WORKLOADS["c2"]
    W = Weights(B, torch, wl)
    X = Inputs(B, torch, W, 1)
    ws = B.Workspace()
    set_copies = copies_for(sum(B.packed_bytes(d["n"], d["k"]) for d in W.mats.values()))
    steps = [fused_call(B, W, X, W.names, c, ws) for c in range(set_copies)]
    for s in steps:
        ws.get(s.nbytes)
    t = time_launches(torch, lambda c: steps[c](), set_copies, set_copies)
    sb = step_bytes_fused(W, 1)
    per = {}
    for nm in W.names:
        d = W.mats[nm]
        cps = W.copies(nm)
        tp = time_launches(torch, lambda c, nm=nm: forward_call(B, W, X, nm, c, ws)(), cps,
                           cps if cps >= 64 else 2 * cps)
        per[nm] = {"copies": cps, "us": tp,
                   "GBs": round(gemv_bytes(1, d["n"], d["k"]) / (tp["median"] * 1e-6) / 1e9, 1)}
    del steps, W, X
    torch.cuda.empty_cache()
    return {"workload": "batch-1 decode at 2B-class shapes (q,o 2560x2560; k,v 640x2560; up "
                        "6912x2560 +ReLU^2; down 2560x6912), bf16 N(0,1) inputs with 1% outlier "
                        "channels x100",
            "fused_step_us": t, "fused_step_bytes": int(sb),
            "fused_step_GBs": round(sb / (t["median"] * 1e-6) / 1e9, 1),
            "fused_step_frac": round(sb / (t["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "set_copies": set_copies, "plain_gemv": per}


def run_stack_c3(B, torch):
    """The c3 stack: the 2B-class set as 30 layers, each with its own copy of
    the packed weights, and a second copy of the whole stack (776 MB in all),
    the two passes alternating.  One pass = every layer in order: q/k/v (one
    shared input), o, up (ReLU^2), down, at 1, 8, 32 and 64 tokens, each
    group one fused decode launch (activation quant in the prologue)."""
    import datagen
    wl = datagen.WORKLOADS["c3"]
    W = Weights(B, torch, wl, copies=2 * wl.layers)
    out = {}
    for m in wl.batches:
        X = Inputs(B, torch, W, m)
        ws = B.Workspace()
        ws.get(max(B.forward_workspace_bytes(m, d["n"], d["k"]) for d in W.mats.values()))
        calls = [[], []]
        for half in (0, 1):
            for l in range(wl.layers):
                cp = half * wl.layers + l
                for grp in LAYER_GROUPS:
                    fc = fused_call(B, W, X, grp, cp, ws)
                    ws.get(fc.nbytes)
                    calls[half].append(fc)
        g = capture(torch, lambda: [c() for h in (0, 1) for c in calls[h]])
        ts = replay_times(torch, g, 2, reps=REPS)
        t = stats(ts)
        by = wl.layers * (sum(fused_bytes(m, d["n"], d["k"]) for d in W.mats.values()) +
                          sum(2 * m * x.shape[1] for x in X.x.values()))
        ops = 2.0 * m * wl.layers * sum(d["n"] * d["k"] for d in W.mats.values())
        out[str(m)] = {"us_per_pass": t, "launches_per_pass": len(calls[0]),
                       "GBs": round(by / (t["median"] * 1e-6) / 1e9, 1),
                       "TOPS": round(ops / (t["median"] * 1e-6) / 1e12, 2)}
        log(f"c3 stack m={m}: {t['median']:.1f} us/pass")
        del g, calls, X, ws
        torch.cuda.empty_cache()
    del W
    torch.cuda.empty_cache()
    return {"workload": "30 layers x {q,k,v,o,up,down} at 2B-class shapes, one pass in layer "
                        "order, packed weights 388 MB per stack, two stacks alternating",
            "per_batch": out}


def run_rmsnorm(B, torch):
    """RMSNorm ahead of the activation quantization: each 2B-class input group
    as one fused decode launch without and with RMSNorm (a gain), at 1, 8 and
    64 tokens over the stack's 60 layer copies; and bitlinear_rmsnorm_quant_act
    against bitlinear_quant_act at decode and prefill sizes."""
    import datagen
    wl = datagen.WORKLOADS["c3"]
    W = Weights(B, torch, wl, copies=2 * wl.layers)
    gains = {g: torch.linspace(0.5, 1.5, wl.input_k(g), device="cuda") for g in wl.groups()}
    fused = {}
    for m in (1, 8, 64):
        X = Inputs(B, torch, W, m)
        ws = B.Workspace()
        for grp in LAYER_GROUPS:
            row = {}
            for norm in (False, True):
                def call(c, grp=grp, norm=norm):
                    ops = []
                    for nm in grp:
                        d = W.mats[nm]
                        o = dict(x=X.x[d["group"]], packed=d["packed"][c % len(d["packed"])],
                                 gamma=d["gamma"], n=d["n"], k=d["k"], y=X.y[nm], relu2=d["relu2"])
                        if norm:
                            o.update(rmsnorm=True, norm_weight=gains[d["group"]])
                        ops.append(o)
                    return B.FusedStep(ops, workspace=ws)()
                row["rmsnorm" if norm else "plain"] = time_launches(torch, call, 2 * wl.layers,
                                                                   2 * wl.layers)["median"]
            fused[f"{'+'.join(grp)} m={m}"] = row
        del X, ws
    del W
    torch.cuda.empty_cache()
    quant = {}
    for m, k in ((1, 2560), (16, 8192), (16, 28672), (2048, 2560), (2048, 6912)):
        xs = [torch.randn(m, k, device="cuda").to(torch.bfloat16) for _ in range(8)]
        g = torch.linspace(0.5, 1.5, k, device="cuda")
        xq = torch.empty((m, B.padded_k(k)), dtype=torch.int8, device="cuda")
        sc = torch.empty(m, dtype=torch.float32, device="cuda")
        q = lambda c: B._check("bitlinear_quant_act", B.lib.bitlinear_quant_act(
            xs[c].data_ptr(), B.BL_BF16, m, k, B.EPS_DEFAULT, xq.data_ptr(), sc.data_ptr(),
            B._stream()))
        rq = lambda c: B._check("bitlinear_rmsnorm_quant_act", B.lib.bitlinear_rmsnorm_quant_act(
            xs[c].data_ptr(), B.BL_BF16, m, k, g.data_ptr(), B.NORM_EPS_DEFAULT, B.EPS_DEFAULT,
            xq.data_ptr(), sc.data_ptr(), B._stream()))
        quant[f"{m}x{k}"] = {"quant_us": time_launches(torch, q, 8, 16)["median"],
                             "rmsnorm_quant_us": time_launches(torch, rq, 8, 16)["median"]}
        del xs
    return {"workload": "2B-class input groups (q/k/v, o, up, down) as fused decode launches "
                        "without / with RMSNorm (fp32 gain), 60 layer copies rotating; bf16 "
                        "activation rows through quant_act / rmsnorm_quant_act",
            "fused_step_us": fused, "act_quant": quant}


# ---------------------------------------------------------- CPU baseline --
def run_cpu_baseline(W, budget_s=8.0):
    """The oracle as it stands on the headline step (one token through the
    100B-class layer): per input group the activation quant, per product the
    integer product and the dequant with its bf16 rounding; codes prepared
    untimed.  Timed on one core and on every core the process may use."""
    import datagen
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    xs = {}
    for g in W.wl.groups():
        bits, _ = datagen.activations(W.wl, g, 1)
        xs[g] = datagen.bf16_bits_to_f32(bits)
    sbytes = step_bytes_fused(W, 1)

    def one_step():
        q = {g: O.quant_act(x) for g, x in xs.items()}
        for name, (codes, g) in W.codes.items():
            d = W.mats[name]
            xq, s = q[d["group"]]
            O.round_output(O.dequant(O.contract(xq, codes), g, s, d["relu2"]), "bf16")

    def timed():
        steps, t0 = 0, time.perf_counter()
        while True:
            one_step()
            steps += 1
            el = time.perf_counter() - t0
            if el > budget_s:
                return steps, el

    allc = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=1):
        s1, e1 = timed()
    with threadpool_limits(limits=allc):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        sa, ea = timed()
    per1, pera = e1 / s1, ea / sa
    return {"value": round(sbytes / pera / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "ms_per_step": round(pera * 1e3, 1),
            "one_core": {"value": round(sbytes / per1 / 1e9, 4), "ms_per_step": round(per1 * 1e3, 1)},
            "host_cpu": host_cpu_model(),
            "sample": f"the headline step (one token, 100B-class layer: 4 act quants, 6 products, "
                      f"dequant; codes prepared untimed): {sa} steps in {ea:.1f} s on all cores, "
                      f"{s1} in {e1:.1f} s on one core"}


def run_cpu_configs(budget_s=1.0):
    """The oracle per configuration on bounded samples, on one core and on
    every core the process may use: the 256x256 layer whole; the 2B-class
    decode set at one token; one 2B-class stack layer at 1, 8 and 64 tokens
    (4 of the tokens timed, scaled to the batch and to 30 layers per pass);
    each 2048-token prefill GEMM (16 tokens timed, scaled to 2048).  The
    oracle's product loops over tokens, so its time is linear in them.
    Per input group the activation quant, per product the integer product
    and the dequant with its output rounding; codes prepared untimed.  The
    100B-class layer is the headline step timed above."""
    import datagen
    import oracle as O
    from threadpoolctl import threadpool_limits

    def prep(wname):
        wl = datagen.WORKLOADS[wname]
        codes = {}
        for nm in wl.matrices:
            w = datagen.workload_weights(wl, nm)
            g = O.absmean_gamma(w)
            codes[nm] = (O.ternary_codes(w, g), g)
            del w
        return wl, codes

    def inputs(wl, m):
        out = {}
        for g in wl.groups():
            if wl.x_dtype == "bf16":
                bits, _ = datagen.activations(wl, g, m)
                out[g] = datagen.bf16_bits_to_f32(bits)
            else:
                out[g] = datagen.activations_f32(wl, g, m)
        return out

    def layer(wl, codes, xs):
        q = {g: O.quant_act(x) for g, x in xs.items()}
        for nm, (c, g) in codes.items():
            _, _, relu2, grp = wl.matrices[nm]
            xq, sv = q[grp]
            O.round_output(O.dequant(O.contract(xq, c), g, sv, relu2), wl.y_dtype)

    allc = len(os.sched_getaffinity(0))

    def per_call(fn):
        out = []
        for lim in (1, allc):
            with threadpool_limits(limits=lim):
                n, t0 = 0, time.perf_counter()
                while True:
                    fn()
                    n += 1
                    el = time.perf_counter() - t0
                    if el > budget_s:
                        break
            out.append(el / n)
        return out                                   # seconds per call: one core, all cores

    def entry(sec, scale, nbytes=None, ops=None, what=""):
        r = {"sample": what}
        for tag, t in zip(("one_core", "all_cores"), sec):
            d = {"ms": round(t * scale * 1e3, 2)}
            if nbytes:
                d["GBs"] = round(nbytes / (t * scale) / 1e9, 4)
            if ops:
                d["TOPS"] = round(ops / (t * scale) / 1e12, 6)
            r[tag] = d
        return r

    res = {"cores": allc}
    wl, codes = prep("c1")
    xs = inputs(wl, 4)
    res["c1"] = entry(per_call(lambda: layer(wl, codes, xs)), 1.0, what="the whole 4x256->256 layer")
    wl, codes = prep("c2")
    xs = inputs(wl, 1)
    nb = sum(fused_bytes(1, n, k) for (n, k, _, _) in wl.matrices.values())
    res["c2"] = entry(per_call(lambda: layer(wl, codes, xs)), 1.0, nbytes=nb,
                      what="the decode set (q,k,v,o,up,down) at one token")
    wl, codes = prep("c3")
    res["c3"] = {}
    for m in (1, 8, 64):
        sm = min(m, 4)
        xs = inputs(wl, m)
        xs = {g: x[:sm] for g, x in xs.items()}
        nb = wl.layers * sum(fused_bytes(m, n, k) for (n, k, _, _) in wl.matrices.values())
        res["c3"][str(m)] = entry(per_call(lambda: layer(wl, codes, xs)), wl.layers * m / sm,
                                  nbytes=nb, what=f"one layer, {sm} of {m} tokens timed, scaled "
                                                  f"x{m / sm:g} to {m} tokens and x{wl.layers} to a pass")
    del codes
    wl, codes = prep("c4")
    res["c4"] = {}
    M, sm = 2048, 16
    xs_all = inputs(wl, sm)
    for nm, (c, g) in codes.items():
        n, k, relu2, grp = wl.matrices[nm]
        x = xs_all[grp]

        def gemm(x=x, c=c, g=g, relu2=relu2):
            xq, sv = O.quant_act(x)
            O.round_output(O.dequant(O.contract(xq, c), g, sv, relu2), wl.y_dtype)
        res["c4"][nm] = entry(per_call(gemm), M / sm, ops=2.0 * M * n * k,
                              what=f"{sm} of {M} tokens through {M}x{k}->{n} timed, scaled x{M // sm}")
    return res


def host_cpu_model():
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name}, {len(os.sched_getaffinity(0))} logical CPUs available"


def environment(torch):
    rocm = "unknown"
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", "unknown"),
            "compute_units": props.multi_processor_count, "rocm": rocm,
            "torch": torch.__version__}


# ---------------------------------------------------------- profiling aids --
KERNEL_SOURCES = ["bit_gemm_int8_amd/csrc/gemv_stream.hip", "bit_gemm_int8_amd/csrc/bl_device.h",
                  "bit_gemm_int8_amd/csrc/bl_internal.h"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_fused_c5_updown_traffic.md")
COPY_BYTES = 256 << 20


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes of one fused up + one fused down launch from the committed
    counter summary, or None when the kernel sources changed since."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    vals = dict(l.split(":", 1) for l in text.splitlines() if l.startswith("- ") and ":" in l)
    vals = {k[2:].strip(): v.strip() for k, v in vals.items()}
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch_pair"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch):
    """A plain copy of COPY_BYTES, three times: what FETCH_SIZE / WRITE_SIZE
    read for it scales the counters of the other kernels to bytes."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def pmc_driver(B, torch, args):
    """Launches to read counters or traces from.
    c5gemv: a plain copy of COPY_BYTES (the counter calibration), then the
            fused up and down launches of the headline, `steps` each, over
            their rotating copies (one token); with --graph one eager launch,
            then graphs of one launch per copy, replayed steps // copies
            times (the roofline leg's timing);
    step:   `steps` headline decode steps (eager);
    prefill: the two 2048-token prefill GEMMs, `steps` times each;
    mfma:   the copy calibration, then bitlinear_forward at --m tokens on the
            2B-class q/up/down (--m <= 64) or the 100B-class k/v (--m > 64),
            `steps` times each over rotating copies;
    c3:     `steps` passes of the 2B-class stack at --m tokens."""
    import datagen
    if args.pmc_driver == "prefill":
        W = Weights(B, torch, datagen.WORKLOADS["c4"], copies=1)
        X = Inputs(B, torch, W, 2048)
        for name in ("up", "down"):
            for _ in range(args.steps):
                forward_call(B, W, X, name, 0, None)()
            torch.cuda.synchronize()
        print(json.dumps({"pmc_driver": "prefill", "steps": args.steps}))
        return
    if args.pmc_driver == "c3":
        # stack passes at args.m tokens, eager, in the launch configuration
        # of run_stack_c3
        wl = datagen.WORKLOADS["c3"]
        W = Weights(B, torch, wl, copies=wl.layers)
        X = Inputs(B, torch, W, args.m)
        ws = B.Workspace()
        for _ in range(args.steps):
            for l in range(wl.layers):
                for grp in LAYER_GROUPS:
                    fused_call(B, W, X, grp, l, ws)()
        torch.cuda.synchronize()
        print(json.dumps({"pmc_driver": "c3", "steps": args.steps, "m": args.m}))
        return
    if args.pmc_driver == "mfma":
        # the copy calibration, then bitlinear_forward at args.m tokens: the
        # 2B-class q, up and down up to 64 tokens, the 100B-class k and v
        # beyond, each over its rotating copies
        copy_calibration(torch)
        wlname, names = ("c2", ("q", "up", "down")) if args.m <= 64 else ("c5", ("k", "v"))
        W = Weights(B, torch, datagen.WORKLOADS[wlname], names=names)
        X = Inputs(B, torch, W, args.m)
        for nm in names:
            for i in range(args.steps):
                forward_call(B, W, X, nm, i, None)()
            torch.cuda.synchronize()
        print(json.dumps({"pmc_driver": "mfma", "steps": args.steps, "m": args.m}))
        return
    copy_calibration(torch)
    W = Weights(B, torch, datagen.WORKLOADS["c5"],
                names=None if args.pmc_driver == "step" else ["up", "down"])
    X = Inputs(B, torch, W, 1)
    ws = B.Workspace()
    if args.pmc_driver == "step":
        layers = copies_for(sum(B.packed_bytes(d["n"], d["k"]) for d in W.mats.values()))
        steps = [[fused_call(B, W, X, grp, l, ws) for grp in LAYER_GROUPS] for l in range(layers)]
        for i in range(args.steps):
            for c in steps[i % layers]:
                c()
    else:
        for nm in ("up", "down"):
            calls = [fused_call(B, W, X, (nm,), c, ws) for c in range(W.copies(nm))]
            if args.graph:
                # as the roofline leg times them: graphs of consecutive launches
                # over the rotating copies, replayed (one eager launch first)
                calls[0]()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                s = torch.cuda.Stream()
                with torch.cuda.graph(g, stream=s):
                    for c in calls:
                        c()
                for _ in range(max(1, args.steps // len(calls))):
                    g.replay()
                torch.cuda.synchronize()
                del g
            else:
                for i in range(args.steps):
                    calls[i % len(calls)]()
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(json.dumps({"pmc_driver": args.pmc_driver, "steps": args.steps}))


def _kname(s):
    return s.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def summarize(directory, command, name):
    """Write profiles/ summaries from rocprofv3 CSV output in `directory`:
    <name>_kernel_stats.md from a kernel trace; from counter runs, the fused
    up/down launches' HBM traffic (FETCH_SIZE / WRITE_SIZE against the copy
    calibration), MFMA counters, or LDS/wait counters."""
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True):
        rows = list(csv.DictReader(open(f)))
        lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "",
                 f"Command: `{command}`", "",
                 "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| {_kname(r['Name'])} | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                         f"{float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} | {float(r['Percentage']):.2f} |")
        out.append((f"{name}_kernel_stats.md", "\n".join(lines) + "\n"))
    vals, durs = {}, {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = _kname(r["Kernel_Name"])
            vals.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
            if "Start_Timestamp" in r:
                durs.setdefault(k, []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    ctrs = {c for (_, c) in vals}

    def med(kern_sub, ctr):
        v = [x for (k, c), xs in vals.items() if kern_sub in k and c == ctr for x in xs]
        return statistics.median(v) if v else None

    f = lambda v, fmt: "-" if v is None else format(v, fmt)
    updown = any("gemv_stream_fused_kernel" in k for (k, c) in vals)
    if updown and ("FETCH_SIZE" in ctrs or "WRITE_SIZE" in ctrs):
        def largest(kern_sub, ctr):
            v = [x for (k, c), xs in vals.items() if kern_sub in k and c == ctr for x in xs]
            return max(v) if v else None
        copy_f, copy_w = largest("copy", "FETCH_SIZE"), largest("copy", "WRITE_SIZE")
        kib = COPY_BYTES / 1024
        ff = kib / copy_f if copy_f else None
        fw = kib / copy_w if copy_w else None
        kernels = sorted({k for (k, c) in vals if "gemv_stream_fused_kernel" in k})
        lines = ["# HBM traffic of the fused one-token GEMV on the 100B-class up and down "
                 "products (rocprofv3 --pmc)", "",
                 f"Commands: `{command}` (one run with FETCH_SIZE, one with WRITE_SIZE)", "",
                 "Median per dispatch, KiB as the counters report them; the copy kernel moves "
                 f"{COPY_BYTES >> 20} MiB each way and sets the scale factors.  One kernel "
                 "instance per product (up: rows of 8192 inputs; down: rows of 28672, the "
                 "long-row instance).", "",
                 f"- copy_fetch_kib: {copy_f}", f"- copy_write_kib: {copy_w}",
                 f"- fetch_scale: {ff}", f"- write_scale: {fw}"]
        total = 0
        ok = ff is not None and fw is not None
        for k in kernels:
            kf, kw = med(k, "FETCH_SIZE"), med(k, "WRITE_SIZE")
            lines += [f"- {k} fetch_kib: {kf}", f"- {k} write_kib: {kw}"]
            if ok and kf is not None and kw is not None:
                total += (kf * ff + kw * fw) * 1024
            else:
                ok = False
        lines += [f"- traffic_bytes_per_launch_pair: {int(round(total)) if ok else None}",
                  f"- kernel_source_sha256_16: {kernel_source_hash()}", ""]
        out.append((f"{name}_traffic.md", "\n".join(lines)))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in ctrs:
        kernels = sorted({k for (k, c), xs in vals.items()
                          if c == "SQ_VALU_MFMA_BUSY_CYCLES" and max(xs) > 0})
        lines = ["# MFMA counters (rocprofv3 --pmc)", "",
                 f"Command: `{command}`", "",
                 "Medians per dispatch.  GRBM_GUI_ACTIVE is summed over the "
                 f"{XCDS} XCDs; per XCD it counts the kernel's GPU cycles, so cycles / duration "
                 "is the clock.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD "
                 f"x {SIMDS} SIMDs); int8 ops = SQ_INSTS_VALU_MFMA_MOPS_I8 x 512 (padded tiles "
                 "included).", "",
                 "| kernel | us | GHz | MFMA busy | int8 ops | int8 TOPS | waves | "
                 "SQ_WAIT_INST_ANY / SQ_BUSY_CYCLES |", "|---|---|---|---|---|---|---|---|"]
        for k in kernels:
            busy, act = med(k, "SQ_VALU_MFMA_BUSY_CYCLES"), med(k, "GRBM_GUI_ACTIVE")
            mops = med(k, "SQ_INSTS_VALU_MFMA_MOPS_I8")
            waves, wait, sqb = med(k, "SQ_WAVES"), med(k, "SQ_WAIT_INST_ANY"), med(k, "SQ_BUSY_CYCLES")
            us = statistics.median(durs[k]) if durs.get(k) else None
            per_xcd = act / XCDS if act else None
            ghz = per_xcd / (us * 1e3) if per_xcd and us else None
            util = busy / (per_xcd * SIMDS) if busy and per_xcd else None
            ops = mops * 512 if mops is not None else None
            tops = ops / (us * 1e-6) / 1e12 if ops and us else None
            wr = wait / sqb if wait and sqb else None
            lines.append(f"| {k} | {f(us, '.2f')} | {f(ghz, '.3f')} | {f(util, '.3f')} | "
                         f"{f(ops, '.4g')} | {f(tops, '.0f')} | {f(waves, '.0f')} | {f(wr, '.2f')} |")
        out.append((f"{name}_mfma_counters.md", "\n".join(lines) + "\n"))
    if "SQ_LDS_BANK_CONFLICT" in ctrs:
        kernels = sorted({k for (k, c), xs in vals.items() if c in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT")
                          and max(xs) > 0})
        lines = ["# LDS and wait counters (rocprofv3 --pmc)", "",
                 f"Command: `{command}`", "",
                 "Medians per dispatch.  SQ_WAIT_INST_LDS and SQ_WAIT_INST_ANY count wave-cycles "
                 "(summed over waves) spent waiting; SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE "
                 "count cycles of the LDS pipes.", "",
                 "| kernel | us | SQ_INSTS_LDS | SQ_LDS_BANK_CONFLICT | SQ_LDS_IDX_ACTIVE | "
                 "SQ_WAIT_INST_LDS | SQ_WAIT_INST_ANY | SQ_BUSY_CYCLES |",
                 "|---|---|---|---|---|---|---|---|"]
        for k in kernels:
            us = statistics.median(durs[k]) if durs.get(k) else None
            lines.append(f"| {k} | {f(us, '.2f')} | " + " | ".join(
                f(med(k, c), ".0f") for c in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
                                               "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS",
                                               "SQ_WAIT_INST_ANY", "SQ_BUSY_CYCLES")) + " |")
        out.append((f"{name}_lds_counters.md", "\n".join(lines) + "\n"))
    if ctrs and not out:
        # any other counter set: one row per kernel, medians per dispatch;
        # FETCH_SIZE / WRITE_SIZE also as bytes, scaled by the copy kernel's
        cols = sorted(ctrs)
        scale = {}
        for ctr, per in (("FETCH_SIZE", "FETCH"), ("WRITE_SIZE", "WRITE")):
            cv = [x for (k, c), xs in vals.items() if "copy" in k and c == ctr for x in xs]
            if cv:
                scale[ctr] = (COPY_BYTES / 1024) / max(cv)
        kernels = sorted({k for (k, c) in vals})
        extra = [c for c in ("FETCH_SIZE", "WRITE_SIZE") if c in scale]
        lines = ["# Counters per dispatch (rocprofv3 --pmc)", "",
                 f"Command: `{command}`", "",
                 "Medians over the dispatches of each kernel instance." +
                 (" Bytes = KiB x 1024 x (copy bytes / the copy kernel's KiB): " +
                  ", ".join(f"{c} scale {scale[c]:.4f}" for c in extra) if extra else ""), "",
                 "| kernel | dispatches | us | " + " | ".join(cols) +
                 "".join(f" | {c} bytes" for c in extra) + " |",
                 "|---|---|---|" + "---|" * (len(cols) + len(extra))]
        for k in kernels:
            us = statistics.median(durs[k]) if durs.get(k) else None
            nd = max(len(xs) for (kk, c), xs in vals.items() if kk == k)
            mv = {c: statistics.median(vals[(k, c)]) if (k, c) in vals else None for c in cols}
            lines.append(f"| {k} | {nd} | {f(us, '.2f')} | " +
                         " | ".join(f(mv[c], ".6g") for c in cols) +
                         "".join(f" | {f(mv[c] * 1024 * scale[c] if mv[c] is not None else None, '.4g')}"
                                 for c in extra) + " |")
        out.append((f"{name}_counters.md", "\n".join(lines) + "\n"))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for fname, text in out:
        with open(os.path.join(ROOT, "profiles", fname), "w") as fh:
            fh.write(text)
        print(f"wrote profiles/{fname}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip every leg after the headline")
    ap.add_argument("--pmc-driver", nargs="?", const="c5gemv",
                    choices=["c5gemv", "step", "prefill", "mfma", "c3"],
                    help="only launch what counters or traces are read from")
    ap.add_argument("--m", type=int, default=64, help="tokens for --pmc-driver mfma / c3")
    ap.add_argument("--graph", action="store_true",
                    help="--pmc-driver c5gemv: replay graphs of the launches instead of eager calls")
    ap.add_argument("--summarize", metavar="DIR", help="write profiles/ summaries from rocprofv3 CSVs")
    ap.add_argument("--name", default="gemv_fused_c5_updown",
                    help="kernel and workload the summaries are named for")
    ap.add_argument("--command", default="", help="command line recorded in the summaries")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.command, args.name)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported (the library has "
              "no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_gemm_int8_amd as B
    import datagen
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.pmc_driver:
        pmc_driver(B, torch, args)
        return
    t0 = time.time()
    log("packing the 100B-class layer")
    W = Weights(B, torch, datagen.WORKLOADS["c5"], codes=not args.no_cpu)
    value, ms, sbytes, layers, rep, roof, plain = run_headline(B, torch, W, args)
    log(f"headline: {ms*1e3:.2f} us/step, {value:.1f} GB/s; fused up+down {roof['achieved']} GB/s")
    extra = {}
    if not args.no_extra:
        extra["c5"] = run_c5(B, torch, W)
    cpu = None if args.no_cpu else run_cpu_baseline(W)
    del W
    if cpu is not None and not args.no_extra:
        log("oracle per configuration")
        cpu["per_config"] = run_cpu_configs()
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra["prefill"] = run_prefill(B, torch)
        log(f"prefill: {extra['prefill']['TOPS']} TOPS")
        extra["c2"] = run_c2(B, torch)
        extra["stack_c3"] = run_stack_c3(B, torch)
        extra["rmsnorm"] = run_rmsnorm(B, torch)
        log("rmsnorm leg done")
    line = {
        "metric": "BitLinear W1.58A8 decode GB/s (% HBM peak) + prefill TOPS (% int8 MFMA)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "batch-1 decode through one 100B-class BitLinear layer: q,o "
                               "8192x8192; k,v 1024x8192; up 28672x8192 (+ReLU^2); down "
                               "8192x28672; bf16 Student-t (nu=3) activations, bf16 outputs; "
                               "one fused launch per input group in layer order",
                   "batch": 1, "layer_copies": layers, "step_bytes": int(sbytes),
                   "step_us_per_replay": rep,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "gemv_plain": plain,
        "cpu_baseline": cpu,
        **extra,
        "env": environment(torch),
        "wall_s": round(time.time() - t0, 1),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
