"""Benchmark of the BitLinear W1.58A8 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Workload (the batch-1 decode set at 2B-class shapes, seeded synthetic data):
q, o 2560x2560; k, v 640x2560; up 6912x2560 with ReLU^2; down 2560x6912;
activations bf16 1 x K ~ N(0,1) with 1% of the channels x100; bf16 outputs.
One step = the whole per-call hot path for that set: absmax int8 quantization
of the four distinct inputs (q/k/v share one) and the six ternary x int8
products with their fused gamma/s (+ReLU^2) epilogues.  Weights are packed
before timing (as at model load) and the packed set is replicated so that
consecutive steps read different copies -- more bytes than the 256 MB
Infinity Cache plus L2 -- so every step streams its weights from HBM.

A step is one launch of the fused decode kernel (bitlinear_forward_fused):
each workgroup quantizes its slice of the activations into LDS and streams
its packed weights.  value = algorithmic bytes of a step / step time (GB/s):
for each matrix N*K/4 (packed W) + 4 (gamma) + 2*M*N (bf16 y), plus each
distinct bf16 input once, 2*M*K (x~ never leaves the chip).

Also reported on the same line:
  roofline      the step's kernel: algorithmic bytes per launch / its mean
                launch duration, from HIP events around a graph replay of
                back-to-back launches on the stream the kernels run on; also
                the same step unfused and each matrix's plain GEMV;
  prefill       2048-token prefill GEMMs (2048x2560 -> 6912 with ReLU^2, and
                2048x6912 -> 2560): 2*M*N*K / kernel time, in TOPS;
  c5            one 100B-class layer (q,o 8192x8192; k,v 1024x8192; up
                28672x8192; down 8192x28672) at 1, 16 and 512 tokens,
                weights rotated past the caches: each matrix alone (GB/s,
                TOPS) and the whole layer with its activation quants;
  stack_c3      the 2B-class set as a 30-layer stack (388 MB packed), one
                pass in layer order at 1/8/32/64 tokens: us per pass;
  cpu_baseline  the CPU oracle (numpy) on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
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
CLOCK_GHZ = 2.4                 # MI355X peak engine clock


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


# --------------------------------------------------------------- helpers --
def gemv_bytes(m, n, k):
    return n * k / 4 + m * k + 4 * m + 4 + 2 * m * n


def quant_bytes(m, k):
    return 2 * m * k + m * k + 4 * m


class DecodeSet:
    """Packed weights (several copies), inputs and outputs of one matrix set."""

    def __init__(self, B, torch, wl, m, copies, names=None, mats=None):
        import datagen
        self.B, self.torch, self.m = B, torch, m
        self.names = names or list(wl.matrices.keys())
        if mats is not None:               # the packed copies of another set
            self.mats = mats
        else:
            self.mats = {}
            for name in self.names:
                n, k, relu2, group = wl.matrices[name]
                w = torch.from_numpy(datagen.workload_weights(wl, name)).cuda()
                packed, gamma = B.pack_weights(w)
                del w
                cps = [packed] + [packed.clone() for _ in range(copies - 1)]
                self.mats[name] = dict(n=n, k=k, relu2=relu2, group=group, packed=cps,
                                       gamma=gamma)
        self.groups = []
        for name in self.names:
            g = self.mats[name]["group"]
            if g not in self.groups:
                self.groups.append(g)
        self.x, self.xq, self.s = {}, {}, {}
        for g in self.groups:
            bits, _ = datagen.activations(wl, g, m)
            x = torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
            self.x[g] = x
            xq, s = B.quant_act(x)
            self.xq[g], self.s[g] = xq, s
        self.y = {nm: torch.empty((m, d["n"]), dtype=torch.bfloat16, device="cuda")
                  for nm, d in self.mats.items()}
        self.ws = B.Workspace()
        need = max(B.forward_workspace_bytes(m, d["n"], d["k"]) for d in self.mats.values())
        self.ws.get(need)
        self.copies = copies

    def bytes_step(self):
        b = sum(gemv_bytes(self.m, d["n"], d["k"]) for d in self.mats.values())
        b += sum(quant_bytes(self.m, self.x[g].shape[1]) for g in self.groups)
        return b

    def bytes_step_fused(self):
        """Bytes a step must move: packed weights, gamma, bf16 outputs, and
        each distinct bf16 input once."""
        b = sum(d["n"] * d["k"] / 4 + 4 + 2 * self.m * d["n"] for d in self.mats.values())
        b += sum(2 * self.m * self.x[g].shape[1] for g in self.groups)
        return b

    def quant_into(self):
        B, lib = self.B, self.B.lib
        st = B._stream()
        for g in self.groups:
            x = self.x[g]
            B._check("quant", lib.bitlinear_quant_act(x.data_ptr(), B.BL_BF16, x.shape[0], x.shape[1],
                                                      B.EPS_DEFAULT, self.xq[g].data_ptr(),
                                                      self.s[g].data_ptr(), st))

    def forward_one(self, name, copy):
        d = self.mats[name]
        self.B.forward(self.xq[d["group"]], self.s[d["group"]], d["packed"][copy], d["gamma"],
                       d["n"], d["k"], relu2=d["relu2"], y=self.y[name], workspace=self.ws)

    def step(self, copy):
        self.quant_into()
        for name in self.names:
            self.forward_one(name, copy)

    def step_multi(self, copy):
        """As step, but the matrices that share an input (q, k, v) go to
        one bitlinear_forward_multi call."""
        self.quant_into()
        for g in self.groups:
            names = [nm for nm in self.names if self.mats[nm]["group"] == g]
            if len(names) == 1:
                self.forward_one(names[0], copy)
                continue
            d0 = self.mats[names[0]]
            ops = [dict(packed=self.mats[nm]["packed"][copy], gamma=self.mats[nm]["gamma"],
                        n=self.mats[nm]["n"], relu2=self.mats[nm]["relu2"], y=self.y[nm])
                   for nm in names]
            self.B.forward_multi(self.xq[g], self.s[g], d0["k"], ops, workspace=self.ws)

    def fused_steps(self):
        """One prepared fused call (all matrices, one launch) per weight copy."""
        out = []
        for c in range(self.copies):
            ops = []
            for nm in self.names:
                d = self.mats[nm]
                ops.append(dict(x=self.x[d["group"]], packed=d["packed"][c], gamma=d["gamma"],
                                n=d["n"], k=d["k"], y=self.y[nm], relu2=d["relu2"]))
            out.append(self.B.FusedStep(ops, workspace=self.ws))
        return out


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # warm once outside capture on the same stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def time_launches(torch, launch, count, per_graph, reps=3):
    """Mean GPU time of one launch: `per_graph` launches launch(i) captured in
    one graph (i cycles through `count` variants, e.g. weight copies), the
    graph replayed after a warm-up; best of `reps` timed replays."""
    g = capture(torch, lambda: [launch(i % count) for i in range(per_graph)])
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        g.replay()
        en.record()
        torch.cuda.synchronize()
        best = min(best, st.elapsed_time(en))
    return best / per_graph        # ms


# ------------------------------------------------------------- workloads --
GRAPH_STEPS = 10


def run_decode(B, torch, args):
    import datagen
    wl = datagen.WORKLOADS["c2"]
    set_bytes = sum(B.packed_bytes(n, k) for (n, k, _, _) in wl.matrices.values())
    copies = max(2, math.ceil(2 * CACHE_BYTES / set_bytes))
    copies = GRAPH_STEPS * math.ceil(copies / GRAPH_STEPS)
    log(f"decode set: {set_bytes/1e6:.2f} MB packed, {copies} copies")
    ds = DecodeSet(B, torch, wl, 1, copies)
    fused = ds.fused_steps()
    torch.cuda.synchronize()

    # the fused step against the unfused one (quant + forward per matrix), bitwise
    ds.step(0)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ds.y.items()}
    for v in ds.y.values():
        v.zero_()
    fused[0]()
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k].view(torch.int16), ds.y[k].view(torch.int16)), k

    # graphs of GRAPH_STEPS consecutive steps (consecutive weight copies), and
    # one-step graphs for a remainder
    groups = copies // GRAPH_STEPS
    big = [capture(torch, lambda g0=g0: [fused[g0 * GRAPH_STEPS + i]() for i in range(GRAPH_STEPS)])
           for g0 in range(groups)]
    single = [capture(torch, lambda c=c: fused[c]()) for c in range(GRAPH_STEPS)]
    # replay check against the eager result
    big[0].replay()
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k].view(torch.int16), ds.y[k].view(torch.int16)), k
    for i in range(max(1, args.warmup // GRAPH_STEPS)):
        big[i % groups].replay()
    torch.cuda.synchronize()
    nbig, rest = divmod(args.steps, GRAPH_STEPS)
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for i in range(nbig):
        big[i % groups].replay()
    for i in range(rest):
        single[i].replay()
    en.record()
    torch.cuda.synchronize()
    ms = st.elapsed_time(en) / args.steps
    step_bytes = ds.bytes_step_fused()
    value = step_bytes / (ms * 1e-3) / 1e9

    # dominant (only) kernel of the step: the fused decode kernel, timed alone
    per = copies
    ms_k = time_launches(torch, lambda c: fused[c](), copies, per)
    achieved = step_bytes / (ms_k * 1e-3) / 1e9
    # the same step unfused (quant per input + one GEMV per matrix), and each
    # matrix's plain GEMV alone
    ms_unf = time_launches(torch, lambda c: ds.step(c), copies, copies)
    per_matrix = {}
    for nm in ds.names:
        d = ds.mats[nm]
        t = time_launches(torch, lambda c, nm=nm: ds.forward_one(nm, c), copies, copies)
        per_matrix[nm] = {"us": round(t * 1e3, 3),
                          "GBs": round(gemv_bytes(1, d["n"], d["k"]) / (t * 1e-3) / 1e9, 1)}
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "gemv_fused_kernel (act quant + batch-1 GEMV + dequant, 6 matrices, one launch)",
            "bytes_per_launch": int(step_bytes), "us_per_launch": round(ms_k * 1e3, 3),
            "unfused_step_us": round(ms_unf * 1e3, 3), "plain_gemv_per_matrix": per_matrix}
    return ds, value, ms, step_bytes, roof, copies


def run_prefill(B, torch, args):
    import datagen
    wl = datagen.WORKLOADS["c4"]
    out = {}
    tot_ops, tot_ms = 0.0, 0.0
    for name in ("up", "down"):
        n, k, relu2, group = wl.matrices[name]
        m = 2048
        w = torch.from_numpy(datagen.workload_weights(wl, name)).cuda()
        packed, gamma = B.pack_weights(w)
        del w
        bits, _ = datagen.activations(wl, group, m)
        x = torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
        xq, s = B.quant_act(x)
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = B.Workspace()
        ws.get(B.forward_workspace_bytes(m, n, k))
        t = time_launches(torch, lambda c: B.forward(xq, s, packed, gamma, n, k, relu2=relu2, y=y,
                                                     workspace=ws), 1, 20)
        tq = time_launches(torch, lambda c: B.quant_act(x), 1, 20)
        ops = 2.0 * m * n * k
        tops = ops / (t * 1e-3) / 1e12
        out[name] = {"shape": f"{m}x{k}->{n}", "us": round(t * 1e3, 2), "TOPS": round(tops, 1),
                     "frac": round(tops / INT8_PEAK_TOPS, 4), "act_quant_us": round(tq * 1e3, 2)}
        tot_ops += ops
        tot_ms += t
        del packed, xq, x, y
    tops = tot_ops / (tot_ms * 1e-3) / 1e12
    return {"workload": "c4 prefill, 2048 tokens", "TOPS": round(tops, 1), "unit": "TOPS",
            "peak": INT8_PEAK_TOPS, "frac": round(tops / INT8_PEAK_TOPS, 4), "per_matrix": out}


def run_c5(B, torch, args):
    """The 100B-class layer (q, o 8192x8192; k, v 1024x8192; up 28672x8192
    with ReLU^2; down 8192x28672) at 1, 16 and 512 tokens, weights rotated
    past the caches: each matrix's forward alone (x~ given) and the whole
    layer (one activation quant per distinct input + the six forwards),
    also with q, k and v in one bitlinear_forward_multi call; at 1 token
    also the fused step of up and of down alone."""
    import datagen
    wl = datagen.WORKLOADS["c5"]
    set_bytes = sum(B.packed_bytes(n, k) for (n, k, _, _) in wl.matrices.values())
    copies = max(2, math.ceil(2 * CACHE_BYTES / set_bytes))
    base = DecodeSet(B, torch, wl, 1, copies)
    out = {}
    for m in wl.batches:
        ds = base if m == 1 else DecodeSet(B, torch, wl, m, copies, mats=base.mats)
        per = {}
        for nm in ds.names:
            d = ds.mats[nm]
            t = time_launches(torch, lambda c, nm=nm: ds.forward_one(nm, c), copies, 4 * copies)
            b = gemv_bytes(m, d["n"], d["k"])
            ops = 2.0 * m * d["n"] * d["k"]
            per[nm] = {"shape": f"{m}x{d['k']}->{d['n']}", "us": round(t * 1e3, 3),
                       "GBs": round(b / (t * 1e-3) / 1e9, 1),
                       "TOPS": round(ops / (t * 1e-3) / 1e12, 2)}
        tl = time_launches(torch, lambda c: ds.step(c), copies, 2 * copies)
        tm = time_launches(torch, lambda c: ds.step_multi(c), copies, 2 * copies)
        ops = 2.0 * m * sum(d["n"] * d["k"] for d in ds.mats.values())
        res = {"layer_us": round(tl * 1e3, 2),
               "layer_GBs": round(ds.bytes_step() / (tl * 1e-3) / 1e9, 1),
               "layer_TOPS": round(ops / (tl * 1e-3) / 1e12, 2),
               "layer_qkv_multi_us": round(tm * 1e3, 2),
               "layer_qkv_multi_TOPS": round(ops / (tm * 1e-3) / 1e12, 2), "per_matrix": per}
        if m == 1:
            fused = {}
            for nm in ("up", "down"):
                one = DecodeSet(B, torch, wl, 1, copies, names=[nm], mats={nm: base.mats[nm]})
                steps = one.fused_steps()
                t = time_launches(torch, lambda c: steps[c](), copies, 4 * copies)
                b = one.bytes_step_fused()
                fused[nm] = {"us": round(t * 1e3, 3), "GBs": round(b / (t * 1e-3) / 1e9, 1),
                             "frac": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                del one, steps
            res["fused_act_quant"] = fused
        out[str(m)] = res
        log(f"c5 m={m}: layer {tl*1e3:.1f} us")
        if ds is not base:
            del ds
        torch.cuda.empty_cache()
    del base
    torch.cuda.empty_cache()
    return {"workload": "c5: one 100B-class layer (q,o 8192x8192; k,v 1024x8192; up "
                        "28672x8192 +ReLU^2; down 8192x28672), packed 155 MB, "
                        f"{copies} copies rotated",
            "per_batch": out}


def run_stack_c3(B, torch, args):
    """The c3 stack: the 2B-class set as 30 layers, each with its own copy of
    the packed weights (388 MB in all, past the caches).  One pass = every
    layer in order: q/k/v (one shared input), o, up (ReLU^2), down, at 1, 8,
    32 and 64 tokens with Student-t activations.  Each group is one fused
    decode launch (activation quant in its prologue) at 1-2 tokens, and at
    3-64 tokens when it holds several matrices; otherwise one activation
    quant per distinct input and one forward per matrix.  A pass
    is captured as one graph; the best of a few replays is reported."""
    import datagen
    wl = datagen.WORKLOADS["c3"]
    layers = wl.layers
    mats = {}
    for name, (n, k, relu2, group) in wl.matrices.items():
        w = torch.from_numpy(datagen.workload_weights(wl, name)).cuda()
        packed, gamma = B.pack_weights(w)
        del w
        mats[name] = dict(n=n, k=k, relu2=relu2, group=group, gamma=gamma,
                          packed=[packed] + [packed.clone() for _ in range(layers - 1)])
    order = [("q", "k", "v"), ("o",), ("up",), ("down",)]
    lib = B.lib
    out = {}
    for m in wl.batches:
        xs = {}
        for g in wl.groups():
            bits, _ = datagen.activations(wl, g, m)
            xs[g] = torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
        ys = {nm: torch.empty((m, d["n"]), dtype=torch.bfloat16, device="cuda")
              for nm, d in mats.items()}
        ws = B.Workspace()
        calls = []
        # a group runs as one fused step (activation quant in the kernel)
        # at 1-2 tokens, and at 3-64 tokens when it has several matrices
        # sharing its input (q, k, v); otherwise as one activation quant plus
        # one forward per matrix (from 3 tokens a fused step re-quantizes
        # the input in every workgroup, which a single matrix does not repay)
        xq = {g: torch.empty((m, B.padded_k(x.shape[1])), dtype=torch.int8, device="cuda")
              for g, x in xs.items()}
        sc = {g: torch.empty(m, dtype=torch.float32, device="cuda") for g in xs}
        ws.get(max(B.forward_workspace_bytes(m, d["n"], d["k"]) for d in mats.values()))

        def quant(g):
            x = xs[g]
            B._check("quant", lib.bitlinear_quant_act(
                x.data_ptr(), B.BL_BF16, m, x.shape[1], B.EPS_DEFAULT, xq[g].data_ptr(),
                sc[g].data_ptr(), B._stream()))

        def gemm(nm, l):
            d = mats[nm]
            B.forward(xq[d["group"]], sc[d["group"]], d["packed"][l], d["gamma"], d["n"],
                      d["k"], relu2=d["relu2"], y=ys[nm], workspace=ws)

        for l in range(layers):
            for grp in order:
                if m <= 2 or (m <= B.BL_FUSED_MAX_M and len(grp) > 1):
                    ops = [dict(x=xs[mats[nm]["group"]], packed=mats[nm]["packed"][l],
                                gamma=mats[nm]["gamma"], n=mats[nm]["n"], k=mats[nm]["k"],
                                y=ys[nm], relu2=mats[nm]["relu2"]) for nm in grp]
                    calls.append(B.FusedStep(ops, workspace=ws))
                else:
                    calls.append(lambda g=mats[grp[0]]["group"]: quant(g))
                    for nm in grp:
                        calls.append(lambda nm=nm, l=l: gemm(nm, l))
        torch.cuda.synchronize()
        g = capture(torch, lambda: [c() for c in calls])
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(5):
            st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            st.record()
            g.replay()
            en.record()
            torch.cuda.synchronize()
            best = min(best, st.elapsed_time(en))
        by = layers * (sum(d["n"] * d["k"] / 4 + 4 + 2 * m * d["n"] for d in mats.values()) +
                       sum(2 * m * x.shape[1] for x in xs.values()))
        ops = 2.0 * m * layers * sum(d["n"] * d["k"] for d in mats.values())
        out[str(m)] = {"us_per_pass": round(best * 1e3, 1), "launches": len(calls),
                       "GBs": round(by / (best * 1e-3) / 1e9, 1),
                       "TOPS": round(ops / (best * 1e-3) / 1e12, 2)}
        log(f"c3 stack m={m}: {best*1e3:.1f} us/pass")
        del g, calls, xs, ys, ws
        torch.cuda.empty_cache()
    return {"workload": "c3: 30 layers x {q,k,v,o,up,down} at 2B-class shapes, one pass in "
                        "layer order, packed weights 388 MB",
            "per_batch": out}


def run_cpu_baseline(budget_s=12.0):
    """The oracle as it stands, on the same decode step: activation quant, the
    six integer products and the dequant, codes prepared beforehand."""
    import numpy as np
    import datagen
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    wl = datagen.WORKLOADS["c2"]
    mats = {}
    for name, (n, k, relu2, group) in wl.matrices.items():
        w = datagen.workload_weights(wl, name)
        g = O.absmean_gamma(w)
        mats[name] = (O.ternary_codes(w, g), g, relu2, group, n, k)
    xs = {}
    for grp in ("attn_in", "o_in", "up_in", "down_in"):
        bits, _ = datagen.activations(wl, grp, 1)
        xs[grp] = O.bf16_bits_to_f32(bits)
    step_bytes = sum(gemv_bytes(1, n, k) for (_, _, _, _, n, k) in mats.values())
    step_bytes += sum(quant_bytes(1, x.shape[1]) for x in xs.values())
    steps = 0
    t0 = time.perf_counter()
    while True:
        q = {grp: O.quant_act(x) for grp, x in xs.items()}
        for name, (codes, g, relu2, grp, n, k) in mats.items():
            xq, s = q[grp]
            acc = O.contract(xq, codes)
            O.round_output(O.dequant(acc, g, s, relu2), "bf16")
        steps += 1
        el = time.perf_counter() - t0
        if el > budget_s:
            break
    per = el / steps
    return {"value": round(step_bytes / per / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "ms_per_step": round(per * 1e3, 2), "host_cpu": host_cpu_model(),
            "sample": f"{steps} full decode steps of the same workload (4 act quants, 6 products, "
                      f"dequant; codes prepared untimed), {el:.1f} s"}


def host_cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo) and the
    logical CPUs this process may use."""
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
    """Software and device the numbers were taken on."""
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
KERNEL_SOURCES = ["bit_gemm_int8_amd/csrc/gemv.hip", "bit_gemm_int8_amd/csrc/bl_device.h"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_fused_decode_2b_traffic.md")
COPY_BYTES = 256 << 20


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the fused decode kernel from the committed
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
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pmc_driver(B, torch, args):
    """Launches to read counters from.  decode: a plain copy of COPY_BYTES
    (the calibration), then eager fused decode steps over rotating weight
    copies.  prefill: the two 2048-token prefill GEMMs, `steps` times each.
    gemv: the 100B-class up and down products at one token (plain GEMV),
    `steps` times each over rotating weight copies."""
    import datagen
    if args.pmc_driver == "gemv":
        wl = datagen.WORKLOADS["c5"]
        ds = DecodeSet(B, torch, wl, 1, 1, names=["up", "down"])
        copies = max(2, math.ceil(2 * CACHE_BYTES / B.packed_bytes(*wl.matrices["up"][:2])))
        for name in ("up", "down"):
            d = ds.mats[name]
            d["packed"] = d["packed"] + [d["packed"][0].clone() for _ in range(copies - 1)]
            for i in range(args.steps):
                ds.forward_one(name, i % copies)
            torch.cuda.synchronize()
            d["packed"] = d["packed"][:1]
            torch.cuda.empty_cache()
        print(json.dumps({"pmc_driver": "gemv", "steps": args.steps, "copies": copies}))
        return
    if args.pmc_driver == "prefill":
        wl = datagen.WORKLOADS["c4"]
        for name in ("up", "down"):
            n, k, relu2, group = wl.matrices[name]
            w = torch.from_numpy(datagen.workload_weights(wl, name)).cuda()
            packed, gamma = B.pack_weights(w)
            del w
            bits, _ = datagen.activations(wl, group, 2048)
            x = torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
            xq, s = B.quant_act(x)
            y = torch.empty((2048, n), dtype=torch.bfloat16, device="cuda")
            for _ in range(args.steps):
                B.forward(xq, s, packed, gamma, n, k, relu2=relu2, y=y)
            torch.cuda.synchronize()
        print(json.dumps({"pmc_driver": "prefill", "steps": args.steps}))
        return
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    wl = datagen.WORKLOADS["c2"]
    set_bytes = sum(B.packed_bytes(n, k) for (n, k, _, _) in wl.matrices.values())
    copies = max(2, math.ceil(2 * CACHE_BYTES / set_bytes))
    ds = DecodeSet(B, torch, wl, 1, copies)
    fused = ds.fused_steps()
    for i in range(args.steps):
        fused[i % copies]()
    torch.cuda.synchronize()
    print(json.dumps({"pmc_driver": "decode", "steps": args.steps, "copies": copies,
                      "step_bytes": int(ds.bytes_step_fused())}))


def _kname(s):
    return s.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def summarize(directory, command, name):
    """Write profiles/ summaries from rocprofv3 CSV output in `directory`:
    <name>_kernel_stats.md from a kernel trace; from counter runs, the
    fused decode kernel's HBM traffic (FETCH_SIZE / WRITE_SIZE against the
    copy calibration) or the GEMM kernels' MFMA counters."""
    import csv
    import glob
    import statistics
    out = []
    stats = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    for f in stats:
        rows = list(csv.DictReader(open(f)))
        lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "",
                 f"Command: `{command}`", "",
                 "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| {_kname(r['Name'])} | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                         f"{float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} | {float(r['Percentage']):.2f} |")
        out.append((f"{name}_kernel_stats.md", "\n".join(lines) + "\n"))
    pmc = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    vals, durs = {}, {}
    for f in pmc:
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

    if "FETCH_SIZE" in ctrs or "WRITE_SIZE" in ctrs:
        def largest(kern_sub, ctr):
            # the calibration copy is the largest copy the driver makes
            v = [x for (k, c), xs in vals.items() if kern_sub in k and c == ctr for x in xs]
            return max(v) if v else None
        copy_f, copy_w = largest("copy", "FETCH_SIZE"), largest("copy", "WRITE_SIZE")
        gv_f, gv_w = med("gemv_fused_kernel", "FETCH_SIZE"), med("gemv_fused_kernel", "WRITE_SIZE")
        kib = COPY_BYTES / 1024
        ff = kib / copy_f if copy_f else None
        fw = kib / copy_w if copy_w else None
        traffic = int(round((gv_f * ff + gv_w * fw) * 1024)) if None not in (gv_f, gv_w, ff, fw) else None
        lines = ["# HBM traffic of the fused decode kernel (rocprofv3 --pmc)", "",
                 f"Commands: `{command}` (one run with FETCH_SIZE, one with WRITE_SIZE)", "",
                 "Median per dispatch, KiB as the counters report them; the copy kernel moves "
                 f"{COPY_BYTES >> 20} MiB each way and sets the scale factors.", "",
                 f"- copy_fetch_kib: {copy_f}", f"- copy_write_kib: {copy_w}",
                 f"- fetch_scale: {ff}", f"- write_scale: {fw}",
                 f"- kernel_fetch_kib: {gv_f}", f"- kernel_write_kib: {gv_w}",
                 f"- traffic_bytes_per_launch: {traffic}",
                 f"- kernel_source_sha256_16: {kernel_source_hash()}", ""]
        out.append(("gemv_fused_decode_2b_traffic.md", "\n".join(lines)))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in ctrs:
        kernels = sorted({k for (k, c), xs in vals.items()
                          if c == "SQ_VALU_MFMA_BUSY_CYCLES" and max(xs) > 0})
        lines = ["# MFMA counters of the prefill GEMM kernels (rocprofv3 --pmc)", "",
                 f"Command: `{command}`", "",
                 "Medians per dispatch (the profiler serialises dispatches, so durations run "
                 "a little above graph replay).  GRBM_GUI_ACTIVE is reported summed over the "
                 f"{XCDS} XCDs; per XCD it counts the kernel's GPU cycles, so cycles / duration "
                 "is the clock.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD "
                 f"x {SIMDS} SIMDs), the MfmaUtil expression rocprofv3 lists for gfx950; int8 ops "
                 "= SQ_INSTS_VALU_MFMA_MOPS_I8 x 512 (padded tiles included).", "",
                 "| kernel | us | GHz | SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE | MFMA busy | "
                 "int8 ops | int8 TOPS |", "|---|---|---|---|---|---|---|---|"]
        for k in kernels:
            busy, act = med(k, "SQ_VALU_MFMA_BUSY_CYCLES"), med(k, "GRBM_GUI_ACTIVE")
            mops = med(k, "SQ_INSTS_VALU_MFMA_MOPS_I8")
            us = statistics.median(durs[k]) if durs.get(k) else None
            per_xcd = act / XCDS if act else None
            ghz = per_xcd / (us * 1e3) if per_xcd and us else None
            util = busy / (per_xcd * SIMDS) if busy and per_xcd else None
            ops = mops * 512 if mops is not None else None
            tops = ops / (us * 1e-6) / 1e12 if ops and us else None
            f = lambda v, fmt: "-" if v is None else format(v, fmt)
            lines.append(f"| {k} | {f(us, '.2f')} | {f(ghz, '.3f')} | {f(busy, '.0f')} | "
                         f"{f(act, '.0f')} | {f(util, '.3f')} | {f(ops, '.4g')} | {f(tops, '.0f')} |")
        out.append((f"{name}_mfma_counters.md", "\n".join(lines) + "\n"))
    if "SQ_ACTIVE_INST_VALU" in ctrs:
        kernels = sorted({k for (k, c), xs in vals.items()
                          if c == "SQ_INSTS_VALU" and max(xs) > 0 and "gemv" in k})
        lines = ["# VALU counters of the batch-1 GEMV (rocprofv3 --pmc)", "",
                 f"Command: `{command}`", "",
                 "Medians per dispatch.  VALU busy = SQ_ACTIVE_INST_VALU x 4 (the counter is in "
                 f"quad-cycles) / ({SIMDS} SIMDs x the kernel's duration at {CLOCK_GHZ} GHz); for "
                 "dispatches this short GRBM_GUI_ACTIVE / 8 XCDs implies a clock above the "
                 "part's peak (the counter window is wider than the kernel), so it is shown but "
                 "not used.  VALU lane-ops per 1000 weights = SQ_INSTS_VALU x 64 lanes / weights "
                 "of the matrix x 1000 (one 28672 x 8192 matrix per dispatch).", "",
                 "| kernel | us | SQ_INSTS_VALU | SQ_ACTIVE_INST_VALU | GRBM_GUI_ACTIVE | "
                 "VALU busy | VALU lane-ops per 1000 weights |", "|---|---|---|---|---|---|---|"]
        for k in kernels:
            insts, act_v, act = (med(k, "SQ_INSTS_VALU"), med(k, "SQ_ACTIVE_INST_VALU"),
                                 med(k, "GRBM_GUI_ACTIVE"))
            us = statistics.median(durs[k]) if durs.get(k) else None
            busy = act_v * 4 / (SIMDS * us * 1e3 * CLOCK_GHZ) if act_v and us else None
            per_w = insts * 64 / (28672 * 8192) * 1000 if insts else None
            f = lambda v, fmt: "-" if v is None else format(v, fmt)
            lines.append(f"| {k} | {f(us, '.2f')} | {f(insts, '.0f')} | "
                         f"{f(act_v, '.0f')} | {f(act, '.0f')} | {f(busy, '.3f')} | {f(per_w, '.0f')} |")
        out.append((f"{name}_valu_counters.md", "\n".join(lines) + "\n"))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for fname, text in out:
        with open(os.path.join(ROOT, "profiles", fname), "w") as f:
            f.write(text)
        print(f"wrote profiles/{fname}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip prefill and 100B-class legs")
    ap.add_argument("--pmc-driver", nargs="?", const="decode", choices=["decode", "prefill", "gemv"],
                    help="only launch what the counters are read from: the fused decode "
                         "step (HBM traffic), the prefill GEMMs (MFMA) or the batch-1 "
                         "100B-class GEMVs (VALU)")
    ap.add_argument("--summarize", metavar="DIR", help="write profiles/ summaries from rocprofv3 CSVs")
    ap.add_argument("--name", default="gemv_fused_decode_2b",
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
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.pmc_driver:
        pmc_driver(B, torch, args)
        return
    t0 = time.time()
    ds, value, ms, step_bytes, roof, copies = run_decode(B, torch, args)
    roof["traffic"] = recorded_traffic()
    log(f"decode: {ms*1e3:.2f} us/step, {value:.1f} GB/s; gemv {roof['achieved']} GB/s")
    prefill = None if args.no_extra else run_prefill(B, torch, args)
    if prefill:
        log(f"prefill: {prefill['TOPS']} TOPS")
    c5 = None if args.no_extra else run_c5(B, torch, args)
    stack = None if args.no_extra else run_stack_c3(B, torch, args)
    cpu = None if args.no_cpu else run_cpu_baseline()
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
        "config": {"workload": "batch-1 decode of the 2B-class BitLinear set: q,o 2560x2560; "
                               "k,v 640x2560; up 6912x2560 (+ReLU^2); down 2560x6912; "
                               "bf16 in/out, 1% outlier channels x100",
                   "batch": 1, "weight_copies": copies, "step_bytes": int(step_bytes),
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "c5": c5,
        "stack_c3": stack,
        "env": environment(torch),
        "wall_s": round(time.time() - t0, 1),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
