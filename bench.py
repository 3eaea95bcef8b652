"""Throughput of the low-rank decomposed linear on one MI355X.

Workload: the seven projections of a LLaMA-7B-shaped decoder layer
(q, k, v, o: 4096x4096; gate, up: 4096x11008; down: 11008x4096), each
decomposed at parameter ratio 0.6 (r = floor(0.6 d_in d_out / (d_in + d_out))
= 1228 / 1791), bf16, decode with T = 1, 8, 32 and 64 tokens.  One step runs
every T over 32 distinct layer sets (7.8 GB of factors, far beyond the 256 MB
MALL), so weights stream from HBM as in a real 32-layer decode.

Prints one JSON line: whole-job tokens/s (tokens x layer sets / s), the
roofline of the dominant launch, and the fp64 CPU oracle timed on a bounded
sample of the same workload.  Also reports, as context: the prefill
configuration (16384 rows, ratio 0.4 and 0.2) under "prefill", the 32-layer
decode step under "decode_step" (and with the reconstruction inside the
attention under "decode_step_fused"), the 32-layer chunked-prefill step (8
prompts of 512 tokens) under "prefill_step", and one of 8 tensor-parallel
shares of the LLaMA-13B projections (ratio 0.4, T = 64 and 4096) under
"tp_share".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # flop/s, MI355X dense bf16 MFMA
SHAPES = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
          "gate": (4096, 11008), "up": (4096, 11008), "down": (11008, 4096)}
ROLES = ("q", "k", "v", "o", "gate", "up", "down")
TOKENS = (1, 8, 32, 64)
# launches of a layer set: projections that read the same input go out as one
# grouped launch (lowrank_linear_forward_group); o and down read other data
GROUPS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")), ("down", ("down",)))


def log(msg):
    """Progress of the legs on stderr (stdout carries only the JSON line)."""
    print("[bench] " + msg, file=sys.stderr, flush=True)


def recorded_traffic(dom):
    """HBM bytes per launch of the dominant class from the committed counter
    summary (profiles/decode_linear_traffic.json), or None when the class
    differs or the decode kernel's sources changed since it was taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(here, "profiles", "decode_linear_traffic.json")))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in ("linear_decode.hip", "lr_common.h"):
        with open(os.path.join(here, "rank_decomposed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if rec.get("class") != dom or rec.get("sources_sha256") != h.hexdigest():
        return None
    return rec.get("traffic_bytes_per_launch")


def rank(rho, a, b):
    from fractions import Fraction
    return int((Fraction(str(rho)) * a * b) // (a + b))


def decode_bytes(T, d_in, r, d_out):
    """Algorithmic HBM bytes of one decode projection: both factors once, x in,
    y out (bf16); the rank-r intermediate stays on chip."""
    return 2 * r * (d_in + d_out) + 2 * T * (d_in + d_out)


def ld8(n):
    return (n + 7) // 8 * 8


def make_layer_sets(torch, dev, rho, n_sets, seed):
    """Layer set 0: seeded factors with the law of a truncated SVD of an
    N(0, 1/d_in) weight (synth.fast_factors).  Sets 1.. reuse them under a
    seeded signed permutation of the rank components (U_r P D, D P^T V_r): the
    same product, distinct bytes in memory."""
    import synth
    base = {}
    for i, role in enumerate(ROLES):
        d_in, d_out = SHAPES[role]
        r = rank(rho, d_in, d_out)
        U, V = synth.fast_factors(synth.seed_of(2, 0, i, synth.KIND_W), d_in, d_out, r)
        ut = torch.zeros((r, ld8(d_in)), dtype=torch.bfloat16, device=dev)
        vt = torch.zeros((d_out, ld8(r)), dtype=torch.bfloat16, device=dev)
        ut[:, :d_in] = torch.from_numpy(synth.bf16_bits(U.T).view(np.int16)).view(
            torch.bfloat16).to(dev)
        vt[:, :r] = torch.from_numpy(synth.bf16_bits(V.T).view(np.int16)).view(
            torch.bfloat16).to(dev)
        base[role] = (ut, vt, r, U, V)
    sets = []
    g = torch.Generator(device="cpu").manual_seed(seed)
    for s in range(n_sets):
        layer = {}
        for role in ROLES:
            ut, vt, r, _, _ = base[role]
            if s == 0:
                layer[role] = (ut, vt, r)
                continue
            perm = torch.randperm(r, generator=g).to(dev)
            sign = (torch.randint(0, 2, (r,), generator=g) * 2 - 1).to(dev).to(torch.bfloat16)
            u2 = torch.zeros_like(ut)
            v2 = torch.zeros_like(vt)
            u2[:, :] = ut[perm] * sign[:, None]
            v2[:, :r] = vt[:, :r][:, perm] * sign[None, :]
            layer[role] = (u2, v2, r)
        sets.append(layer)
    return base, sets


def pack_sets(lr, sets):
    """Replace each set's row-major factors by fragment-packed copies."""
    for layer in sets:
        for role in list(layer):
            ut, vt, r = layer[role]
            d_in = SHAPES[role][0]
            layer[role] = (lr.pack_factor(ut[:, :d_in]), lr.pack_factor(vt[:, :r]), r)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layer-sets", type=int, default=32)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-step", action="store_true", help="skip the 32-layer decode step")
    ap.add_argument("--no-tp", action="store_true",
                    help="skip the 13B tensor-parallel share leg")
    ap.add_argument("--no-prefill-step", action="store_true",
                    help="skip the 32-layer chunked-prefill step")
    ap.add_argument("--step-layers", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--layout", choices=("packed", "rowmajor"), default="packed",
                    help="device layout of the decode factors")
    ap.add_argument("--probe-class", default=None,
                    help="for hardware-counter runs: negate 256 Mi bf16 (a reference kernel "
                         "of known traffic: 512 MiB in, 512 MiB out), run one launch class "
                         "(e.g. gateup_T64) eagerly over every layer set twice, and exit")
    ap.add_argument("--probe-step", action="store_true",
                    help="for hardware-counter runs: the same reference kernel, then 2 layers "
                         "of the unfused and of the fused decode step, eagerly, twice each, "
                         "and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the low-rank path here has no "
              "cross-GPU exchange; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_decomposed_amd as lr

    dev = torch.device("cuda:0")
    lr.load()
    stream = torch.cuda.current_stream(dev)
    if args.probe_step:
        probe_step(torch, lr, dev)
        return
    base, sets = make_layer_sets(torch, dev, 0.6, args.layer_sets, 1234)
    if args.layout == "packed":
        pack_sets(lr, sets)
        torch.cuda.synchronize()
    gen = torch.Generator(device=dev).manual_seed(2_000_001)
    xs = {T: {d: torch.randn((T, d), generator=gen, device=dev).to(torch.bfloat16)
              for d in (4096, 11008)} for T in TOKENS}
    ys = {T: {role: torch.empty((T, SHAPES[role][1]), dtype=torch.bfloat16, device=dev)
              for role in ROLES} for T in TOKENS}

    def member(T, layer, role):
        ut, vt, r = layer[role]
        d_in, d_out = SHAPES[role]
        if args.layout == "rowmajor":
            ut, vt = ut[:, :d_in], vt[:, :r]
        return dict(x=xs[T][d_in], Ut=ut, Vt=vt, y=ys[T][role])

    ws_bytes = max(lr.lowrank_group_workspace_bytes(T, [member(T, sets[0], r) for r in roles])
                   for T in TOKENS for _, roles in GROUPS)
    ws = torch.zeros(ws_bytes + 256, dtype=torch.uint8, device=dev)

    def call(T, layer, roles):
        if len(roles) == 1:
            m = member(T, layer, roles[0])
            lr.lowrank_linear_forward(m["x"], m["Ut"], m["Vt"], y=m["y"], workspace=ws)
        else:
            lr.lowrank_linear_forward_group([member(T, layer, r) for r in roles], workspace=ws)

    def step():
        for T in TOKENS:
            for layer in sets:
                for _, roles in GROUPS:
                    call(T, layer, roles)

    def capture(fn):
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    log("factors ready (%s layout)" % args.layout)
    if args.probe_class:
        name, T = args.probe_class.split("_T")
        roles = dict(GROUPS)[name]
        reference_kernel(torch, dev)
        for _ in range(2):
            for layer in sets:
                call(int(T), layer, roles)
        torch.cuda.synchronize()
        log("probe done: reference kernel, then %d launches of %s" % (2 * len(sets),
                                                                     args.probe_class))
        return
    # the whole step (512 launches) is one HIP graph, as in the pages' decode
    step_graph = capture(step)
    log("decode step graph captured")
    for _ in range(args.warmup):
        step_graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = time_graph(step_graph, args.steps)
    wall = time.perf_counter() - t0
    tokens_per_step = sum(TOKENS) * len(sets)
    value = tokens_per_step / (ms_step / 1e3)
    log("decode step timed: %.3f ms" % ms_step)

    # per-launch durations: for each launch class and T, a graph of one launch
    # per layer set (distinct weights), timed with events on the stream
    per = {}
    for T in TOKENS:
        for name, roles in GROUPS:
            g = capture(lambda: [call(T, layer, roles) for layer in sets])
            us = 1e3 * time_graph(g, max(3, args.steps)) / len(sets)
            del g
            nbytes = sum(decode_bytes(T, SHAPES[r][0], rank(0.6, *SHAPES[r]), SHAPES[r][1])
                         for r in roles)
            per["%s_T%d" % (name, T)] = {"us": round(us, 3), "GBps": round(nbytes / us / 1e3, 1),
                                         "frac": round(nbytes / (us * 1e-6) / HBM_PEAK, 4),
                                         "bytes": nbytes, "share": us}
        log("per-launch timing T=%d done" % T)
    total_share = sum(v["share"] for v in per.values())
    for v in per.values():
        v["share"] = round(v["share"] / total_share, 4)
    per_T = {}
    for T in TOKENS:
        bt = sum(decode_bytes(T, SHAPES[r][0], rank(0.6, *SHAPES[r]), SHAPES[r][1]) for r in ROLES)
        per_T[str(T)] = bt
    dom = max(per, key=lambda k: per[k]["share"])
    dom_name, dom_T = dom.split("_T")
    dom_roles = dict(GROUPS)[dom_name]
    dom_bytes = per[dom]["bytes"]
    dom_us = per[dom]["us"]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    result = {
        "metric": "low-rank linear tokens/s at 7B shapes (decode+prefill); % of HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "tokens/s (x 7-projection layer set)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LLaMA-7B decomposed projections (q,k,v,o 4096x4096; gate,up "
                               "4096x11008; down 11008x4096), ratio 0.6, decode T=1,8,32,64, "
                               "32 rotating layer sets; q,k,v and gate,up as grouped launches",
                   "tokens_per_step": tokens_per_step, "layer_sets": len(sets),
                   "factor_layout": args.layout},
        "roofline": {"bound": "hbm",
                     "kernel": "decode linear, one launch (%s), %s T=%s" % (
                         "lowrank_linear_forward_group" if len(dom_roles) > 1
                         else "lowrank_linear_forward",
                         " + ".join("%s %dx%dx%d" % (r, SHAPES[r][0], rank(0.6, *SHAPES[r]),
                                                     SHAPES[r][1]) for r in dom_roles), dom_T),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved * 1e9 / HBM_PEAK, 4),
                     "traffic": recorded_traffic(dom),
                     "bytes_per_launch": dom_bytes, "us_per_launch": dom_us},
        "launches": per,
        "wall_s": round(wall, 3),
    }

    # whole-step roofline fraction (all T, all projections)
    step_bytes = len(sets) * sum(per_T.values())
    result["step_hbm_frac"] = round(step_bytes / (ms_step * 1e-3) / HBM_PEAK, 4)

    if not args.no_prefill:
        result["prefill"] = prefill(torch, lr, dev, stream)
        log("prefill leg done")
    if not args.no_step:
        del sets
        torch.cuda.empty_cache()
        result["decode_step"] = decode_step(torch, lr, dev, stream, args.step_layers,
                                            max(3, args.steps // 2))
        log("decode-step leg done")
        torch.cuda.empty_cache()
        result["decode_step_fused"] = decode_step(torch, lr, dev, stream, args.step_layers,
                                                  max(3, args.steps // 2), fused=True)
        log("fused decode-step leg done")

    if not args.no_prefill_step:
        torch.cuda.empty_cache()
        result["prefill_step"] = prefill_step(torch, lr, dev, stream, args.step_layers,
                                              max(3, args.steps // 2))
        log("prefill-step leg done")

    if not args.no_tp:
        torch.cuda.empty_cache()
        result["tp_share"] = tp_share(torch, lr, dev, stream, max(3, args.steps // 2))
        log("tp-share leg done")

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(base, args.cpu_seconds)
        log("cpu baseline done")
    print(json.dumps(result), flush=True)


def prefill(torch, lr, dev, stream, M=16384, reps=3):
    """16384 rows (8 x 2048) through the seven projections at ratio 0.4 and
    0.2, each on its two large-tile GEMMs with t through HBM (the path the
    library takes from 1024 rows on); MFMA-bound, so one layer set suffices.
    A context entry times the fused kernel (t kept in LDS) on the same rows
    for three projections."""
    import synth
    out = {}
    gen = torch.Generator(device=dev).manual_seed(3_000_001)
    x = {d: torch.randn((M, d), generator=gen, device=dev).to(torch.bfloat16) for d in (4096, 11008)}
    y = {d: torch.empty((M, d), dtype=torch.bfloat16, device=dev) for d in (4096, 11008)}
    for rho in (0.4, 0.2):
        fac = {}
        flops = 0
        for i, role in enumerate(ROLES):
            d_in, d_out = SHAPES[role]
            r = rank(rho, d_in, d_out)
            ut = (torch.randn((r, d_in), generator=gen, device=dev) * 0.05).to(torch.bfloat16)
            vt = torch.zeros((d_out, ld8(r)), dtype=torch.bfloat16, device=dev)
            vt[:, :r] = (torch.randn((d_out, r), generator=gen, device=dev) * 0.05)
            fac[role] = (ut, vt[:, :r], r)
            flops += 2 * M * r * (d_in + d_out)
        ws = torch.zeros(max(lr.lowrank_workspace_bytes(0, lr.LR_BF16, M, SHAPES[r_][0],
                                                        fac[r_][2], SHAPES[r_][1])
                             for r_ in ROLES) + 256, dtype=torch.uint8, device=dev)

        def run():
            for role in ROLES:
                ut, vt, r = fac[role]
                d_in, d_out = SHAPES[role]
                lr.lowrank_linear_forward(x[d_in], ut, vt, y=y[d_out], workspace=ws)
        run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        # single-launch time of the largest projection (gate)
        ut, vt, r = fac["gate"]
        a.record(stream)
        for _ in range(reps):
            lr.lowrank_linear_forward(x[4096], ut, vt, y=y[11008], workspace=ws)
        b.record(stream)
        torch.cuda.synchronize()
        gate_us = 1e3 * a.elapsed_time(b) / reps
        gate_fl = 2 * M * r * (4096 + 11008)
        # context: the fused kernel (rank tile kept in LDS, 64-row tiles) at
        # the same 16384 rows, per projection, against the two-GEMM path
        cmp = {}
        for role in ("q", "gate", "down"):
            ut, vt, r_ = fac[role]
            d_in, d_out = SHAPES[role]
            us = {}
            for name, fl in (("two_gemm", lr.LR_FULL), ("fused", lr.LR_PREFILL_FUSED)):
                lr.lowrank_linear_forward(x[d_in], ut, vt, y=y[d_out], flags=fl, workspace=ws)
                a.record(stream)
                for _ in range(reps):
                    lr.lowrank_linear_forward(x[d_in], ut, vt, y=y[d_out], flags=fl,
                                              workspace=ws)
                b.record(stream)
                torch.cuda.synchronize()
                us[name] = 1e3 * a.elapsed_time(b) / reps
            fl_ = 2 * M * r_ * (d_in + d_out)
            cmp[role] = {"r": r_, "two_gemm_us": round(us["two_gemm"], 2),
                         "fused_us": round(us["fused"], 2),
                         "two_gemm_frac": round(fl_ / (us["two_gemm"] * 1e-6) / BF16_PEAK, 4),
                         "fused_frac": round(fl_ / (us["fused"] * 1e-6) / BF16_PEAK, 4)}
        out["rho%.1f" % rho] = {
            "tokens_per_s": round(M / (ms * 1e-3), 1), "ms_per_layer_set": round(ms, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac": round(flops / (ms * 1e-3) / BF16_PEAK, 4),
            "gate_us": round(gate_us, 2),
            "gate_frac": round(gate_fl / (gate_us * 1e-6) / BF16_PEAK, 4),
            "fused_vs_two_gemm": cmp}
    return out


SHAPES_13B = {"q": (5120, 5120), "k": (5120, 5120), "v": (5120, 5120), "o": (5120, 5120),
              "gate": (5120, 13824), "up": (5120, 13824), "down": (13824, 5120)}


def tp_share(torch, lr, dev, stream, reps, n_sets=32, P=8):
    """One of 8 tensor-parallel shares of the LLaMA-13B projections at ratio
    0.4 (r = 1024 / 1494): U_r split by input rows, so stage 1 forms the
    share's partial rank-space t_s [T, r], materialized in fp32 (the tensor
    the shares would all-reduce); V_r split by output columns, so stage 2
    writes [T, d_out / 8].  32 distinct share sets (1 GB of factors) stream
    from HBM; each pass over them is one HIP graph.  T = 64 is HBM-bound
    (fragment-packed factors, as in the decode leg; projections that read the
    same x_s grouped into one launch per stage), T = 4096 MFMA-bound
    (row-major factors on the large-tile GEMMs)."""
    import math
    gen = torch.Generator(device=dev).manual_seed(4_000_001)
    sets = []
    for _ in range(n_sets):
        layer = {}
        for role in ROLES:
            d_in, d_out = SHAPES_13B[role]
            r, wi, wo = rank(0.4, d_in, d_out), d_in // P, d_out // P
            ut = torch.zeros((r, ld8(wi)), dtype=torch.bfloat16, device=dev)
            vt = torch.zeros((wo, ld8(r)), dtype=torch.bfloat16, device=dev)
            ut[:, :wi] = torch.randn((r, wi), generator=gen, device=dev) / math.sqrt(d_in)
            vt[:, :r] = torch.randn((wo, r), generator=gen, device=dev) / math.sqrt(r)
            layer[role] = (ut[:, :wi], vt[:, :r], r)
        sets.append(layer)
    out = {}
    for T in (64, 4096):
        use = sets
        if T <= 64:
            use = [{role: (lr.pack_factor(ut), lr.pack_factor(vt), r)
                    for role, (ut, vt, r) in layer.items()} for layer in sets]
        xs = {w: torch.randn((T, w), generator=gen, device=dev).to(torch.bfloat16)
              for w in (640, 1728)}
        ts = {role: torch.empty((T, rank(0.4, *SHAPES_13B[role])), dtype=torch.float32,
                                device=dev) for role in ROLES}
        ys = {role: torch.empty((T, SHAPES_13B[role][1] // P), dtype=torch.bfloat16,
                                device=dev) for role in ROLES}
        need = 0
        nbytes = flops = 0
        for role in ROLES:
            d_in, d_out = SHAPES_13B[role]
            r, wi, wo = rank(0.4, d_in, d_out), d_in // P, d_out // P
            need = max(need, lr.lowrank_workspace_bytes(0, lr.LR_BF16, T, wi, r, wo))
            # shares, x_s, y_s, and t written and read once (counted at 2 bytes)
            nbytes += 2 * r * (wi + wo) + 2 * T * (wi + wo) + 2 * 2 * T * r
            flops += 2 * T * r * (wi + wo)
        if T <= 64:
            # the layer's dependency order: q,k,v read one x_s, gate,up
            # another; each group is one stage-1 launch, then (after the
            # shares' all-reduce of t_s) one stage-2 launch
            groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
            layer0 = use[0]
            s1 = [[dict(x=xs[SHAPES_13B[m][0] // P], Ut=layer0[m][0], t_io=ts[m]) for m in grp]
                  for grp in groups]
            s2 = [[dict(Vt=layer0[m][1], t_io=ts[m], y=ys[m]) for m in grp] for grp in groups]
            need = max(need, max(lr.lowrank_group_workspace_bytes(T, lin) for lin in s1 + s2))
        ws = torch.zeros(need + 256, dtype=torch.uint8, device=dev)

        def run():
            for layer in use:
                if T <= 64:
                    for grp in groups:
                        lr.lowrank_linear_forward_group(
                            [dict(x=xs[SHAPES_13B[m][0] // P], Ut=layer[m][0], t_io=ts[m])
                             for m in grp], workspace=ws)
                        lr.lowrank_linear_forward_group(
                            [dict(Vt=layer[m][1], t_io=ts[m], y=ys[m]) for m in grp],
                            workspace=ws)
                    continue
                for role in ROLES:
                    ut, vt, r = layer[role]
                    lr.lowrank_linear_forward(xs[SHAPES_13B[role][0] // P], ut, None,
                                              t_io=ts[role], flags=lr.LR_STAGE1_ONLY,
                                              workspace=ws)
                    lr.lowrank_linear_forward(None, None, vt, y=ys[role], t_io=ts[role],
                                              flags=lr.LR_STAGE2_ONLY, workspace=ws)
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ms_set = a.elapsed_time(b) / reps / len(use)
        del g
        s = ms_set * 1e-3
        out["T%d" % T] = {
            "tokens_per_s": round(T / s, 1), "us_per_layer_set": round(ms_set * 1e3, 2),
            "bytes_per_layer_set": nbytes, "GBps": round(nbytes / s / 1e9, 1),
            "hbm_frac": round(nbytes / s / HBM_PEAK, 4),
            "flop_per_layer_set": flops, "TFLOPs": round(flops / s / 1e12, 2),
            "mfma_frac": round(flops / s / BF16_PEAK, 4),
            "bound": "hbm" if T <= 64 else "mfma",
            "factor_layout": "packed" if T <= 64 else "rowmajor"}
    return out


def reference_kernel(torch, dev):
    """One elementwise kernel of known traffic for counter runs: negating 256 Mi
    bf16 reads 512 MiB and writes 512 MiB."""
    src = torch.empty(256 << 20, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def probe_step(torch, lr, dev):
    """Counter-run workload of the decode step: the reference kernel, then 2
    layers of the unfused and of the fused step (the decode-step inputs of the
    timed leg), eagerly, twice each."""
    from synth.decode_step import DecodeStepInputs
    reference_kernel(torch, dev)
    si = DecodeStepInputs(n_layers=2, device=dev)
    c = si.cfg
    prep = lr.lowrank_prepare_decode(si.lengths, si.tables, si.block, si.cap)
    rope = torch.empty((si.max_seq_rows, c["head_dim"] // 2, 2), dtype=torch.float32, device=dev)
    lr.lowrank_rope_table(c["head_dim"], si.max_seq_rows, 10000.0, rope)
    dp = {k: torch.from_numpy(np.ascontiguousarray(prep[k])).to(dev)
          for k in ("remap", "seq_off", "pos", "slot_mapping")}
    nv = torch.tensor([prep["n_valid"]], dtype=torch.int32, device=dev)
    layers = []
    for li in range(2):
        Ut, Vt, g1, g2 = si.device_layer(li)
        w = lr.layer_weights(c, Ut, Vt, g1, g2, rope, si.max_seq_rows)
        st = lr.decode_state(si.device_pool(li, 0), si.device_pool(li, 1), dp["slot_mapping"],
                             dp["remap"], dp["seq_off"], dp["pos"], nv, si.max_seq_rows)
        layers.append((w, st))
    for fused in (False, True):
        size = (lr.lowrank_decode_step_fused_workspace_bytes if fused
                else lr.lowrank_decode_step_workspace_bytes)
        fn = lr.lowrank_layer_decode_step_fused if fused else lr.lowrank_layer_decode_step
        ws = torch.zeros(size(*layers[0]), dtype=torch.uint8, device=dev)
        h = torch.from_numpy(si.h0.astype(np.float32)).to(dev)
        for _ in range(2):
            for w, st in layers:
                fn(w, st, h, ws)
        torch.cuda.synchronize()
        log("probe: %s decode step, 2 layers twice" % ("fused" if fused else "unfused"))
        del ws
        torch.cuda.empty_cache()


def decode_step(torch, lr, dev, stream, n_layers, reps, fused=False):
    """The 32-layer decode step of a LLaMA-7B-shaped decoder decomposed at
    ratio 0.2 (64 sequences, cached lengths uniform in [128, 4096]) captured
    once in a HIP graph and replayed; preparation stage timed separately.
    fused: lowrank_layer_decode_step_fused (K expanded per 256-row block
    inside the attention from the latents read in place, V applied after the
    softmax-weighted sum of its latents; no reconstructed K/V and no compact
    latent copy in memory)."""
    from synth.decode_step import DecodeStepInputs
    si = DecodeStepInputs(n_layers=n_layers, device=dev)
    c = si.cfg
    t0 = time.perf_counter()
    prep = lr.lowrank_prepare_decode(si.lengths, si.tables, si.block, si.cap)
    prep_ms = 1e3 * (time.perf_counter() - t0)
    rope = torch.empty((si.max_seq_rows, c["head_dim"] // 2, 2), dtype=torch.float32, device=dev)
    lr.lowrank_rope_table(c["head_dim"], si.max_seq_rows, 10000.0, rope)
    dp = {k: torch.from_numpy(np.ascontiguousarray(prep[k])).to(dev)
          for k in ("remap", "seq_off", "pos", "slot_mapping")}
    nv = torch.tensor([prep["n_valid"]], dtype=torch.int32, device=dev)
    layers = []
    for li in range(n_layers):
        Ut, Vt, g1, g2 = si.device_layer(li)
        w = lr.layer_weights(c, Ut, Vt, g1, g2, rope, si.max_seq_rows)
        st = lr.decode_state(si.device_pool(li, 0), si.device_pool(li, 1), dp["slot_mapping"],
                             dp["remap"], dp["seq_off"], dp["pos"], nv, si.max_seq_rows)
        layers.append((w, st))
    size = (lr.lowrank_decode_step_fused_workspace_bytes if fused
            else lr.lowrank_decode_step_workspace_bytes)
    layer_step = lr.lowrank_layer_decode_step_fused if fused else lr.lowrank_layer_decode_step
    ws = torch.zeros(size(*layers[0]), dtype=torch.uint8, device=dev)
    h0 = torch.from_numpy(si.h0.astype(np.float32)).to(dev)
    h = h0.clone()

    def step():
        h.copy_(h0)
        for w, st in layers:
            layer_step(w, st, h, ws)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    # per-kernel roofline budget of one layer (algorithmic bytes / flops)
    nvr, B = prep["n_valid"], c["B"]
    dkv = c["n_kv_heads"] * c["head_dim"]
    rk, rv = si.ranks["k"], si.ranks["v"]
    from synth.decode_step import dims
    lin_bytes = sum(2 * si.ranks[n] * (a_ + b_) + 2 * B * (a_ + b_)
                    for n, (a_, b_) in dims(c).items())
    # the fused step reads the latents in place through the remap list (no
    # compact copy); the unfused one copies them first (read + write)
    gather_bytes = 0 if fused else 2 * nvr * (rk + rv) * 2
    # unfused: K and V reconstructed; fused: K expanded on chip, V never formed
    # (the p-weighted sum of V latent rows per block and head, then V_v once
    # per sequence and head in the combine)
    H, hd = c["n_heads"], c["head_dim"]
    recon_flops = (2.0 * nvr * rk * dkv + 2.0 * nvr * rv * H + 2.0 * B * H * rv * hd
                   if fused else 2.0 * nvr * (rk + rv) * dkv)
    # fused: the latents read once (nothing reconstructed reaches HBM)
    recon_bytes = nvr * (rk + rv) * 2 + (0 if fused else 2 * nvr * dkv * 2)
    attn_bytes = 0 if fused else 2 * nvr * dkv * 2
    roof_s = (lin_bytes / HBM_PEAK + gather_bytes / HBM_PEAK
              + max(recon_flops / BF16_PEAK, recon_bytes / HBM_PEAK) + attn_bytes / HBM_PEAK)
    roof_ms = 1e3 * roof_s * n_layers
    del layers, ws, g
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(B / (ms * 1e-3), 1), "ms_per_step": round(ms, 3),
            "layers": n_layers, "sequences": B, "n_valid_rows": int(nvr),
            "roof_ms": round(roof_ms, 3), "frac": round(roof_ms / ms, 4),
            "prep_ms_host": round(prep_ms, 3),
            "per_layer_roof_us": {"linears": round(1e6 * lin_bytes / HBM_PEAK, 2),
                                  "gather": round(1e6 * gather_bytes / HBM_PEAK, 2),
                                  "recon": round(1e6 * max(recon_flops / BF16_PEAK,
                                                           recon_bytes / HBM_PEAK), 2),
                                  "attention": round(1e6 * attn_bytes / HBM_PEAK, 2)}}


def prefill_step(torch, lr, dev, stream, n_layers, reps, S=8, chunk=512):
    """The chunked-prefill step of the same 32-layer decoder (ratio 0.2):
    S new prompts of `chunk` tokens each (no cached rows) through every
    layer, one lowrank_layer_prefill_step call per layer; tokens/s and the
    MFMA roofline of the step's flops (projections, reconstruction, causal
    attention)."""
    from synth.decode_step import DecodeStepInputs, dims
    si = DecodeStepInputs(n_layers=n_layers, device=dev)
    c = si.cfg
    lengths = np.zeros(S, np.int64)
    chunks = np.full(S, chunk, np.int64)
    import synth
    tables, nblocks = synth.block_tables(synth.seed_of(5, 0, 2, synth.KIND_PLACE),
                                         chunks - 1, si.block, slack_blocks=4)
    pool_rows = nblocks * si.block
    max_rows = chunk
    cap = S * chunk
    prep = lr.lowrank_prepare_prefill(lengths, chunks, tables, si.block, cap)
    dp = {k: torch.from_numpy(np.ascontiguousarray(prep[k])).to(dev)
          for k in ("remap", "seq_off", "tok_seq", "pos", "slot_mapping")}
    nv = torch.tensor([prep["n_valid"]], dtype=torch.int32, device=dev)
    rope = torch.empty((max_rows, c["head_dim"] // 2, 2), dtype=torch.float32, device=dev)
    lr.lowrank_rope_table(c["head_dim"], max_rows, 10000.0, rope)
    layers = []
    for li in range(n_layers):
        Ut, Vt, g1, g2 = si.device_layer(li)
        w = lr.layer_weights(c, Ut, Vt, g1, g2, rope, max_rows)
        pk = torch.zeros((pool_rows, si.pool_ld), dtype=torch.bfloat16, device=dev)
        pv = torch.zeros_like(pk)
        st = lr.prefill_state(pk, pv, dp["slot_mapping"], dp["remap"], dp["seq_off"],
                              dp["tok_seq"], dp["pos"], nv, max_rows)
        layers.append((w, st))
    ws = torch.zeros(lr.lowrank_prefill_step_workspace_bytes(*layers[0]), dtype=torch.uint8,
                     device=dev)
    T = int(chunks.sum())
    g = torch.Generator(device=dev).manual_seed(4_000_001)
    h0 = torch.randn((T, c["d_model"]), generator=g, device=dev)
    h = h0.clone()

    def step():
        h.copy_(h0)
        for w, st in layers:
            lr.lowrank_layer_prefill_step(w, st, h, ws, stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    dkv = c["n_kv_heads"] * c["head_dim"]
    lin_fl = sum(2.0 * T * si.ranks[n] * (a_ + b_) for n, (a_, b_) in dims(c).items())
    rec_fl = 2.0 * T * (si.ranks["k"] + si.ranks["v"]) * dkv
    att_fl = 4.0 * c["n_heads"] * c["head_dim"] * S * chunk * (chunk + 1) / 2
    per_layer = lin_fl + rec_fl + att_fl
    roof_ms = 1e3 * n_layers * per_layer / BF16_PEAK
    del layers, ws
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 3),
            "layers": n_layers, "sequences": S, "chunk": chunk,
            "roof_ms": round(roof_ms, 3), "frac": round(roof_ms / ms, 4),
            "per_layer_gflop": {"linears": round(lin_fl / 1e9, 2),
                                "recon": round(rec_fl / 1e9, 2),
                                "attention": round(att_fl / 1e9, 2)}}


def cpu_baseline(base, seconds):
    """fp64 oracle on the host: the seven projections of layer set 0 at each
    decode T, repeated until about `seconds` of CPU time; tokens x layer sets
    per second, as the GPU value."""
    import oracle
    import synth
    threads, vendor = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count()), "unknown"
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            threads = max(i.get("num_threads", 1) for i in blas)
            vendor = ",".join(sorted({str(i.get("internal_api", "?")) for i in blas}))
    except Exception:
        pass
    xs = {T: {d: synth.tokens(synth.seed_of(2, 0, 0, synth.KIND_X) + T, T, d)
              for d in (4096, 11008)} for T in TOKENS}
    tokens, passes = 0, 0
    t0 = time.perf_counter()
    while True:
        for T in TOKENS:
            for role in ROLES:
                _, _, r, U, V = base[role]
                oracle.linear(xs[T][SHAPES[role][0]], U, V)
            tokens += T
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(tokens / el, 2), "unit": "tokens/s (x 7-projection layer set)",
            "cores": int(threads), "host_cpu_count": os.cpu_count(), "blas_vendor": vendor,
            "blas_threads": int(threads), "kind": "oracle",
            "sample": "%d passes of layer set 0 (7 projections) at T=1,8,32,64, fp64 numpy, "
                      "%.1f s" % (passes, el)}


if __name__ == "__main__":
    main()
