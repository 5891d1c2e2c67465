#!/usr/bin/env python3
"""Benchmark of the IKBO hot path on one MI355X.

Default workload ("block"): the full ROCS block at production-like scale, bf16 --
R = 128 requests x 2048 candidates; a 2-layer GLM-masked MLP over [request 4096 | candidate 2048]
features (hidden 2048 per group, GELU; output 4096 per group = 4 query tokens x 8 heads x 128)
feeds IKBO-DCA over a shared request history of L = 8192 keys (H = 8, d = 128). One step = one
ikbo_glm_mlp_forward (two IKBO-LCB layers) + one ikbo_dca_forward on the same stream, inputs
resident in HBM. Other workloads (--workload dca_fixed | dca_ragged | lcb) time a single operator.

Prints ONE JSON line: throughput in effective TFLOP/s (no broadcast counted), ms per step, the
roofline of the dominant kernel from HIP events on its stream, and the fp64 CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "IKBO-DCA TFLOP/s + ms; IKBO-LCB ms; % of MI355X bf16 MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
FM_SHAPE = (128, 2048, 32, 32, 64)   # requests, candidates per request, n_r, n_c, d
# timed after the block workload in the default run: fixed-length DCA, ragged DCA, and IKBO-LCB
EXTRA_WORKLOADS = ("dca_fixed", "dca_ragged", "lcb")
# requests, candidates per request, n_r, n_c (input embeddings), d, k_r, k_c (output embeddings)
LCBE_SHAPE = (128, 2048, 32, 32, 64, 32, 32)

# The kernel figures the pages print, as context beside the measured line (not a target: their
# hardware, precision and shapes differ and are not all stated). ROCS: Request-Oriented Compute
# Sharing, Sec. 5.2.5 (Tables 4 and 5); Request-Level Sharing Cuts Recommendation Inference Cost,
# "Technical Approach".
PAGES_CONTEXT = {
    "hardware": "Hopper-class GPU (the kernels use WGMMA and TMA; the tables name no GPU)",
    "shapes_and_precision": "not stated for these tables",
    "ikbo_lcb_ms": {"original": 1.944, "after_decomposition": 1.389, "after_alignment": 0.798,
                    "after_broadcast_fusion": 0.580, "after_pipelining_and_fusion": 0.482},
    "ikbo_dca": {"tflops": 594, "ms": 0.230, "gbs": 681},
    "fa_baselines_with_explicit_broadcast": {"tlx_fa3_tflops": 245, "tlx_fa3_ms": 1.473,
                                              "cutedsl_fa_tflops": 250, "cutedsl_fa_ms": 1.462},
}


def stack_layer2(np, synth, s):
    """The second interaction layer of the stack workload: its query generator reads the first
    layer's [Q | A] rows (2 W = 8192 wide per group): [8192 | 8192] -> 2048 (GELU) -> 4096, weights
    N(0, 1/fan-in), biases N(0, 1/fan-in); its own sequence rows S_2 (N(0, 1)) and K/V weights
    N(0, 1/1024)."""
    W = s.Lq * s.H * s.d
    hd, rows = s.H * s.d, s.kv_rows
    layers = []
    for i, (kr, kc, n, act) in enumerate(((2 * W, 2 * W, 2048, "gelu"), (2048, 2048, W, "none"))):
        t = 200 + 8 * i
        layers.append(dict(w_rr=synth.draw(7, t, n * kr, "bf16", 1 / np.sqrt(kr)).reshape(n, kr),
                           w_cr=synth.draw(7, t + 1, n * kr, "bf16", 1 / np.sqrt(kr)).reshape(n, kr),
                           w_cc=synth.draw(7, t + 2, n * kc, "bf16", 1 / np.sqrt(kc)).reshape(n, kc),
                           b_r=synth.draw(7, t + 3, n, "f32", 1 / np.sqrt(kr)),
                           b_c=synth.draw(7, t + 4, n, "f32", 1 / np.sqrt(kc)), act=act))
    seq = lambda start=0, count=rows: synth.draw(7, 220, count * hd, "bf16", 1.0, start=start * hd).reshape(count, hd)
    kv = [synth.draw(7, 221 + i, hd * hd, "bf16", 1 / np.sqrt(hd)).reshape(hd, hd) for i in range(4)]
    return layers, seq, kv


def mlp_flops(C, R, layers):
    """2 C sum k_c n_c + 2 R sum k_r (n_r + n_c) over GLM layers given as (k_r, k_c, n_r, n_c)."""
    return sum(2.0 * C * kc * nc + 2.0 * R * kr * (nr + nc) for kr, kc, nr, nc in layers)


def lcbe_params(np, synth):
    """Weights N(0, 1/n_in) and per-group gamma, beta of the LCB embedding-form workload."""
    import math
    R, per_r, n_r, n_c, d, k_r, k_c = LCBE_SHAPE
    return dict(w_rr=synth.draw(0, 92, k_r * n_r, "bf16", 1 / math.sqrt(n_r)).reshape(k_r, n_r),
                w_cr=synth.draw(0, 93, k_c * n_r, "bf16", 1 / math.sqrt(n_r)).reshape(k_c, n_r),
                w_cc=synth.draw(0, 94, k_c * n_c, "bf16", 1 / math.sqrt(n_c)).reshape(k_c, n_c),
                gamma_r=(1.0 + 0.25 * synth.draw(0, 95, d, "f32")).astype(np.float32),
                beta_r=(0.25 * synth.draw(0, 96, d, "f32")).astype(np.float32),
                gamma_c=(1.0 + 0.25 * synth.draw(0, 97, d, "f32")).astype(np.float32),
                beta_c=(0.25 * synth.draw(0, 98, d, "f32")).astype(np.float32))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="block", choices=["block", "layer", "dca_fixed", "dca_ragged", "lcb", "fm", "lcb_emb",
                                                           "stack"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="with the block workload, skip timing the single-operator workloads after it")
    p.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA / HBM / exp2 ceilings")
    p.add_argument("--flush-mib", type=int, default=512,
                   help="cold-cache pass after the timed steps: this many MiB written between steps, outside "
                        "their events, so no input stays in L2 or the 256 MiB MALL (0 = skip the pass)")
    p.add_argument("--cpu-sample", type=int, default=0, help="candidates in the oracle sample (0 = default)")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="per-kernel HBM bytes measured with rocprofv3 counters, if present")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (for scaling the HBM byte counters)")
    return p.parse_args()


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, three launches."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 3}))


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import request_candidate_broadcast_amd as ikbo
    import synth

    if not os.path.exists(ikbo.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    ikbo.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()   # default priority

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        if a.dtype == np.int32 or a.dtype == np.int64:
            return torch.from_numpy(a.astype(np.int32)).to(dev)
        return torch.from_numpy(a.astype(np.float32)).to(dev)

    t_gen = time.time()
    with torch.cuda.stream(stream):
        W = setup(args.workload, args, np, torch, ikbo, synth, dev, stream, up)
    step, names, dominant, config = W["step"], W["names"], W["dominant"], W["config"]
    flops, algo_bytes = W["flops"], W["algo_bytes"]
    torch.cuda.synchronize()
    log("inputs ready in %.1f s (%s)" % (time.time() - t_gen, args.workload))

    nev = max(e for _, _, e in names) + 1
    timed, ms_step = run_steps(step, nev, args.steps, args.warmup, torch)
    log("timed %d steps: %.3f ms/step" % (args.steps, ms_step))

    # cold-cache pass: the same steps, each after a write of flush-mib MiB on the same stream that
    # evicts the previous step's data from L2 and the MALL (outside the events, not in ms_per_step)
    cold = None
    if args.flush_mib > 0:
        fbuf = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                fbuf.fill_(i & 0xff)
                step(cev[i])
        torch.cuda.synchronize()
        del fbuf
        cold = {"flush_mib": args.flush_mib}
        for name, a, b in names:
            d = [cev[i][a].elapsed_time(cev[i][b]) for i in range(args.steps)]
            cold[name] = {"ms_median": float(np.median(d)), "ms_min": float(np.min(d)),
                          "ms_p90": float(np.percentile(d, 90))}
        log("cold-cache pass done")

    per = part_stats(timed, names, flops, algo_bytes, np)
    total_flops = sum(flops.values())
    value = total_flops / (ms_step * 1e-3) / 1e12
    # roofline of the dominant kernel (its own events on its stream)
    roofline = roofline_of(args.workload, dominant, per, flops, algo_bytes, traffic_for(args, args.workload, dominant))
    if args.workload == "stack":
        roofline["kernel"] = "layer2: one ikbo_dca_layer_forward call (11 launches; its DCA alone is the block workload's)"

    # IKBO-LCB also has a persistent request/candidate launch (IKBO_LCB_FUSED=1, same bits); time it
    # after the timed region, on the same inputs, for comparison
    alt = None
    if args.workload == "lcb":
        os.environ["IKBO_LCB_FUSED"] = "1"
        try:
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps + 1)]
            for i in range(args.steps + 1):
                step(ev[i])
            torch.cuda.synchronize()
            d = [ev[i][0].elapsed_time(ev[i][1]) for i in range(1, args.steps + 1)]
            alt = {"lcb_persistent_launch_ms_avg": round(float(np.mean(d)), 4),
                   "lcb_two_launches_ms_avg": round(per["lcb"]["ms_avg"], 4)}
            log("persistent LCB launch: %.3f ms" % alt["lcb_persistent_launch_ms_avg"])
        finally:
            os.environ.pop("IKBO_LCB_FUSED", None)

    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(torch, ikbo, stream)
        log("ceilings: %s" % ceilings)
        add_exp_rate(per, flops, config, ceilings)
        roofline["measured_peak"] = (ceilings["mfma_bf16_tflops"] if roofline["bound"] == "mfma"
                                     else ceilings["hbm_copy_gbs"])
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, np)

    # The default run also times the other workloads the metric names, each on its own inputs
    # (the headline's are freed first): IKBO-DCA with a fixed K/V length, IKBO-DCA ragged, and
    # IKBO-LCB on its own, each with its roofline.
    extra = {}
    if args.workload == "block" and not args.no_extra:
        del W, step
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        for wl in EXTRA_WORKLOADS:
            t_gen = time.time()
            with torch.cuda.stream(stream):
                X = setup(wl, args, np, torch, ikbo, synth, dev, stream, up)
            torch.cuda.synchronize()
            log("inputs ready in %.1f s (%s)" % (time.time() - t_gen, wl))
            xnev = max(e for _, _, e in X["names"]) + 1
            xt, xms = run_steps(X["step"], xnev, args.steps, args.warmup, torch)
            xper = part_stats(xt, X["names"], X["flops"], X["algo_bytes"], np)
            if ceilings:
                add_exp_rate(xper, X["flops"], X["config"], ceilings)
            xroof = roofline_of(wl, X["dominant"], xper, X["flops"], X["algo_bytes"], traffic_for(args, wl, X["dominant"]))
            if ceilings:
                xroof["measured_peak"] = ceilings["mfma_bf16_tflops"]
            extra[wl] = {"config": X["config"], "ms_per_step": round(xms, 4),
                         "parts": {k: {kk: round(vv, 4) for kk, vv in d.items()} for k, d in xper.items()},
                         "roofline": xroof}
            log("%s: %.4f ms/step, %.1f TFLOP/s" % (wl, xms, xroof["achieved"]))
            del X
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded SplitMix64 normals)",
        "config": config,
        "parts": {k: {kk: round(vv, 4) for kk, vv in d.items()} for k, d in per.items()},
        "roofline": roofline, "cpu_baseline": cpu, "ceilings": ceilings,
    }
    if extra:
        line["workloads"] = extra
        if "lcb" in extra:
            line["ikbo_lcb_ms"] = extra["lcb"]["parts"]["lcb"]["ms_avg"]
    if alt:
        line["alternate_forms"] = alt
    line["pages_context"] = PAGES_CONTEXT
    if cold:
        line["cold_l2"] = {k: ({kk: round(vv, 4) for kk, vv in d.items()} if isinstance(d, dict) else d)
                           for k, d in cold.items()}
    print(json.dumps(line), flush=True)


def run_steps(step, nev, steps, warmup, torch):
    """warmup untimed steps, then `steps` back to back between two synchronisations; returns the
    per-step events and the wall-clock ms per step."""
    warm = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(max(warmup, 0))]
    timed = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    for i in range(warmup):
        step(warm[i])
        torch.cuda.synchronize()
        log("warmup step %d done" % i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(timed[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return timed, (t1 - t0) * 1e3 / steps


def part_stats(timed, names, flops, algo_bytes, np):
    per = {}
    for name, a, b in names:
        d = [ev[a].elapsed_time(ev[b]) for ev in timed]
        per[name] = {"ms_avg": float(np.mean(d)), "ms_min": float(np.min(d)), "ms_median": float(np.median(d)),
                     "ms_p90": float(np.percentile(d, 90))}
        per[name]["tflops"] = flops[name] / (per[name]["ms_avg"] * 1e-3) / 1e12
        per[name]["gbs_algorithmic"] = algo_bytes[name] / (per[name]["ms_avg"] * 1e-3) / 1e9
        per[name]["mfma_frac"] = per[name]["tflops"] / PEAK_BF16_TFLOPS
    return per


def add_exp_rate(per, flops, config, ceilings):
    """DCA parts: one exp2 per score (the fixed-reference softmax), FLOPs = 4 d per score."""
    if "dca" in per:
        d_head = config.get("head_dim", 128)
        exps = flops["dca"] / (4.0 * d_head)
        per["dca"]["exps_per_s"] = exps / (per["dca"]["ms_avg"] * 1e-3)
        per["dca"]["exp_frac_of_measured"] = per["dca"]["exps_per_s"] / ceilings["exp2_per_s"]


def traffic_for(args, workload, dominant):
    """HBM bytes per launch from rocprofv3 counters (scaled by a plain copy), valid only while the
    kernel sources hash to the value recorded with them; else None."""
    import hashlib
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f)
        ent = tj.get(workload, {}).get(dominant)
        if not ent:
            return None
        h = hashlib.sha256()            # the kernel's sources, hashed together in the listed order
        for name in ent["files"]:
            with open(os.path.join(ROOT, name), "rb") as f:
                h.update(f.read())
        return ent.get("bytes_per_launch") if h.hexdigest()[:16] == ent.get("source_sha256_prefix") else None
    except (OSError, ValueError, KeyError):
        return None


def roofline_of(workload, dominant, per, flops, algo_bytes, traffic):
    dk = per[dominant]
    if dominant in ("fm", "lcb_emb"):      # HBM-bound (16-32 FLOP per byte at bf16 in and out)
        gbs = dk["gbs_algorithmic"]
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": dominant,
                "bytes_per_launch": algo_bytes[dominant], "ms_per_launch": round(dk["ms_avg"], 4)}
    return {"bound": "mfma", "achieved": round(dk["tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(dk["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": dominant,
            "flops_per_launch": flops[dominant], "ms_per_launch": round(dk["ms_avg"], 4)}


def setup(workload, args, np, torch, ikbo, synth, dev, stream, up):
    """Inputs of one workload resident in HBM, and one step of it: a callable that records HIP events
    on `stream` around each part. Returns the step, its parts [(name, first event, last event)], the
    dominant part, the config, and the effective FLOPs and algorithmic bytes per part."""
    flops = {}
    algo_bytes = {}
    if workload in ("block", "layer"):
        g, s = synth.block_specs()
        x_r = up(synth.glm_x(g, "x_r"))
        x_c = up(synth.glm_x(g, "x_c"))
        layers = []
        for li in range(len(g.layers)):
            w = synth.glm_weights(g, li)
            layers.append({"w_rr": up(w["w_rr"]), "w_cr": up(w["w_cr"]), "w_cc": up(w["w_cc"]),
                           "b_r": up(w["b_r"]), "b_c": up(w["b_c"]), "act": g.layers[li].act})
        k = up(synth.dca_kv(s, "k")).view(s.R, s.L, s.H, s.d)
        v = up(synth.dca_kv(s, "v")).view(s.R, s.L, s.H, s.d)
        off = up(s.offsets)
        m = up(s.cand_to_req)
        last = g.layers[-1]
        y_req = torch.empty((g.R, last.n_req), dtype=torch.bfloat16, device=dev)
        y_cand = torch.empty((g.C, last.n_cand), dtype=torch.bfloat16, device=dev)
        q = y_cand.view(s.C, s.Lq, s.H, s.d)
        out = torch.empty((s.C, s.Lq, s.H, s.d), dtype=torch.bfloat16, device=dev)
        ws_mlp = torch.empty(ikbo.ikbo_glm_mlp_workspace_size(g.C, g.R, layers, torch.bfloat16),
                             dtype=torch.uint8, device=dev)
        ws_dca = torch.empty(max(1, ikbo.ikbo_dca_workspace_size(s.C, s.R)), dtype=torch.uint8, device=dev)
        flops["mlp"] = g.flops()
        flops["dca"] = s.flops()
        algo_bytes["dca"] = 2 * (s.C * s.Lq * s.H * s.d) * 2 + 2 * (s.R * s.L * s.H * s.d) * 2 + 4 * s.C
        ly0, ly1 = g.layers
        algo_bytes["mlp"] = 2 * (g.C * (ly0.k_cand + ly0.n_cand + ly1.n_cand + ly1.n_cand)
                                 + g.R * (ly0.k_req + ly0.n_req + ly1.n_req))

        def step(ev):
            ev[0].record(stream)
            ikbo.ikbo_glm_mlp_forward(x_r, x_c, layers, cand_to_req=m, sorted_index=True, y_req=y_req,
                                      y_cand=y_cand, workspace=ws_mlp, stream=stream)
            ev[1].record(stream)
            ikbo.ikbo_dca_forward(q, k, v, req_cand_offsets=off, out=out, workspace=ws_dca, stream=stream)
            ev[2].record(stream)

        names = [("mlp", 0, 1), ("dca", 1, 2)]
        dominant = "dca"
        config = {"workload": "full ROCS block: GLM-MLP (2 IKBO-LCB layers) -> IKBO-DCA",
                  "requests": s.R, "candidates": s.C, "cand_per_request": int(s.counts[0]),
                  "mlp": "[4096|2048] -> 2048 (GELU) -> 4096", "kv_len": s.L, "heads": s.H, "head_dim": s.d,
                  "q_tokens": s.Lq}
        if workload == "layer":
            # the whole DCA layer: K/V of both halves projected from the request sequence rows
            # S once per request, A^C = IKBO-DCA(q_c, K^C, V^C), A^R = Attn(q_r, K^R, V^R)
            del k, v
            seq = up(synth.seq_rows(s))
            wk = {n: up(synth.kv_weight(s, n)) for n in ("w_kc", "w_vc", "w_kr", "w_vr")}
            hd, rows = s.H * s.d, s.kv_rows
            kc = torch.empty((rows, hd), dtype=torch.bfloat16, device=dev)
            vc, kr, vr = torch.empty_like(kc), torch.empty_like(kc), torch.empty_like(kc)
            q_r = y_req.view(s.R, s.Lq, s.H, s.d)
            out_r = torch.empty((s.R, s.Lq, s.H, s.d), dtype=torch.bfloat16, device=dev)
            ws_ra = torch.empty(ikbo.ikbo_request_attention_workspace_size(s.R), dtype=torch.uint8, device=dev)
            d_in = synth.seq_width(s)
            flops["kv_proj_c"] = flops["kv_proj_r"] = 2 * 2.0 * rows * d_in * hd
            flops["attn_r"] = 4.0 * s.R * s.Lq * s.H * s.d * s.L
            algo_bytes["kv_proj_c"] = algo_bytes["kv_proj_r"] = 2 * (rows * d_in + 2 * rows * hd + 2 * hd * d_in)
            algo_bytes["attn_r"] = 2 * (2 * s.R * s.Lq * hd + 2 * rows * hd)

            def step(ev):
                ev[0].record(stream)
                ikbo.ikbo_glm_mlp_forward(x_r, x_c, layers, cand_to_req=m, sorted_index=True, y_req=y_req,
                                          y_cand=y_cand, workspace=ws_mlp, stream=stream)
                ev[1].record(stream)
                ikbo.ikbo_kv_project(seq, wk["w_kc"], wk["w_vc"], k_out=kc, v_out=vc, stream=stream)
                ev[2].record(stream)
                ikbo.ikbo_dca_forward(q, kc.view(s.R, s.L, s.H, s.d), vc.view(s.R, s.L, s.H, s.d),
                                      req_cand_offsets=off, out=out, workspace=ws_dca, stream=stream)
                ev[3].record(stream)
                ikbo.ikbo_kv_project(seq, wk["w_kr"], wk["w_vr"], k_out=kr, v_out=vr, stream=stream)
                ev[4].record(stream)
                ikbo.ikbo_request_attention(q_r, kr.view(s.R, s.L, s.H, s.d), vr.view(s.R, s.L, s.H, s.d),
                                            out=out_r, workspace=ws_ra, stream=stream)
                ev[5].record(stream)

            names = [("mlp", 0, 1), ("kv_proj_c", 1, 2), ("dca", 2, 3), ("kv_proj_r", 3, 4), ("attn_r", 4, 5)]
            config = dict(config, workload="ROCS DCA layer: GLM-MLP -> K/V projections of S (once per request) "
                          "-> A^C (IKBO-DCA) + A^R (request-side attention)", seq_width=d_in)
    elif workload == "fm":
        # GLM factorization machine (Eq. 10) on the block's batch: 128 requests x 2048 candidates,
        # 32 request and 32 candidate features of width 64, N(0,1), bf16 in and out
        R, per_r, n_r, n_c, d = FM_SHAPE
        C = R * per_r
        fm_counts = np.full(R, per_r)
        x_r = up(synth.draw(0, 80, R * n_r * d, "bf16").reshape(R, n_r, d))
        x_c = up(synth.draw(0, 81, C * n_c * d, "bf16").reshape(C, n_c, d))
        off = up(synth.offsets_from_counts(fm_counts))
        y_r = torch.empty((R, n_r, n_r), dtype=torch.bfloat16, device=dev)
        y_c = torch.empty((C, n_c, n_r + n_c), dtype=torch.bfloat16, device=dev)
        flops["fm"] = 2.0 * C * n_c * (n_r + n_c) * d + 2.0 * R * n_r * n_r * d
        algo_bytes["fm"] = 2 * (C * n_c * d + C * n_c * (n_r + n_c) + R * n_r * d + R * n_r * n_r) + 4 * (R + 1)

        def step(ev):
            ev[0].record(stream)
            ikbo.ikbo_fm_forward(x_r, x_c, req_cand_offsets=off, y_req=y_r, y_cand=y_c, stream=stream)
            ev[1].record(stream)

        names = [("fm", 0, 1)]
        dominant = "fm"
        config = {"workload": "GLM factorization machine (two groups, in-kernel broadcast)", "requests": R,
                  "candidates": C, "n_req_feat": n_r, "n_cand_feat": n_c, "dim": d}
    elif workload == "stack":
        # two DCA interaction layers (Eq. 12-13 and the [Q | A] rows that feed the next), one
        # ikbo_dca_layer_forward call each: the block's layer, then a layer reading its output
        g, s = synth.block_specs()
        W, hd, rows = s.Lq * s.H * s.d, s.H * s.d, s.kv_rows
        x_r = up(synth.glm_x(g, "x_r"))
        x_c = up(synth.glm_x(g, "x_c"))
        l1 = []
        for li in range(len(g.layers)):
            w = synth.glm_weights(g, li)
            l1.append({"w_rr": up(w["w_rr"]), "w_cr": up(w["w_cr"]), "w_cc": up(w["w_cc"]),
                       "b_r": up(w["b_r"]), "b_c": up(w["b_c"]), "act": g.layers[li].act})
        s1 = up(synth.seq_rows(s))
        kv1 = [up(synth.kv_weight(s, n)) for n in ("w_kc", "w_vc", "w_kr", "w_vr")]
        l2h, seq2, kv2h = stack_layer2(np, synth, s)
        l2 = [{kk: (up(vv) if isinstance(vv, np.ndarray) else vv) for kk, vv in ly.items()} for ly in l2h]
        s2 = up(seq2())
        kv2 = [up(w) for w in kv2h]
        off = up(s.offsets)
        y1_r = torch.empty((s.R, 2 * W), dtype=torch.bfloat16, device=dev)
        y1_c = torch.empty((s.C, 2 * W), dtype=torch.bfloat16, device=dev)
        y2_r, y2_c = torch.empty_like(y1_r), torch.empty_like(y1_c)
        nbytes = max(ikbo.load_library().ikbo_dca_layer_workspace_size(s.C, s.R, len(ls), ikbo._layer_structs(ls),
                                                                       rows, s.H, s.d, ikbo.IKBO_BF16)
                     for ls in (l1, l2))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        attn = 2 * 2 * 2.0 * rows * hd * hd + s.flops() + 4.0 * s.R * s.Lq * s.H * s.d * s.L
        ly0, ly1 = g.layers
        flops["layer1"] = mlp_flops(s.C, s.R, [(ly0.k_req, ly0.k_cand, ly0.n_req, ly0.n_cand),
                                                (ly1.k_req, ly1.k_cand, ly1.n_req, ly1.n_cand)]) + attn
        flops["layer2"] = mlp_flops(s.C, s.R, [(2 * W, 2 * W, 2048, 2048), (2048, 2048, W, W)]) + attn
        algo_bytes["layer1"] = algo_bytes["layer2"] = 0
        kw = dict(q_len=s.Lq, num_heads=s.H, head_dim=s.d, req_cand_offsets=off, workspace=ws, stream=stream)

        def step(ev):
            ev[0].record(stream)
            ikbo.ikbo_dca_layer_forward(x_r, x_c, l1, s1, *kv1, y_req=y1_r, y_cand=y1_c, **kw)
            ev[1].record(stream)
            ikbo.ikbo_dca_layer_forward(y1_r, y1_c, l2, s2, *kv2, y_req=y2_r, y_cand=y2_c, **kw)
            ev[2].record(stream)

        names = [("layer1", 0, 1), ("layer2", 1, 2)]
        dominant = "layer2"
        config = {"workload": "ROCS interaction stack: 2 DCA layers (GLM-MLP -> K/V of S -> A^C + A^R, "
                  "[Q | A] to the next layer), one call per layer", "requests": s.R, "candidates": s.C,
                  "mlp_layer1": "[4096|2048] -> 2048 (GELU) -> 4096", "mlp_layer2": "[8192|8192] -> 2048 (GELU) -> 4096",
                  "kv_len": s.L, "heads": s.H, "head_dim": s.d, "q_tokens": s.Lq, "seq_width": hd}
    elif workload == "lcb_emb":
        # LCB embedding form (Eq. 5-6) with a per-group LayerNorm (Eq. 7) on the block's batch:
        # 128 requests x 2048 candidates, 32 -> 32 embeddings of width 64 per group, bf16 in and out
        R, per_r, n_r, n_c, d, k_r, k_c = LCBE_SHAPE
        C = R * per_r
        x_r = up(synth.draw(0, 90, R * n_r * d, "bf16").reshape(R, n_r, d))
        x_c = up(synth.draw(0, 91, C * n_c * d, "bf16").reshape(C, n_c, d))
        prm = {kk: up(vv) for kk, vv in lcbe_params(np, synth).items()}
        off = up(synth.offsets_from_counts(np.full(R, per_r)))
        y_r = torch.empty((R, k_r, d), dtype=torch.bfloat16, device=dev)
        y_c = torch.empty((C, k_c, d), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(ikbo.ikbo_lcb_emb_workspace_size(R, k_c, d), dtype=torch.uint8, device=dev)
        flops["lcb_emb"] = 2.0 * C * k_c * n_c * d + 2.0 * R * (k_r + k_c) * n_r * d
        algo_bytes["lcb_emb"] = 2 * (C * n_c * d + C * k_c * d + R * n_r * d + R * k_r * d
                                     + (k_r + k_c) * n_r + k_c * n_c) + 4 * (R + 1) + 4 * 4 * d

        def step(ev):
            ev[0].record(stream)
            ikbo.ikbo_lcb_emb_forward(x_r, x_c, prm["w_rr"], prm["w_cr"], prm["w_cc"], req_cand_offsets=off,
                                      norm="layer", gamma_req=prm["gamma_r"], beta_req=prm["beta_r"],
                                      gamma_cand=prm["gamma_c"], beta_cand=prm["beta_c"], y_req=y_r, y_cand=y_c,
                                      workspace=ws, stream=stream)
            ev[1].record(stream)

        names = [("lcb_emb", 0, 1)]
        dominant = "lcb_emb"
        config = {"workload": "LCB embedding form + group-local LayerNorm (two groups, in-kernel broadcast)",
                  "requests": R, "candidates": C, "n_req_in": n_r, "n_cand_in": n_c, "dim": d,
                  "n_req_out": k_r, "n_cand_out": k_c, "norm": "layer"}
    elif workload in ("dca_fixed", "dca_ragged"):
        s = synth.dca_spec(workload)
        q = up(synth.dca_q(s))
        k, v = up(synth.dca_kv(s, "k")), up(synth.dca_kv(s, "v"))
        kw = {}
        if s.varlen:
            kw["kv_cu_seqlens"] = up(s.kv_cu)
        else:
            k = k.view(s.R, s.L, s.H, s.d)
            v = v.view(s.R, s.L, s.H, s.d)
        off = up(s.offsets)
        out = torch.empty((s.C, s.Lq, s.H, s.d), dtype=torch.bfloat16, device=dev)
        ws_dca = torch.empty(max(1, ikbo.ikbo_dca_workspace_size(s.C, s.R)), dtype=torch.uint8, device=dev)
        flops["dca"] = s.flops()
        algo_bytes["dca"] = 2 * (s.C * s.Lq * s.H * s.d) * 2 + 2 * (s.kv_rows * s.H * s.d) * 2 + 4 * s.C

        def step(ev):
            ev[0].record(stream)
            ikbo.ikbo_dca_forward(q, k, v, num_req=s.R, req_cand_offsets=off, out=out, workspace=ws_dca,
                                  stream=stream, **kw)
            ev[1].record(stream)

        names = [("dca", 0, 1)]
        dominant = "dca"
        config = {"workload": "IKBO-DCA " + workload, "requests": s.R, "candidates": s.C,
                  "kv_len": "varlen" if s.varlen else s.L, "heads": s.H, "head_dim": s.d, "q_tokens": s.Lq}
    else:
        g = synth.glm_spec("lcb")
        x_r = up(synth.glm_x(g, "x_r"))
        x_c = up(synth.glm_x(g, "x_c"))
        w = synth.glm_weights(g, 0)
        wd = {kk: up(vv) for kk, vv in w.items()}
        m = up(g.cand_to_req)
        ly = g.layers[0]
        y_req = torch.empty((g.R, ly.n_req), dtype=torch.bfloat16, device=dev)
        y_cand = torch.empty((g.C, ly.n_cand), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(ikbo.ikbo_lcb_workspace_size(g.C, g.R, ly.k_req, ly.k_cand, ly.n_req, ly.n_cand),
                         dtype=torch.uint8, device=dev)
        flops["lcb"] = g.flops()
        algo_bytes["lcb"] = 2 * (g.C * (ly.k_cand + ly.n_cand) + g.R * (ly.k_req + ly.n_req)
                                 + (ly.n_req + ly.n_cand) * ly.k_req + ly.n_cand * ly.k_cand) + 4 * g.C

        def step(ev):
            ev[0].record(stream)
            ikbo.ikbo_lcb_forward(x_r, x_c, wd["w_rr"], wd["w_cr"], wd["w_cc"], b_r=wd["b_r"], b_c=wd["b_c"],
                                  cand_to_req=m, sorted_index=True, activation="gelu", y_req=y_req, y_cand=y_cand,
                                  workspace=ws, stream=stream)
            ev[1].record(stream)

        names = [("lcb", 0, 1)]
        dominant = "lcb"
        config = {"workload": "IKBO-LCB broadcast-fused GLM linear", "requests": g.R, "candidates": g.C,
                  "k_req": ly.k_req, "k_cand": ly.k_cand, "n_out": ly.n_cand, "activation": "gelu"}
    return dict(step=step, names=names, dominant=dominant, config=config, flops=flops, algo_bytes=algo_bytes)


def measure_ceilings(torch, ikbo, stream):
    """What kernels of this part reach on their own (libikbo_probe.so), beside the published peaks:
    dense bf16 MFMA from register operands, HBM copy and read streams, v_exp_f32 evaluations, LDS
    reads (ds_read_b128, and ds_read_b64_tr_b16 over 320-byte rows, the transposed V^T reads of the
    d = 128 attention kernel). Median of 5 timed launches after one warm-up each."""
    dev = torch.device("cuda:0")

    def timed(kind, buf, iters, blocks):
        ikbo.ikbo_probe_launch(kind, buf, iters, blocks, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for i in range(5):
            ev[i].record(stream)
            ikbo.ikbo_probe_launch(kind, buf, iters, blocks, stream)
        ev[5].record(stream)
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(5))[2] * 1e-3

    out = {}
    small = torch.empty(4096 * 1024, dtype=torch.uint8, device=dev)
    best = 0.0
    for blocks in (512, 1024):                 # 2 and 4 waves per SIMD
        iters = 20000
        sec = timed(ikbo.IKBO_PROBE_MFMA_BF16, small, iters, blocks)
        best = max(best, blocks * 4 * iters * 4 * 32768.0 / sec / 1e12)
    out["mfma_bf16_tflops"] = round(best, 1)
    # the same four chains with one wave per SIMD (256 blocks of 4 waves): what one wave can issue
    sec = timed(ikbo.IKBO_PROBE_MFMA_BF16, small, 20000, 256)
    out["mfma_bf16_tflops_one_wave_per_simd"] = round(256 * 4 * 20000 * 4 * 32768.0 / sec / 1e12, 1)
    iters, blocks = 8000, 2048
    sec = timed(ikbo.IKBO_PROBE_EXP2, small, iters, blocks)
    out["exp2_per_s"] = float("%.4g" % (blocks * 256 * iters * 8 / sec))
    iters, blocks = 2000, 1024                 # four blocks of 4 waves and 32 KiB of LDS per CU
    for kind, key, per in ((ikbo.IKBO_PROBE_LDS_B128, "lds_read_b128_tbs", 1024),
                           (ikbo.IKBO_PROBE_LDS_TR16, "lds_read_tr16_tbs", 512)):
        out[key] = round(blocks * 4 * iters * 16 * per / timed(kind, small, iters, blocks) / 1e12, 1)
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    big.zero_()
    # 1 GiB read + 1 GiB written; the best of three grid sizes (one to four rounds of resident waves)
    out["hbm_copy_gbs"] = round(max(2 * (1 << 30) / timed(ikbo.IKBO_PROBE_COPY, big, 0, b) / 1e9
                                    for b in (2048, 4096, 8192)), 1)
    out["hbm_read_gbs"] = round(max(((2 << 30) - b * 1024) / timed(ikbo.IKBO_PROBE_READ, big, 0, b) / 1e9
                                    for b in (2048, 4096, 8192)), 1)
    del big
    out["spec"] = {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
    return out


def host_info():
    """The host's thread count and CPU model (from /proc/cpuinfo, what lscpu prints as Model name)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_nproc": os.cpu_count(), "cpu_model": model}


# Threads for the oracle: every host thread up to the CPU share one GPU's process has on the box
# (16); host_nproc in the JSON says how many the machine shows.
CPU_SHARE = 16


def cpu_baseline(args, np):
    """The fp64 oracle, untuned, on a bounded sample of the same workload (about 10-30 s of CPU
    work). Its rate (effective FLOPs of the sampled candidates / seconds) is the baseline; the
    full workload's CPU time is extrapolated from it (work x total / sample)."""
    import oracle
    import synth
    nthreads = max(1, min(CPU_SHARE, os.cpu_count() or 1))
    t0 = time.perf_counter()
    total_work = None
    if args.workload in ("block", "layer"):
        g, s = synth.block_specs()
        total_work = g.flops() + s.flops() if args.workload == "block" else None
        n_per = args.cpu_sample // 4 if args.cpu_sample else 96
        reqs = [0, 1, g.R // 2, g.R - 1]
        off = g.offsets
        # the sample: n_per candidates spread evenly over each of requests 0, 1, R/2 and R - 1 (all
        # candidates cost the same: one request length, one MLP); compact inputs: the sampled
        # candidates' rows, and the K/V blocks of their requests only
        picks = [np.linspace(off[r], off[r + 1] - 1, n_per).round().astype(np.int64) for r in reqs]
        x_r = synth.glm_x(g, "x_r")
        x_c = np.concatenate([synth.glm_x(g, "x_c", int(c), 1) for p in picks for c in p])
        m_sub = np.repeat(np.array(reqs, np.int32), n_per)
        layers = [dict(synth.glm_weights(g, li), act=g.layers[li].act) for li in range(len(g.layers))]
        k = np.stack([synth.dca_kv_request(s, "k", r) for r in reqs])
        v = np.stack([synth.dca_kv_request(s, "v", r) for r in reqs])
        m_kv = np.repeat(np.arange(len(reqs), dtype=np.int32), n_per)
        n = len(m_sub)
        log("cpu baseline: oracle on %d candidates with %d threads" % (n, nthreads))
        t0 = time.perf_counter()
        res = oracle.glm(x_r, x_c, layers, m=m_sub, want_request=args.workload == "layer", nthreads=nthreads)
        qo = res["y_c"]
        oracle.dca(qo.reshape(n, s.Lq, s.H, s.d), k, v, len(reqs), m=m_kv, nthreads=nthreads)
        secs = time.perf_counter() - t0
        work = (g.flops() + s.flops()) / g.C * n
        sample = ("%d candidates (%d spread evenly over each of requests %s): GLM-MLP then DCA, chained in fp64"
                  % (n, n_per, reqs))
        if args.workload == "layer":
            # plus, for request 0: its four K/V projections and its request-side attention
            r0, hd, d_in = reqs[0], s.H * s.d, synth.seq_width(s)
            rows_r = synth.seq_rows(s, r0 * s.L, s.L)
            wts = [synth.kv_weight(s, nm) for nm in ("w_kc", "w_vc", "w_kr", "w_vr")]
            t1 = time.perf_counter()
            proj = [oracle.linear(rows_r, w) for w in wts]
            kr = proj[2].astype(np.float32).reshape(1, s.L, s.H, s.d)
            vr = proj[3].astype(np.float32).reshape(1, s.L, s.H, s.d)
            q_r = res["y_r"][r0].astype(np.float32).reshape(1, s.Lq, s.H, s.d)
            oracle.request_attention(q_r, kr, vr, nthreads=nthreads)
            secs += time.perf_counter() - t1
            work += 4 * 2.0 * s.L * d_in * hd + 4.0 * s.Lq * s.H * s.d * s.L
            sample += "; plus the four K/V projections of request %d's %d sequence rows and its A^R" % (r0, s.L)
    elif args.workload == "fm":
        R, per_r, n_r, n_c, d = FM_SHAPE
        # every request and all their candidates: the whole workload (a few seconds of oracle work)
        reqs = list(range(R))
        n_per = min(per_r, args.cpu_sample // len(reqs)) if args.cpu_sample else per_r
        x_r = synth.draw(0, 80, R * n_r * d, "bf16").reshape(R, n_r, d)
        x_c = np.concatenate([synth.draw(0, 81, n_per * n_c * d, "bf16", start=r * per_r * n_c * d)
                              for r in reqs]).reshape(-1, n_c, d)
        m_sub = np.repeat(np.array(reqs, np.int32), n_per)
        t0 = time.perf_counter()
        oracle.fm(x_r, x_c, m=m_sub)
        secs = time.perf_counter() - t0
        work = 2.0 * len(m_sub) * n_c * (n_r + n_c) * d
        sample = "%d candidates (the first %d of each of the %d requests)" % (len(m_sub), n_per, len(reqs))
    elif args.workload == "stack":
        g, s = synth.block_specs()
        r0 = 0
        n = args.cpu_sample if args.cpu_sample else 64
        cands = np.arange(s.offsets[r0], s.offsets[r0] + n)
        W, hd = s.Lq * s.H * s.d, s.H * s.d
        # request 0's rows of every input, then both layers on the sample (the first layer's output
        # goes to the second as fp32)
        x_r = synth.glm_x(g, "x_r", r0, 1)
        x_c = synth.glm_x(g, "x_c", int(cands[0]), n)
        l1 = [dict(synth.glm_weights(g, li), act=g.layers[li].act) for li in range(len(g.layers))]
        l2h, seq2, kv2h = stack_layer2(np, synth, s)
        m1 = np.zeros(n, np.int32)
        t0 = time.perf_counter()
        y1 = oracle.dca_layer(x_r, x_c, l1, synth.seq_rows(s, r0 * s.L, s.L),
                              *[synth.kv_weight(s, nm) for nm in ("w_kc", "w_vc", "w_kr", "w_vr")],
                              q_len=s.Lq, heads=s.H, m=m1, nthreads=nthreads)
        f32 = lambda a: oracle.decode(a).astype(np.float32)
        l2 = [{k: (f32(v) if k in ("w_rr", "w_cr", "w_cc") else v) for k, v in ly.items()} for ly in l2h]
        oracle.dca_layer(y1["y_r"].astype(np.float32), y1["y_c"].astype(np.float32), l2, f32(seq2(r0 * s.L, s.L)),
                         *[f32(w) for w in kv2h], q_len=s.Lq, heads=s.H, m=m1, nthreads=nthreads)
        secs = time.perf_counter() - t0
        attn_req = 2 * 2 * 2.0 * s.L * hd * hd + 4.0 * s.Lq * s.H * s.d * s.L
        attn_c = 4.0 * s.Lq * s.H * s.d * s.L
        ly0, ly1 = g.layers
        work = (mlp_flops(n, 1, [(ly0.k_req, ly0.k_cand, ly0.n_req, ly0.n_cand), (ly1.k_req, ly1.k_cand, ly1.n_req, ly1.n_cand)])
                + mlp_flops(n, 1, [(2 * W, 2 * W, 2048, 2048), (2048, 2048, W, W)]) + 2 * (attn_req + n * attn_c))
        sample = "request %d and its first %d candidates through both layers" % (r0, n)
    elif args.workload == "lcb_emb":
        R, per_r, n_r, n_c, d, k_r, k_c = LCBE_SHAPE
        # every request and all their candidates: the whole workload (a few seconds of oracle work)
        reqs = list(range(R))
        n_per = min(per_r, args.cpu_sample // len(reqs)) if args.cpu_sample else per_r
        x_r = synth.draw(0, 90, R * n_r * d, "bf16").reshape(R, n_r, d)
        x_c = np.concatenate([synth.draw(0, 91, n_per * n_c * d, "bf16", start=r * per_r * n_c * d)
                              for r in reqs]).reshape(-1, n_c, d)
        m_sub = np.repeat(np.array(reqs, np.int32), n_per)
        prm = lcbe_params(np, synth)
        t0 = time.perf_counter()
        oracle.lcb_emb(x_r, x_c, prm["w_rr"], prm["w_cr"], prm["w_cc"], m=m_sub, norm="layer",
                       gamma_r=prm["gamma_r"], beta_r=prm["beta_r"], gamma_c=prm["gamma_c"], beta_c=prm["beta_c"],
                       want_request=True)
        secs = time.perf_counter() - t0
        work = 2.0 * len(m_sub) * k_c * n_c * d + 2.0 * R * (k_r + k_c) * n_r * d
        sample = "%d candidates (the first %d of each of the %d requests)" % (len(m_sub), n_per, len(reqs))
    elif args.workload in ("dca_fixed", "dca_ragged"):
        s = synth.dca_spec(args.workload)
        reqs = [0, 1, s.R // 2, s.R - 1]
        n_per = args.cpu_sample // 4 if args.cpu_sample else 16
        off = s.offsets
        cands = np.concatenate([np.arange(off[r], min(off[r] + n_per, off[r + 1])) for r in reqs]).astype(np.int64)
        q = synth.dca_q(s)
        k, v = synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
        kw = {"kv_cu": s.kv_cu} if s.varlen else {}
        if not s.varlen:
            k = k.reshape(s.R, s.L, s.H, s.d)
            v = v.reshape(s.R, s.L, s.H, s.d)
        t0 = time.perf_counter()
        oracle.dca(q, k, v, s.R, m=s.cand_to_req, cands=cands, nthreads=nthreads, **kw)
        secs = time.perf_counter() - t0
        work = 4.0 * s.Lq * s.H * s.d * float(np.sum(s.kv_lens[s.cand_to_req[cands]]))
        total_work = s.flops()
        sample = "%d candidates of requests %s" % (len(cands), reqs)
    else:
        g = synth.glm_spec("lcb")
        # ten requests spread over the batch, up to 1024 candidates each (about 10 s of oracle work)
        reqs = sorted(set(np.linspace(0, g.R - 1, 10).astype(int).tolist()))
        n_per = args.cpu_sample // len(reqs) if args.cpu_sample else 1024
        off = g.offsets
        cands = np.concatenate([np.arange(off[r], min(off[r] + n_per, off[r + 1])) for r in reqs]).astype(np.int64)
        x_r, x_c = synth.glm_x(g, "x_r"), synth.glm_x(g, "x_c")
        ly = dict(synth.glm_weights(g, 0), act="gelu")
        t0 = time.perf_counter()
        oracle.glm(x_r, x_c, [ly], m=g.cand_to_req, cands=cands, nthreads=nthreads)
        secs = time.perf_counter() - t0
        work = g.flops() / g.C * len(cands)
        total_work = g.flops()
        sample = "%d candidates of requests %s" % (len(cands), reqs)
    log("cpu baseline: %.1f s" % secs)
    out = {"value": round(work / secs / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
           "sample": sample, "seconds": round(secs, 2)}
    out.update(host_info())
    if total_work:
        out["extrapolated_full_seconds"] = round(secs * total_work / work, 1)
        out["extrapolated"] = "full-workload CPU time = sample time x (workload FLOPs / sample FLOPs)"
    return out


if __name__ == "__main__":
    main()
