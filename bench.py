#!/usr/bin/env python3
"""Throughput of the denoise-step hot path on one MI355X.

A step is one dg_denoise_step + dg_sample_commit over the canvas batch; at the
end of each canvas's step budget the canvas is appended to the KV cache
(dg_commit_canvas_to_kv, inside the timed region) and a fresh canvas starts.
value = committed canvas tokens per second = B * 256 * (K / S) / seconds for
K timed steps of an S-step canvas budget, the seconds being the timed steps
plus the pro-rata share K / S of one canvas commit (whatever commits fall in
the timed region are replaced by that share).  The default workload is the
26B-A4B-scale proxy (30 layers, d 2048, 128 experts top-8, vocabulary
262144); the small, multi-canvas and batched workloads follow in short runs
reported under other_workloads.  Inputs (weights, prompt) are seeded
synthetic data already resident in device memory when timing starts; the
prompt encode is timed separately.  Per-step latencies come from one event
per step on the launch stream (median and p90 reported).

The dominant stage is picked from an all-stage timing pass during warm-up, then
timed live with HIP events inside the library (on the launch stream) during
the timed region; its algorithmic bytes / flops per launch give the roofline.
stage_roofline_warmup gives every stage's fraction of its own roofline from
the warm-up timings (the same event pairs, before the timed region).
The CPU baseline is the oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import dg_inputs as di  # noqa: E402

METRIC = "committed canvas tok/s + denoise-step latency (ms), 1×MI355X"
HBM_PEAK_GBS = 8000.0

# HBM traffic per launch of a stage's kernel from two rocprofv3 --pmc passes over
# this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, averaged over the
# stage's dispatches of the timed steps), each scaled by what the counter reads
# for a plain 256 MiB copy (--calibrate-copy): FETCH_SIZE x2.0, WRITE_SIZE x1.0.
# Keyed by (workload, stage); valid only for the kernel source it was taken on
# (sha1 of the file), reported as null otherwise.
MEASURED_TRAFFIC = {
    # gate/up expert streaming, small workload: FETCH 43067.6 KiB x2.0 + WRITE 2048.1 KiB x1.0
    ("small", "expert_up"): {"bytes_per_launch": 90290784, "sha1": "bd5783d754f0351abad89e32efe0de52f165e312"},
    # gate/up expert streaming, 30-layer proxy (one step's 30 launches): FETCH 84028.6 KiB x2.0 + WRITE 3072.1 KiB x1.0
    ("proxy", "expert_up"): {"bytes_per_launch": 175236422, "sha1": "6238650c9184f54eb8bb54b9e7f012bf021065fe"},
}
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_work(stage: str, mc, B: int, ctx: int, n_experts_active: int):
    """Algorithmic (bytes, flops) of one launch of a stage at canvas shape."""
    es = 2 if mc.dtype == "bf16" else 4
    n = mc.canvas_len
    R = B * n
    d, F, k, V = mc.d_model, mc.ffn_hidden, mc.top_k, mc.vocab
    hd, Hq, Hkv = mc.head_dim, mc.n_q_heads, mc.n_kv_heads
    keys = ctx + n
    # expert weight bytes per element: 1 for FP8 codes (plus one fp32 scale per output channel)
    fp8 = getattr(mc, "expert_dtype", "") == "fp8"
    wes = 1 if fp8 else es
    if stage == "expert_up":
        by = n_experts_active * (2 * F * d * wes + (2 * F * 4 if fp8 else 0)) + R * d * es + R * k * F * es
        fl = 2 * R * k * d * F * 2
    elif stage == "expert_down":
        by = n_experts_active * (d * F * wes + (d * 4 if fp8 else 0)) + R * k * F * es + R * k * d * es
        fl = 2 * R * k * F * d
    elif stage == "lm_head":     # with the head statistics in its epilogue: writes P~ and the chunk records
        # head rows: bf16 E, or (FP8 head) one E4M3 code per weight plus one fp32 scale per id
        hb = V * d + V * 4 if getattr(mc, "head_dtype", "") == "fp8" else V * d * es
        by = hb + R * d * es + (R * V * es if mc.self_cond else 0) + R * ((V + 127) // 128) * 32
        fl = 2 * R * d * V
    elif stage == "attn":
        by = 2 * B * Hkv * keys * hd * es + 2 * R * Hq * hd * es
        fl = 4 * R * Hq * keys * hd
    elif stage == "sampler":     # per-row merge of the 128-id chunk records
        by = R * ((V + 127) // 128) * 32 + (R * ((V + 127) // 128) * 4 if mc.self_cond else 0)
        fl = 0
    elif stage == "selfcond":
        by = R * V * es + V * d * es + R * d * 4
        fl = 2 * R * V * d
    elif stage == "qkv":
        by = (Hq + 2 * Hkv) * hd * d * es + R * d * es + R * (Hq + 2 * Hkv) * hd * 4
        fl = 2 * R * d * (Hq + 2 * Hkv) * hd
    elif stage == "oproj":
        by = Hq * hd * d * es + R * Hq * hd * es + 2 * R * d * 4
        fl = 2 * R * Hq * hd * d
    elif stage == "router":      # logits GEMM + top-k + bucketing
        E = mc.n_experts
        by = E * d * es + R * d * es + R * E * 4 + 3 * R * k * 4
        fl = 2 * R * d * E
    elif stage == "embed":       # gather (+ self-conditioning projection)
        by = R * d * es + R * d * 4 + ((d * d * es + R * d * 4) if mc.self_cond else 0)
        fl = 2 * R * d * d if mc.self_cond else 0
    elif stage == "norm":
        by = R * d * 4 + R * d * es
        fl = 0
    elif stage == "combine":     # expert outputs in the operand type, residual h in fp32
        by = R * k * d * es + 2 * R * d * 4
        fl = 2 * R * k * d
    elif stage == "commit":
        by = R * 16
        fl = 0
    else:
        return None
    return by, fl


STAGE_SOURCE = {"expert_up": "k_expert.hip", "expert_down": "k_expert.hip", "attn": "k_attn.hip",
                "router": "k_misc.hip", "sampler": "k_sampler.hip", "lm_head": "k_gemm.hip", "qkv": "k_gemm.hip"}


def measured_traffic(workload: str, stage: str):
    """Counter-derived HBM bytes per launch, or None if absent or taken on another kernel source."""
    import hashlib
    rec = MEASURED_TRAFFIC.get((workload, stage))
    src = STAGE_SOURCE.get(stage)
    if rec is None or src is None:
        return None
    path = os.path.join(ROOT, "discrete_text_diffusion_dg_amd", "csrc", src)
    with open(path, "rb") as f:
        if hashlib.sha1(f.read()).hexdigest() != rec["sha1"]:
            return None
    return rec["bytes_per_launch"]


def roofline(stage, ms_total, launches, mc, B, ctx, n_act, traffic=None):
    w = stage_work(stage, mc, B, ctx, n_act)
    if w is None or launches == 0:
        return None
    by, fl = w
    t = ms_total / launches / 1e3
    peak_t = MFMA_PEAK_TFLOPS[mc.dtype]
    if fl / max(by, 1) > peak_t * 1e12 / (HBM_PEAK_GBS * 1e9):
        ach = fl / t / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_t, "unit": "TFLOP/s",
                "frac": round(ach / peak_t, 4), "traffic": traffic, "kernel": stage,
                "launch_us": round(t * 1e6, 2), "bytes_per_launch": by, "flops_per_launch": fl}
    ach = by / t / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": stage,
            "launch_us": round(t * 1e6, 2), "bytes_per_launch": by, "flops_per_launch": fl}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(wl, budget_s: float):
    """The oracle on the host cores, on a bounded sample of the workload.

    Models of up to 8 layers run whole: prompt encode, denoise + commit steps
    until about half the budget is spent (at least 2), one canvas commit.
    Deeper models run their first 2 layers (the same seeded weights) with the
    full embedding, LM head and sampler; each pass's time is extrapolated to
    all layers from the measured per-layer time (labelled as such)."""
    import dataclasses
    from oracle.model import OracleModel
    from oracle import sampler as osmp
    mc, sp = wl.model, wl.sampler
    B = wl.batch
    L_full = mc.n_layers
    L_run = L_full if L_full <= 8 else 2
    mrun = dataclasses.replace(mc, n_layers=L_run)
    weights = di.make_weights(mrun, wl.seed)
    prompts = di.make_prompts(mc.vocab, B, wl.prompt_len, wl.seed)
    seeds = di.request_seeds(wl.seed, B)
    om = OracleModel(mrun, weights, B, wl.prompt_len + 2 * mc.canvas_len)
    om.W("emb")                        # widened once, as a resident model would hold it
    marks = []
    om.on_layer = lambda l: marks.append(time.perf_counter())

    def timed(fn):
        """(seconds, seconds extrapolated to L_full layers) of one pass over the requests."""
        marks.clear()
        t0 = time.perf_counter()
        fn()
        t = time.perf_counter() - t0
        if L_run == L_full:
            return t, t
        # marks: end of each layer, request after request; a layer's time is the gap
        # to the previous layer's end within the same request
        gaps = [marks[j + l] - marks[j + l - 1] for j in range(0, len(marks), L_run) for l in range(1, L_run)]
        per_layer = float(np.mean(gaps)) if gaps else 0.0
        return t, t + (L_full - L_run) * per_layer * (len(marks) // L_run)

    t_enc, x_enc = timed(lambda: om.encode_prompt(prompts))
    canvas = np.stack([osmp.init_canvas(int(seeds[b]), 0, mc.canvas_len, mc.vocab) for b in range(B)])
    steps, t_steps, x_steps = 0, 0.0, 0.0
    while steps < 2 or (t_steps < budget_s * 0.5 and steps < sp.max_steps):
        def one():
            out = om.denoise_step(canvas, steps, sp, seeds)
            for b in range(B):
                canvas[b], _, _, _ = osmp.commit(out["H"][b], out["y"][b], out["am"][b], None, canvas[b], steps,
                                                 sp.max_steps, sp.entropy_bound, sp.stop_mode, sp.stop_tau,
                                                 int(seeds[b]), 0, mc.vocab)
        t, x = timed(one)
        t_steps += t
        x_steps += x
        steps += 1
    _, x_commit = timed(lambda: om.commit_canvas_to_kv(canvas))
    x_step = x_steps / steps
    tok_s = B * mc.canvas_len / (sp.max_steps * x_step + x_commit)
    part = ("" if L_run == L_full else
            f"; first {L_run} of {L_full} layers run (same weights, full embedding, LM head and sampler), "
            f"each pass extrapolated to {L_full} layers from its measured per-layer time")
    return {"value": round(tok_s, 4), "unit": "tok/s", "cores": int(_blas_threads()), "kind": "oracle",
            "sample": (f"{wl.name}: prompt encode ({wl.prompt_len} tokens x {B}) {x_enc:.2f} s, "
                       f"{steps} denoise+commit steps {x_step:.3f} s/step, canvas commit {x_commit:.2f} s; "
                       f"tok/s = {B}*{mc.canvas_len} / ({sp.max_steps} steps * s/step + commit){part}"),
            "ms_per_step": round(x_step * 1e3, 2), "extrapolated": L_run != L_full}


class Runner:
    """One workload on the device: weights, engine, prompt encode, the step loop.

    Steps run through the library's device-driven loop (dg_run_canvas), one
    step per call so that an event can follow each: the step index,
    temperature and done flags stay on the device, a finished canvas is
    committed to the KV cache by the same call, and the next call starts a new
    canvas."""

    def __init__(self, wl, steps: int, warmup: int, device_weights=None):
        import torch
        from discrete_text_diffusion_dg_amd.runtime import Engine, upload_weights
        self.torch = torch
        self.wl = wl
        mc, sp = wl.model, wl.sampler
        self.B, self.n, self.S = wl.batch, mc.canvas_len, sp.max_steps
        total = warmup + steps + 2 * self.S          # + the accounting canvas
        canvases = (total + self.S - 1) // self.S + 2
        max_ctx = wl.prompt_len + self.n * (canvases + 1)
        t0 = time.perf_counter()
        W = di.make_weights(mc, wl.seed, cache=False)       # streamed: generated, uploaded, dropped
        names = W.names()
        if device_weights is not None:                      # the same seeded weights, already on the device
            dw = device_weights
        else:
            dw, done_b, next_log = {}, 0, 4e9
            for nm_ in names:
                dw.update(upload_weights(W, [nm_], "cuda"))
                done_b += dw[nm_].numel() * dw[nm_].element_size()
                if done_b >= next_log:
                    log(f"[bench] {wl.name}: {done_b / 1e9:.1f} of {W.nbytes() / 1e9:.1f} GB of weights on the device")
                    next_log += 4e9
            log(f"[bench] {wl.name}: weights {W.nbytes() / 1e9:.2f} GB generated+uploaded in "
                f"{time.perf_counter() - t0:.1f} s")
        self.weights = dw
        self.eng = Engine(mc, dw, names, self.B, max_ctx)
        self.eng.set_seeds(di.request_seeds(wl.seed, self.B))
        prompts = torch.from_numpy(di.make_prompts(mc.vocab, self.B, wl.prompt_len, wl.seed)).cuda()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        self.eng.encode_prompt(prompts)
        e1.record()
        torch.cuda.synchronize()
        self.encode_ms = e0.elapsed_time(e1)
        log(f"[bench] {wl.name}: prompt encode {self.encode_ms:.2f} ms")
        self.t = 0
        self.canvases_done = 0

    def step(self, graph: bool, commit: bool = True) -> bool:
        """One step of the current canvas (a new canvas when t == 0); True if the canvas finished."""
        sp = self.wl.sampler
        issued, finished = self.eng.run_canvas_device(sp, first_step=self.t, n_steps=1, graph=graph,
                                                      early_exit=sp.stop_mode != 0, commit_kv=commit)
        self.t += issued
        if finished:
            self.canvases_done += 1
            self.t = 0
        return finished

    def close(self):
        self.eng.close()
        del self.eng
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def measure(wl, steps: int, warmup: int, stage_detail: bool, graph: bool = True, device_weights=None):
    """Timed run of one workload; returns the bench fields (and the Runner, still open)."""
    import torch
    r = Runner(wl, steps, warmup, device_weights)
    eng, mc = r.eng, wl.model
    B, n, S = r.B, r.n, r.S
    # warm-up: the first step without timers (one-off costs), then every stage's event
    # pairs (the captured graph carries none, so these steps run uncaptured)
    n_first = 1 if warmup > 1 else 0
    for _ in range(n_first):
        r.step(graph=False)
    prof = {}
    if stage_detail:
        eng.profile(STAGES)
    for _ in range(warmup - n_first):
        r.step(graph=False)
    torch.cuda.synchronize()
    if stage_detail:
        prof = eng.profile_read()
        eng.profile([])
    ctx_w = eng.ctx_len
    dominant = max(prof, key=lambda k: prof[k][0]) if prof else None
    routed = eng.route_view(B * n).cpu().numpy()
    act_per_layer = [int(np.unique(x[x >= 0]).size) for x in routed]
    n_act = float(np.mean(act_per_layer))
    if graph:
        r.step(graph=True)       # capture outside the timed region
        torch.cuda.synchronize()
    r.canvases_done = 0
    t_first = r.t
    # timed region: exactly `steps` steps; one event after each step (same stream as the
    # library's launches) gives the per-step latencies
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        r.step(graph=graph)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    ms = float(ev[0].elapsed_time(ev[steps]))
    commits_timed = r.canvases_done
    # the dominant stage's kernels timed with the library's event pairs over the same
    # steps replayed uncaptured (same kernels and launch shapes; the graph holds no events)
    dom_ms, dom_n = 0.0, 0
    if dominant:
        while r.t != t_first:
            r.step(graph=graph)
        eng.profile([dominant])
        for _ in range(steps):
            r.step(graph=False)
        torch.cuda.synchronize()
        dom_ms, dom_n = eng.profile_read().get(dominant, (0.0, 0))
        eng.profile([])
    # accounting canvas (untimed): positions committed per step over one whole canvas,
    # then the time of one canvas commit to the KV cache
    while r.t != 0:
        r.step(graph=graph)
    ncom = []
    while True:
        fin = r.step(graph=graph, commit=False)
        ncom.append(int(eng.n_committed.sum().item()))
        if fin:
            break
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    eng.commit_canvas_to_kv()
    c1.record()
    torch.cuda.synchronize()
    commit_ms = c0.elapsed_time(c1)
    # committed canvas tokens over the step + commit time they cost: the timed region's
    # own commits are replaced by the pro-rata share of one commit (steps / S canvases)
    canv = steps / S
    ms_adj = ms - commits_timed * commit_ms + canv * commit_ms
    tok_s = B * n * canv / (ms_adj / 1e3)
    out = {"value": round(tok_s, 2), "ms_per_step": round(ms / steps, 4), "commit_ms": round(commit_ms, 3),
           "canvases_per_timed_region": round(canv, 4), "commits_in_timed_region": commits_timed,
           "ms_per_step_median": round(float(np.median(per)), 4),
           "ms_per_step_p90": round(float(np.percentile(per, 90)), 4),
           "steps_per_s": round(steps / (ms / 1e3), 2), "encode_ms": round(r.encode_ms, 3),
           "wall_ms": round(wall * 1e3, 2), "loop": "device loop, captured graph" if graph else "device loop",
           "n_committed_per_step": ncom, "active_experts_per_layer": act_per_layer}
    if stage_detail:
        out["stage_ms_warmup"] = {k: round(v[0] / max(warmup - n_first, 1), 4) for k, v in prof.items()}
        out["roofline"] = roofline(dominant, dom_ms, dom_n, mc, B, ctx_w, n_act,
                                   measured_traffic(wl.name, dominant)) if dominant else None
        stage_rl = {}
        for k, (k_ms, k_n) in prof.items():
            x = roofline(k, k_ms, k_n, mc, B, ctx_w, n_act)
            if x is not None:
                stage_rl[k] = {f: x[f] for f in ("bound", "achieved", "unit", "frac", "launch_us")}
        out["stage_roofline_warmup"] = stage_rl
        log(f"[bench] {wl.name}: warm-up stage ms: " + ", ".join(f"{k} {v[0]:.2f}/{v[1]}" for k, v in prof.items()))
        log(f"[bench] {wl.name}: dominant {dominant}: {dom_ms / max(dom_n, 1) * 1e3:.1f} us/launch")
    log(f"[bench] {wl.name}: {steps} steps in {ms:.2f} ms (median {np.median(per):.3f}, p90 "
        f"{np.percentile(per, 90):.3f} ms/step; wall {wall * 1e3:.1f} ms); {tok_s:.1f} committed tok/s")
    return out, r


STAGES = ["embed", "norm", "qkv", "attn", "oproj", "router", "expert_up", "expert_down", "combine",
          "lm_head", "sampler", "selfcond", "commit"]
EXTRA_WORKLOADS = ("small", "multicanvas", "batched", "batched-topk")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--workload", default="proxy", choices=sorted(di.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the short runs of the other workloads reported as extra keys")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-graph", action="store_true", help="device loop without the captured step graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 256 MiB three times (the reference kernel for the HBM counters)")
    a = ap.parse_args()
    if a.calibrate_copy:
        import torch
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 256 MiB three times")
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the multi-GPU sharding of this path "
              "is a design note, not an implemented mode", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    wl = di.workload(a.workload)
    mc, sp = wl.model, wl.sampler
    res, runner = measure(wl, a.steps, a.warmup, stage_detail=True, graph=not a.no_graph)
    dw = {wl.name: runner.weights}
    runner.close()
    extras = {}

    def same_model(name):
        """Workloads on the same seeded weights share the device copy."""
        x = di.workload(name)
        base = dataclasses.replace(x.model, expert_dtype="", head_dtype="")
        for k in list(dw):
            w0 = di.workload(k)
            if dataclasses.replace(w0.model, expert_dtype="", head_dtype="") == base and w0.seed == x.seed:
                return dw[k]
        return None

    # the headline model with its experts in FP8, with experts and LM head in FP8,
    # and with top-k sampling, then the other workloads (the batched shape also
    # with top-k sampling)
    names = [n_ for n_ in (wl.name + "-fp8", wl.name + "-fp8-head", wl.name + "-topk") if n_ in di.WORKLOADS]
    names += [n_ for n_ in EXTRA_WORKLOADS if n_ != wl.name]
    if a.no_extras:
        names = []
    for name in names:
        try:
            xw = di.workload(name)
            detail = name.startswith(wl.name)
            x, r = measure(xw, a.steps if detail else 24, a.warmup if detail else 3, stage_detail=detail,
                           graph=not a.no_graph, device_weights=same_model(name))
            if name not in dw and same_model(name) is None:
                dw[name] = r.weights
            r.close()
            keys = ["value", "ms_per_step", "ms_per_step_median", "ms_per_step_p90", "steps_per_s", "encode_ms"]
            if detail:
                keys += ["stage_ms_warmup", "roofline"]
            extras[name] = {k: x[k] for k in keys if k in x}
            extras[name]["steps"] = a.steps if detail else 24
            if xw.model.expert_dtype == "fp8":
                extras[name]["dtype"] = ("bf16 activations, fp8 e4m3 expert and LM-head weights"
                                         if xw.model.head_dtype == "fp8" else "bf16 activations, fp8 e4m3 expert weights")
            if xw.sampler.top_k:
                extras[name]["sampler"] = f"top-{xw.sampler.top_k} truncated"
        except Exception as ex:   # reported, never fatal for the headline
            extras[name] = {"error": repr(ex)}
    dw.clear()
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    cpu = None
    if not a.no_cpu_baseline:
        try:
            cpu = cpu_baseline(wl, a.cpu_budget)
            log(f"[bench] cpu baseline {cpu['value']} tok/s ({cpu['sample']})")
        except Exception as ex:  # reported, never fatal for the GPU number
            cpu = {"value": None, "unit": "tok/s", "cores": os.cpu_count(), "kind": "oracle",
                   "sample": f"failed: {ex!r}"}

    line = {
        "metric": METRIC, "value": res["value"], "unit": "tok/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": mc.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "canvas": mc.canvas_len, "prompt_len": wl.prompt_len,
                   "steps_per_canvas": sp.max_steps, "layers": mc.n_layers, "d_model": mc.d_model,
                   "heads": f"{mc.n_q_heads}/{mc.n_kv_heads}x{mc.head_dim}",
                   "experts": f"{mc.top_k}/{mc.n_experts}", "ffn_hidden": mc.ffn_hidden, "vocab": mc.vocab,
                   "self_cond": mc.self_cond, "stop": "mean H < %g" % sp.stop_tau if sp.stop_mode else "none",
                   "parallelism": "none (1 GPU)"},
    }
    line.update({k: v for k, v in res.items() if k not in ("value", "ms_per_step")})
    line["cpu_baseline"] = cpu
    line["other_workloads"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
