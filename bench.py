#!/usr/bin/env python3
"""Throughput of the denoise-step hot path on one MI355X.

A step is one dg_denoise_step + dg_sample_commit over the canvas batch; at the
end of each canvas's step budget the canvas is appended to the KV cache
(dg_commit_canvas_to_kv, inside the timed region) and a fresh canvas starts.
value = committed canvas tokens per second = B * 256 * canvases / seconds,
with a partially finished canvas counted pro rata.  Inputs (weights, prompt)
are seeded synthetic data already resident in device memory when timing
starts; the prompt encode is timed separately.

The dominant stage is picked from an all-stage timing pass during warm-up, then
timed live with HIP events inside the library (on the launch stream) during
the timed region; its algorithmic bytes / flops per launch give the roofline.
stage_roofline_warmup gives every stage's fraction of its own roofline from
the warm-up timings (the same event pairs, before the timed region).
The CPU baseline is the oracle timed on a bounded sample of the same workload.
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
    if stage == "expert_up":
        by = n_experts_active * 2 * F * d * es + R * d * es + R * k * F * es
        fl = 2 * R * k * d * F * 2
    elif stage == "expert_down":
        by = n_experts_active * d * F * es + R * k * F * es + R * k * d * 4
        fl = 2 * R * k * F * d
    elif stage == "lm_head":     # with the head statistics in its epilogue: writes P~ and the chunk records
        by = V * d * es + R * d * es + (R * V * es if mc.self_cond else 0) + R * ((V + 127) // 128) * 32
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
    elif stage == "combine":
        by = R * k * d * 4 + 2 * R * d * 4
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


def cpu_baseline(wl, weights, prompts, seeds, budget_s: float):
    """Oracle on the host cores: prompt encode, then denoise steps and one canvas commit."""
    from oracle.model import OracleModel
    from oracle import sampler as osmp
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    mc, sp = wl.model, wl.sampler
    B = wl.batch
    om = OracleModel(mc, weights, B, wl.prompt_len + 2 * mc.canvas_len)
    t0 = time.perf_counter()
    om.encode_prompt(prompts)
    t_enc = time.perf_counter() - t0
    canvas = np.stack([osmp.init_canvas(int(seeds[b]), 0, mc.canvas_len, mc.vocab) for b in range(B)])
    steps, t_steps = 0, 0.0
    while steps < 2 or (t_steps < budget_s * 0.5 and steps < sp.max_steps):
        t0 = time.perf_counter()
        out = om.denoise_step(canvas, steps, sp, seeds)
        for b in range(B):
            canvas[b], _, _, _ = osmp.commit(out["H"][b], out["y"][b], out["am"][b], None, canvas[b], steps,
                                             sp.max_steps, sp.entropy_bound, sp.stop_mode, sp.stop_tau,
                                             int(seeds[b]), 0, mc.vocab)
        t_steps += time.perf_counter() - t0
        steps += 1
    t0 = time.perf_counter()
    om.commit_canvas_to_kv(canvas)
    t_commit = time.perf_counter() - t0
    t_step = t_steps / steps
    tok_s = B * mc.canvas_len / (sp.max_steps * t_step + t_commit)
    return {"value": round(tok_s, 3), "unit": "tok/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{wl.name}: prompt encode ({wl.prompt_len} tokens x {B}) {t_enc:.2f} s, "
                       f"{steps} denoise+commit steps {t_step:.3f} s/step, canvas commit {t_commit:.2f} s; "
                       f"tok/s = {B}*{mc.canvas_len} / ({sp.max_steps} steps * s/step + commit)"),
            "ms_per_step": round(t_step * 1e3, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--workload", default="small", choices=sorted(di.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
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
    from discrete_text_diffusion_dg_amd.runtime import Engine, upload_weights
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    wl = di.workload(a.workload)
    mc, sp = wl.model, wl.sampler
    B, n, S = wl.batch, mc.canvas_len, sp.max_steps
    total_steps = a.warmup + a.steps
    canvases = (total_steps + S - 1) // S + 1
    max_ctx = wl.prompt_len + n * (canvases + 1)
    t0 = time.perf_counter()
    # host copies are kept only for the CPU baseline; large models stream to the device
    W = di.make_weights(mc, wl.seed, cache=not a.no_cpu_baseline)
    names = W.names()
    dw, done_b, next_log = {}, 0, 4e9
    for nm in names:
        dw.update(upload_weights(W, [nm], "cuda"))
        done_b += dw[nm].numel() * dw[nm].element_size()
        if done_b >= next_log:
            log(f"[bench] {wl.name}: {done_b / 1e9:.1f} of {W.nbytes() / 1e9:.1f} GB of weights on the device")
            next_log += 4e9
    log(f"[bench] {wl.name}: weights {W.nbytes() / 1e9:.2f} GB generated+uploaded in {time.perf_counter() - t0:.1f} s")
    eng = Engine(mc, dw, names, B, max_ctx)
    seeds = di.request_seeds(wl.seed, B)
    eng.set_seeds(seeds)
    prompts = di.make_prompts(mc.vocab, B, wl.prompt_len, wl.seed)
    pt = torch.from_numpy(prompts).cuda()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    eng.encode_prompt(pt)
    e1.record()
    torch.cuda.synchronize()
    encode_ms = e0.elapsed_time(e1)
    log(f"[bench] prompt encode {encode_ms:.2f} ms")

    state = {"t": 0, "canvases_done": 0}
    eng.init_canvas()

    def one_step():
        t = state["t"]
        eng.denoise_step(t, sp)
        eng.sample_commit(t, sp)
        t += 1
        if sp.stop_mode != 0:
            finished = bool((eng.done != 0).all())
        else:
            finished = t >= S
        if finished or t >= S:
            eng.commit_canvas_to_kv()
            state["canvases_done"] += 1
            eng.init_canvas()
            eng.done.zero_()
            t = 0
        state["t"] = t

    # warm-up; every stage is timed after the first step (first launches pay
    # one-off costs) to find the dominant one
    n_first = 1 if a.warmup > 1 else 0
    for _ in range(n_first):
        one_step()
    eng.profile(["embed", "norm", "qkv", "attn", "oproj", "router", "expert_up", "expert_down", "combine",
                 "lm_head", "sampler", "selfcond", "commit"])
    for _ in range(a.warmup - n_first):
        one_step()
    torch.cuda.synchronize()
    prof = eng.profile_read()
    ctx_w = eng.ctx_len
    dominant = max(prof, key=lambda k: prof[k][0]) if prof else "expert_up"
    log("[bench] warm-up stage ms: " + ", ".join(f"{k} {v[0]:.2f}/{v[1]}" for k, v in prof.items()))
    # experts that receive rows, averaged over the layers (one expert launch per layer)
    routed = eng.route_view(B * n).cpu().numpy()
    act_per_layer = [int(np.unique(r).size) for r in routed]
    n_act = float(np.mean(act_per_layer))
    log(f"[bench] active experts per layer: {act_per_layer}")

    # timed region: exactly K steps, only the dominant stage carries events
    eng.profile([dominant])
    state["canvases_done"] = 0
    t_start_step = state["t"]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e0.record()
    for _ in range(a.steps):
        one_step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = e0.elapsed_time(e1)
    dom_ms, dom_n = eng.profile_read().get(dominant, (0.0, 0))
    eng.profile([])
    canv = a.steps / S
    tok_s = B * n * canv / (ms / 1e3)
    rl = roofline(dominant, dom_ms, dom_n, mc, B, ctx_w, n_act, measured_traffic(wl.name, dominant))
    # every stage against its own roofline, from the warm-up event timings
    # (matrix-core fraction for the products and attention, HBM fraction for
    # the streaming stages)
    stage_rl = {}
    for k, (k_ms, k_n) in prof.items():
        r = roofline(k, k_ms, k_n, mc, B, ctx_w, n_act)
        if r is not None:
            stage_rl[k] = {f: r[f] for f in ("bound", "achieved", "unit", "frac", "launch_us")}
    log(f"[bench] {a.steps} steps in {ms:.2f} ms (wall {wall * 1e3:.1f} ms); dominant {dominant}: "
        f"{dom_ms / max(dom_n, 1) * 1e3:.1f} us/launch")

    cpu = None
    if not a.no_cpu_baseline:
        try:
            cpu = cpu_baseline(wl, W, prompts, seeds, a.cpu_budget)
            log(f"[bench] cpu baseline {cpu['value']} tok/s ({cpu['sample']})")
        except Exception as ex:  # reported, never fatal for the GPU number
            cpu = {"value": None, "unit": "tok/s", "cores": os.cpu_count(), "kind": "oracle",
                   "sample": f"failed: {ex!r}"}

    line = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms / a.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": mc.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "canvas": n, "prompt_len": wl.prompt_len,
                   "steps_per_canvas": S, "layers": mc.n_layers, "d_model": mc.d_model,
                   "experts": f"{mc.top_k}/{mc.n_experts}", "vocab": mc.vocab,
                   "self_cond": mc.self_cond, "parallelism": "none (1 GPU)"},
        "steps_per_s": round(a.steps / (ms / 1e3), 2),
        "encode_ms": round(encode_ms, 3),
        "stage_ms_warmup": {k: round(v[0] / max(a.warmup - n_first, 1), 4) for k, v in prof.items()},
        "roofline": rl,
        "stage_roofline_warmup": stage_rl,
        "active_experts_per_layer": act_per_layer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    eng.close()


if __name__ == "__main__":
    main()
