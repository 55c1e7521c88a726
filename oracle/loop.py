"""Oracle generate loop: prompt encode, then block-autoregressive canvases.

[bohu] 一 and [chooseai] (multi-canvas paragraph): each 256-token canvas starts
from random tokens, is denoised over several rounds, and once final is appended
to the KV cache before the next canvas starts.  [mlqm] 四: at most 48 rounds,
with an adaptive early stop.
"""
from __future__ import annotations

from typing import Callable, List, Optional

import numpy as np

from . import sampler as smp
from .model import OracleModel


def run_canvas(model: OracleModel, sp, seeds: np.ndarray, steps_limit: Optional[int] = None,
               on_step: Optional[Callable] = None) -> dict:
    """Denoise one canvas for every request; returns the final canvas and per-step records."""
    cfg = model.cfg
    B, n = model.B, cfg.canvas_len
    canvas = np.stack([smp.init_canvas(int(seeds[b]), model.canvas_index, n, cfg.vocab)
                       for b in range(B)])
    done = np.zeros(B, bool)
    prev_am: List[Optional[np.ndarray]] = [None] * B
    steps = []
    S = sp.max_steps if steps_limit is None else min(sp.max_steps, steps_limit)
    for t in range(S):
        out = model.denoise_step(canvas, t, sp, seeds, active=~done)
        rec = {"n_committed": np.zeros(B, np.int32), "done": done.copy()}
        for b in range(B):
            if done[b]:
                continue
            new, mask, ncom, d = smp.commit(out["H"][b], out["y"][b], out["am"][b], prev_am[b],
                                            canvas[b], t, sp.max_steps, sp.entropy_bound,
                                            sp.stop_mode, sp.stop_tau, int(seeds[b]),
                                            model.canvas_index, cfg.vocab)
            canvas[b] = new
            prev_am[b] = out["am"][b].copy()
            rec["n_committed"][b] = ncom
            done[b] = d
        rec["done"] = done.copy()
        steps.append(rec)
        if on_step is not None:
            on_step(t, out, canvas, rec)
        if done.all():
            break
    return {"canvas": canvas, "steps": steps, "done": done}


def generate(model: OracleModel, prompts: np.ndarray, sp, seeds: np.ndarray, canvases: int,
             steps_limit: Optional[int] = None) -> List[np.ndarray]:
    model.encode_prompt(prompts)
    finals = []
    for _ in range(canvases):
        res = run_canvas(model, sp, seeds, steps_limit)
        model.commit_canvas_to_kv(res["canvas"])
        finals.append(res["canvas"])
    return finals
