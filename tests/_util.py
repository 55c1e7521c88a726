"""Helpers shared by the GPU parity tests: build both sides from the same seeded inputs."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import dg_inputs as di


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def make_engine(mc, weights, batch, max_ctx):
    import torch
    from discrete_text_diffusion_dg_amd.runtime import Engine, upload_weights
    names = weights.names()
    dw = upload_weights(weights, names, "cuda")
    eng = Engine(mc, dw, names, batch, max_ctx)
    torch.cuda.synchronize()
    return eng


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """max |got - ref| / max |ref| per row (last axis)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return np.abs(got - ref).max(axis=-1) / den


def tol_for(mc) -> float:
    # tolerance on logits and entropies: 2e-2 relative for bf16, 1e-4 for fp32
    return 2e-2 if mc.dtype == "bf16" else 1e-4


def micro(**kw) -> di.ModelConfig:
    base = dict(n_layers=2, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64, n_experts=8,
                ffn_hidden=256, top_k=2, vocab=4096, dtype="bf16", self_cond=True)
    base.update(kw)
    return di.ModelConfig(**base)


def replace(cfg, **kw):
    return dataclasses.replace(cfg, **kw)
