"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds shapes, workload definitions and seeded generators for the
model weights and prompts, and nothing of the method's arithmetic: no norm,
attention, routing, softmax or sampler step lives here.  The method's own
random draws (initial canvas, Gumbel noise, re-noise tokens) are not made here:
the oracle and the HIP library each implement the counter-based Philox4x32-10
generator themselves.

Shapes come from the five workloads of the denoise-step hot path.  The pages
(mlqm.cn summary of the DiffusionGemma report, sections 二 and 五) only fix the
256-token canvas, 128 experts with 8 active and a ~262k vocabulary; every other
size below is a stand-in chosen for the workload, not a figure from the pages.

Weights are N(0, 0.02) in a fixed per-tensor seeding, stored either as float32
or as bfloat16 bit patterns (numpy uint16, round-to-nearest-even from the
float32 draw).  Norm gains default to ones.  Matrices use the [out, in] layout
(the input dimension is contiguous), which is the layout the library takes.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

__all__ = [
    "ModelConfig", "SamplerConfig", "Workload", "WORKLOADS", "workload",
    "WeightSet", "make_weights", "make_prompts", "request_seeds",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
]

STOP_NONE, STOP_MEAN, STOP_PAGES = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    ffn_hidden: int
    top_k: int
    vocab: int
    dtype: str            # "f32" or "bf16": storage type of weights and matmul operands
    self_cond: bool
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    canvas_len: int = 256
    expert_dtype: str = ""   # "" = dtype; "fp8": experts served as OCP FP8 E4M3 with per-channel scales
    head_dtype: str = ""     # "" = dtype; "fp8": the LM head reads E as OCP FP8 E4M3 with one scale per id

    def n_params(self) -> int:
        d, L = self.d_model, self.n_layers
        per_layer = (d * self.n_q_heads * self.head_dim * 2
                     + d * self.n_kv_heads * self.head_dim * 2
                     + d * self.n_experts
                     + 3 * self.n_experts * d * self.ffn_hidden)
        return self.vocab * d + (d * d if self.self_cond else 0) + L * per_layer


@dataclasses.dataclass(frozen=True)
class SamplerConfig:
    max_steps: int
    entropy_bound: float
    stop_mode: int = STOP_NONE
    stop_tau: float = 0.0
    t_start: float = 0.8
    t_end: float = 0.4
    top_k: int = 0           # 0: the full vocabulary; k: top-k truncated sampling


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    sampler: SamplerConfig
    prompt_len: int
    batch: int
    canvases: int
    seed: int


_TINY = ModelConfig(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                    n_experts=8, ffn_hidden=512, top_k=2, vocab=2048, dtype="f32",
                    self_cond=False)
_SMALL = ModelConfig(n_layers=4, d_model=1024, n_q_heads=16, n_kv_heads=4, head_dim=64,
                     n_experts=32, ffn_hidden=1024, top_k=4, vocab=32768, dtype="bf16",
                     self_cond=True)
_PROXY = ModelConfig(n_layers=30, d_model=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                     n_experts=128, ffn_hidden=768, top_k=8, vocab=262144, dtype="bf16",
                     self_cond=True)

WORKLOADS: Dict[str, Workload] = {
    # 1 layer fp32 model; 12 steps, bound 0.5 nats, no stop, no self-conditioning.
    "tiny": Workload("tiny", _TINY, SamplerConfig(12, 0.5), prompt_len=32, batch=1,
                     canvases=1, seed=0),
    # 4 layer bf16 model, self-conditioning on; 24 steps, no stop rule given.
    "small": Workload("small", _SMALL, SamplerConfig(24, 0.1), prompt_len=512, batch=1,
                      canvases=1, seed=1),
    # 30 layer bf16 proxy at the reported expert count and vocabulary.
    "proxy": Workload("proxy", _PROXY, SamplerConfig(48, 0.1, STOP_MEAN, 0.05),
                      prompt_len=2048, batch=1, canvases=1, seed=2),
    # Block-autoregressive: four canvases after an 8192-token prompt, small model.
    "multicanvas": Workload("multicanvas", _SMALL, SamplerConfig(48, 0.1, STOP_MEAN, 0.05),
                            prompt_len=8192, batch=1, canvases=4, seed=1),
    # 32 concurrent requests with 4096-token prompts, small model.
    "batched": Workload("batched", _SMALL, SamplerConfig(48, 0.1, STOP_MEAN, 0.05),
                        prompt_len=4096, batch=32, canvases=1, seed=1),
    # The proxy and small workloads with their experts served in FP8 (the same
    # seeded bf16 weights, quantised per output channel by the model).
    "proxy-fp8": Workload("proxy-fp8", dataclasses.replace(_PROXY, expert_dtype="fp8"),
                          SamplerConfig(48, 0.1, STOP_MEAN, 0.05), prompt_len=2048, batch=1, canvases=1, seed=2),
    "small-fp8": Workload("small-fp8", dataclasses.replace(_SMALL, expert_dtype="fp8"), SamplerConfig(24, 0.1),
                          prompt_len=512, batch=1, canvases=1, seed=1),
    # The same with the LM head's rows of E in FP8 as well (the model served in FP8).
    "proxy-fp8-head": Workload("proxy-fp8-head", dataclasses.replace(_PROXY, expert_dtype="fp8", head_dtype="fp8"),
                               SamplerConfig(48, 0.1, STOP_MEAN, 0.05), prompt_len=2048, batch=1, canvases=1, seed=2),
    "small-fp8-head": Workload("small-fp8-head", dataclasses.replace(_SMALL, expert_dtype="fp8", head_dtype="fp8"),
                               SamplerConfig(24, 0.1), prompt_len=512, batch=1, canvases=1, seed=1),
    # Top-k truncated sampling (k = 8) on the proxy and on the batched shape.
    "proxy-topk": Workload("proxy-topk", _PROXY, SamplerConfig(48, 0.1, STOP_MEAN, 0.05, top_k=8),
                           prompt_len=2048, batch=1, canvases=1, seed=2),
    "batched-topk": Workload("batched-topk", _SMALL, SamplerConfig(48, 0.1, STOP_MEAN, 0.05, top_k=8),
                             prompt_len=4096, batch=32, canvases=1, seed=1),
}


def workload(name: str, **overrides) -> Workload:
    """Named workload, optionally with top-level fields replaced (prompt_len, batch ...)."""
    w = WORKLOADS[name]
    return dataclasses.replace(w, **overrides) if overrides else w


# ---------------------------------------------------------------- bf16 storage

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- weights

_KIND = {"emb": 0, "w_sc": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5, "w_router": 6,
         "w_gate": 7, "w_up": 8, "w_down": 9, "attn_norm": 10, "ffn_norm": 11,
         "final_norm": 12}
WEIGHT_STD = 0.02


def tensor_list(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """Canonical tensor order and shapes ([out, in] for every matrix).

    Expert matrices are stacked per layer: w_gate/w_up [E, F, d], w_down [E, d, F].
    Norm gains are float32 vectors in every dtype.
    """
    d, hd, E, F = cfg.d_model, cfg.head_dim, cfg.n_experts, cfg.ffn_hidden
    out = [("emb", (cfg.vocab, d))]
    if cfg.self_cond:
        out.append(("w_sc", (d, d)))
    out.append(("final_norm", (d,)))
    for l in range(cfg.n_layers):
        out += [
            (f"l{l}.attn_norm", (d,)),
            (f"l{l}.wq", (cfg.n_q_heads * hd, d)),
            (f"l{l}.wk", (cfg.n_kv_heads * hd, d)),
            (f"l{l}.wv", (cfg.n_kv_heads * hd, d)),
            (f"l{l}.wo", (d, cfg.n_q_heads * hd)),
            (f"l{l}.ffn_norm", (d,)),
            (f"l{l}.w_router", (E, d)),
            (f"l{l}.w_gate", (E, F, d)),
            (f"l{l}.w_up", (E, F, d)),
            (f"l{l}.w_down", (E, d, F)),
        ]
    return out


def _split(name: str) -> Tuple[int, str]:
    if name.startswith("l") and "." in name:
        head, kind = name.split(".", 1)
        return int(head[1:]), kind
    return -1, name


class WeightSet:
    """Lazily generated, optionally cached, seeded weights of one model.

    ``get(name)`` returns float32 (dtype "f32", and every norm gain) or uint16
    bfloat16 bits (dtype "bf16").  With ``cache=False`` each call regenerates the
    tensor, which keeps host memory bounded for the large proxy model.
    """

    def __init__(self, cfg: ModelConfig, seed: int, cache: bool = True,
                 gain_std: float = 0.0, threads: Optional[int] = None):
        self.cfg, self.seed, self.cache, self.gain_std = cfg, seed, cache, gain_std
        self.threads = threads or min(16, os.cpu_count() or 1)
        self._shapes = dict(tensor_list(cfg))
        self._store: Dict[str, np.ndarray] = {}

    def names(self) -> List[str]:
        return [n for n, _ in tensor_list(self.cfg)]

    def shape(self, name: str) -> Tuple[int, ...]:
        return self._shapes[name]

    def is_gain(self, name: str) -> bool:
        return name.endswith("_norm")

    def _normal(self, kind: str, layer: int, part: int, n: int) -> np.ndarray:
        ss = np.random.SeedSequence([self.seed, _KIND[kind], layer + 1, part + 1])
        return np.random.Generator(np.random.PCG64(ss)).standard_normal(n, dtype=np.float32)

    def _make(self, name: str) -> np.ndarray:
        layer, kind = _split(name)
        shape = self._shapes[name]
        if kind.endswith("_norm"):
            g = np.ones(shape, np.float32)
            if self.gain_std:
                g += np.float32(self.gain_std) * self._normal(kind, layer, 0, g.size)
            return g
        # one independent stream per expert slice (or per whole matrix), so the
        # large stacks can be filled by several threads
        parts = shape[0] if len(shape) == 3 else 1
        per = int(np.prod(shape)) // parts
        to_bf16 = self.cfg.dtype == "bf16"
        out = np.empty((parts, per), np.uint16 if to_bf16 else np.float32)

        def fill(p: int) -> None:
            v = self._normal(kind, layer, p, per)
            v *= np.float32(WEIGHT_STD)
            out[p] = f32_to_bf16_bits(v) if to_bf16 else v

        if parts > 1 and self.threads > 1:
            with ThreadPoolExecutor(self.threads) as ex:
                list(ex.map(fill, range(parts)))
        else:
            for p in range(parts):
                fill(p)
        return out.reshape(shape)

    def get(self, name: str) -> np.ndarray:
        if name in self._store:
            return self._store[name]
        arr = self._make(name)
        if self.cache:
            self._store[name] = arr
        return arr

    def scale_by_power_of_two(self, name: str, exponent: int) -> None:
        """Multiply one cached tensor by 2^exponent (exact in fp32 and bf16 while in range)."""
        assert self.cache, "scaling needs the cached weights"
        arr = self.get(name)
        f = bf16_bits_to_f32(arr) if arr.dtype == np.uint16 else arr
        f = np.ldexp(f, exponent).astype(np.float32)
        self._store[name] = f32_to_bf16_bits(f) if arr.dtype == np.uint16 else f

    def items(self) -> Iterator[Tuple[str, np.ndarray]]:
        for n in self.names():
            yield n, self.get(n)

    def nbytes(self) -> int:
        tot = 0
        for n, s in tensor_list(self.cfg):
            el = 4 if (self.is_gain(n) or self.cfg.dtype == "f32") else 2
            tot += el * int(np.prod(s))
        return tot


def make_weights(cfg: ModelConfig, seed: int, cache: bool = True,
                 gain_std: float = 0.0) -> WeightSet:
    return WeightSet(cfg, seed, cache=cache, gain_std=gain_std)


def make_prompts(vocab: int, batch: int, length: int, seed: int) -> np.ndarray:
    """Prompt token ids int32 [batch, length], uniform over the vocabulary."""
    out = np.empty((batch, length), np.int32)
    for b in range(batch):
        ss = np.random.SeedSequence([seed, 100, b])
        out[b] = np.random.Generator(np.random.PCG64(ss)).integers(0, vocab, size=length)
    return out


def request_seeds(seed: int, batch: int) -> np.ndarray:
    """Per-request 64-bit Philox seeds: high word = workload seed, low word = request index."""
    return (np.uint64(seed) << np.uint64(32)) | np.arange(batch, dtype=np.uint64)
