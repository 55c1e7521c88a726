"""Elementary numerics of the oracle (fp64), each written from its plain definition.

Readings taken where the pages are silent (they give no formula for any layer;
[mlqm] section 二 only says the model is the Gemma 4 MoE transformer with causal
attention over the prompt and bidirectional attention over the canvas):
  * RMSNorm  y = x * g / sqrt(mean(x^2) + eps)
  * RoPE in rotate-half form: pairs (j, j + hd/2), angle = pos * theta^(-2j/hd)
  * scaled dot-product attention with scale 1/sqrt(hd), grouped-query sharing
    kv head floor(h * Hkv / Hq)
  * SwiGLU expert  W_down (silu(W_gate m) * W_up m)
  * bf16 models round matmul operands (normed activations, q/k/v, attention
    output, SwiGLU product, self-conditioning vector) to bf16, nearest-even
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as fp64.

    Works from the fp64 value directly: keep 8 significant bits.  Uses the
    float32 bit pattern of the fp64 value only after an exact split, so that no
    double rounding through float32 can occur.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    scaled = m * 256.0                      # 8 significant bits above the point
    r = np.round(scaled)                    # numpy rounds half to even
    return np.ldexp(r / 256.0, e)


def upcast(w: np.ndarray) -> np.ndarray:
    """Stored weight -> fp64: float32 as is, uint16 as bfloat16 bit patterns."""
    w = np.asarray(w)
    if w.dtype == np.uint16:
        return (w.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return w.astype(np.float64)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.  x: [n, heads, hd]; pos: [n] absolute positions."""
    n, _, hd = x.shape
    half = hd // 2
    freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, np.float64)[:, None] * freq[None, :]      # [n, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
              k_pos: np.ndarray, causal: bool) -> np.ndarray:
    """Grouped-query scaled dot-product attention, fp64.

    q: [nq, Hq, hd]; k, v: [nk, Hkv, hd]; q_pos, k_pos: absolute positions.
    Causal: query at position p sees keys at positions <= p.  Otherwise every
    query sees every key (the canvas is attended bidirectionally, [mlqm] 二).
    """
    nq, Hq, hd = q.shape
    Hkv = k.shape[1]
    out = np.empty((nq, Hq, hd), np.float64)
    scale = 1.0 / np.sqrt(hd)
    # Query rows are independent; they are evaluated in blocks to bound memory.
    # Under the causal mask a block needs only the keys up to its last position
    # (the others would get probability exactly 0).
    blk = 1024

    def head(h):
        g = (h * Hkv) // Hq
        for q0 in range(0, nq, blk):
            q1 = min(nq, q0 + blk)
            qp = q_pos[q0:q1]
            kmax = int(np.searchsorted(k_pos, qp.max(), side="right")) if causal else len(k_pos)
            s = (q[q0:q1, h, :] @ k[:kmax, g, :].T) * scale               # [block, keys]
            if causal:
                s = np.where(k_pos[None, :kmax] <= qp[:, None], s, -np.inf)
            out[q0:q1, h, :] = softmax(s, axis=-1) @ v[:kmax, g, :]

    # heads are independent; numpy releases the interpreter lock in these kernels
    if nq * len(k_pos) >= 1 << 20 and Hq > 1:
        with ThreadPoolExecutor(min(Hq, os.cpu_count() or 1)) as ex:
            list(ex.map(head, range(Hq)))
    else:
        for h in range(Hq):
            head(h)
    return out
