"""Training-side forward pass: uniform corruption of a clean canvas and the denoising loss.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/.

Pages followed ([mlqm] = mlqm.cn summary of the DiffusionGemma report):
  * [mlqm] 一: in training a proportion of a sequence's tokens, anywhere from
    0% to 100%, is replaced by random vocabulary tokens, and the model learns
    to restore the original (multinomial diffusion: corruption is uniform
    replacement, not masking).

Readings where the pages leave a step open:
  * each position of request b is replaced independently with probability
    rate_b; a replaced position takes a uniform vocabulary token (which may be
    the clean token again).  Draws: one Philox call per position, tag CORRUPT,
    counter (0, position, 0, CORRUPT << 24 | canvas index); word 0 gives the
    uniform u (replace iff u < rate_b, compared in fp32), word 1 the token;
  * the model sees the corrupted canvas exactly as a denoising round sees its
    canvas (after the request's context, bidirectional attention over it) with
    no self-conditioning term;
  * the loss is the cross-entropy of the clean token under softmax(logits)
    (temperature 1, nats) at every canvas position, CE_i = logsumexp(l_i) -
    l_i[x0_i], and a request's loss is the mean over its positions.
"""
from __future__ import annotations

import numpy as np

from . import numerics as nm
from . import philox

TAG_CORRUPT = 5


def corrupt(clean: np.ndarray, rate: float, seed: int, canvas_index: int, vocab: int):
    """One request's corrupted canvas and the replaced positions."""
    clean = np.asarray(clean, np.int32)
    n = clean.size
    pos = np.arange(n)
    u = philox.uniform01(philox.words(seed, TAG_CORRUPT, canvas_index, 0, pos, 0))
    tok = philox.uniform_token(philox.words(seed, TAG_CORRUPT, canvas_index, 0, pos, 1), vocab)
    replaced = u < np.float32(rate)
    return np.where(replaced, tok, clean).astype(np.int32), replaced


def logsumexp(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    m = x.max(axis=-1)
    return m + np.log(np.exp(x - m[..., None]).sum(axis=-1))


def forward_loss(model, clean: np.ndarray, rates, seeds, want_logits: bool = False) -> dict:
    """Corrupt each request's clean canvas [B, n], run the model over it and score the clean tokens.

    Returns corrupted [B, n], replaced [B, n], ce [B, n] (fp64), loss [B] (fp64)
    and, optionally, the logits [B, n, V]."""
    cfg = model.cfg
    B, n = np.asarray(clean).shape
    out = {"corrupted": np.zeros((B, n), np.int32), "replaced": np.zeros((B, n), bool),
           "ce": np.zeros((B, n)), "loss": np.zeros(B)}
    if want_logits:
        out["logits"] = np.zeros((B, n, cfg.vocab))
    pos = model.ctx + np.arange(n)
    for b in range(B):
        x, rep = corrupt(clean[b], float(rates[b]), int(seeds[b]), model.canvas_index, cfg.vocab)
        out["corrupted"][b], out["replaced"][b] = x, rep
        h = model._stack(b, x, pos, False, False, None, None)
        xf = model.rnd(nm.rmsnorm(h, model.W("final_norm"), cfg.rms_eps))
        logits = xf @ model.head_weight().T
        ce = logsumexp(logits) - logits[np.arange(n), np.asarray(clean[b])]
        out["ce"][b] = ce
        out["loss"][b] = ce.mean()
        if want_logits:
            out["logits"][b] = logits
    return out
