"""Oracle sampler: temperature schedule, head statistics, commit / re-noise / stop.

Pages followed ([mlqm] = mlqm.cn summary of the DiffusionGemma report):
  * [mlqm] 四: positions are ordered by entropy from low to high and locked from
    the most certain one on, until the running entropy total passes the
    threshold (0.1); the positions past it are re-randomised and revised next
    round.  The temperature starts at 0.8 and falls linearly to 0.4.  Generation
    stops early once the mean entropy is below 0.005 and the most likely token
    sequence is unchanged over two consecutive rounds, within a 48-round cap.
  * [mlqm] 一: multinomial (uniform replacement) diffusion: an uncertain position
    is replaced by any vocabulary token, and a locked token stays revisable.
  * [chooseai] (llama.cpp support paragraph): the entropy-bounded denoising
    sampler with linear temperature 0.8 -> 0.4 and adaptive stop.

Readings where the pages leave a step open:
  * entropy is in nats, of the tempered distribution softmax(l / T);
  * the sort is stable: equal entropies keep position order;
  * the position whose addition makes the running total exceed the bound is not
    committed; a committed position takes the sampled token y (Gumbel-max draw);
  * the schedule runs over the step budget S: T_t = T0 + (T1 - T0) * t / (S - 1);
  * stop mode 1 is "mean entropy < tau"; mode 2 adds the pages' unchanged-argmax
    condition; on the stopping step and on the last step every position takes y.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import philox

STOP_NONE, STOP_MEAN, STOP_PAGES = 0, 1, 2


def temperature(t: int, max_steps: int, t_start: float = 0.8, t_end: float = 0.4) -> np.float32:
    """Linear schedule over the step budget, evaluated in fp64 from the fp32 parameters."""
    t0 = float(np.float32(t_start))
    t1 = float(np.float32(t_end))
    if max_steps <= 1:
        return np.float32(t0)
    return np.float32(t0 + (t1 - t0) * float(t) / float(max_steps - 1))


def inv_temperature(T: np.float32) -> np.float32:
    return np.float32(1.0 / float(T))


def gumbel_call_of(v: np.ndarray):
    """(counter word 0, output word) of vocabulary id v in the GUMBEL stream.

    Each aligned group of 64 ids is served by 16 Philox calls: id v takes output
    word (v >> 4) & 3 of the call whose first counter word is 16 * (v >> 6) + (v & 15),
    so ids c, c + 16, c + 32, c + 48 of a group share one call.
    """
    v = np.asarray(v, np.int64)
    return (((v >> 6) << 4) | (v & 15)), ((v >> 4) & 3)


def gumbel_block(seed: int, canvas: int, step: int, pos: np.ndarray, vocab: int) -> np.ndarray:
    """Gumbel noise g[len(pos), vocab] (fp32) of the GUMBEL stream at one step."""
    pos = np.asarray(pos, np.int64)
    call, word = gumbel_call_of(np.arange(vocab))
    ncall = int(call.max()) + 1
    ctr = np.empty((pos.size, ncall, 4), np.uint32)
    ctr[..., 0] = np.arange(ncall, dtype=np.uint32)[None, :]
    ctr[..., 1] = pos.astype(np.uint32)[:, None]
    ctr[..., 2] = np.uint32(step)
    ctr[..., 3] = np.uint32((philox.TAG_GUMBEL << 24) | (canvas & 0xFFFFFF))
    out = philox.philox4x32_10(ctr, philox.seed_key(seed))          # [pos, call, 4]
    return philox.gumbel(out[:, call, word])


def head_stats(logits: np.ndarray, inv_t: np.float32, seed: int, canvas: int, step: int,
               pos: np.ndarray, want_probs: bool = False, chunk: int = 16) -> Dict[str, np.ndarray]:
    """Per-row statistics of the tempered distribution and the Gumbel-max draw.

    logits: fp32 [n, V].  z = logits * (1/T) in fp32.  Returns
      H      entropy of softmax(z) in nats (fp64 evaluation, fp32 result)
      am     argmax of the logits (lowest id on ties)
      y      argmax_v (z_v + g_v) with fp32 scores (lowest id on ties)
      margin best minus second-best perturbed score (fp32)
      m, logS  max of z and log of sum exp(z - m)  (fp64)
      p      softmax(z) (fp64), only if want_probs
    """
    logits = np.asarray(logits, np.float32)
    n, V = logits.shape
    out = {k: np.empty(n, t) for k, t in
           (("H", np.float32), ("am", np.int32), ("y", np.int32), ("margin", np.float32),
            ("m", np.float64), ("logS", np.float64))}
    probs = np.empty((n, V), np.float64) if want_probs else None
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        z = logits[r0:r1] * np.float32(inv_t)                         # fp32
        z64 = z.astype(np.float64)
        m = z64.max(axis=1, keepdims=True)
        e = np.exp(z64 - m)
        S = e.sum(axis=1, keepdims=True)
        H = np.log(S[:, 0]) - (e * (z64 - m)).sum(axis=1) / S[:, 0]
        out["H"][r0:r1] = H.astype(np.float32)
        out["m"][r0:r1] = m[:, 0]
        out["logS"][r0:r1] = np.log(S[:, 0])
        out["am"][r0:r1] = np.argmax(logits[r0:r1], axis=1)
        g = gumbel_block(seed, canvas, step, pos[r0:r1], V)
        score = z + g                                                 # fp32
        y = np.argmax(score, axis=1)
        best = score[np.arange(r1 - r0), y]
        masked = score.copy()
        masked[np.arange(r1 - r0), y] = -np.inf
        out["y"][r0:r1] = y
        out["margin"][r0:r1] = best - masked.max(axis=1)
        if want_probs:
            probs[r0:r1] = e / S
    if want_probs:
        out["p"] = probs
    return out


def gumbel_of_ids(seed: int, canvas: int, step: int, pos: int, ids: np.ndarray) -> np.ndarray:
    """Gumbel noise (fp32) of the given vocabulary ids at one position, from the GUMBEL stream."""
    ids = np.asarray(ids, np.int64)
    call, word = gumbel_call_of(ids)
    ctr = np.empty((ids.size, 4), np.uint32)
    ctr[:, 0] = call.astype(np.uint32)
    ctr[:, 1] = np.uint32(pos)
    ctr[:, 2] = np.uint32(step)
    ctr[:, 3] = np.uint32((philox.TAG_GUMBEL << 24) | (canvas & 0xFFFFFF))
    out = philox.philox4x32_10(ctr, philox.seed_key(seed))
    return philox.gumbel(out[np.arange(ids.size), word])


def head_stats_topk(logits: np.ndarray, inv_t: np.float32, top_k: int, seed: int, canvas: int, step: int,
                    pos: np.ndarray, want_probs: bool = False, forced_ids=None) -> Dict[str, np.ndarray]:
    """Head statistics of the distribution truncated to the top_k largest logits of each row.

    [mlqm] 九: top-k truncation of the vocabulary at high batch (named as an
    optimisation not yet built).  Reading: the usual top-k sampling -- the k
    largest logits of a position (ties to the lower id) keep their softmax
    weights renormalised over the k, every other id has probability 0.  The
    entropy, the Gumbel-max draw (over the k ids, each with its own Gumbel
    word of the GUMBEL stream), the top-2 margin and the self-conditioning
    vector all use that distribution; the argmax is the largest logit as
    before.  Returns H, am, y, margin like head_stats, the selected ids (in
    descending logit order) and, if asked, their probabilities (fp64).

    forced_ids [n, top_k] (tests only): where a row's entry is given, that id
    set replaces the row's own selection (a caller that has shown the two sets
    to be a near-tie at the k-th logit); it is ordered by descending logit,
    ties to the lower id, and everything else follows as above.
    """
    logits = np.asarray(logits, np.float32)
    n, V = logits.shape
    out = {k: np.empty(n, t) for k, t in
           (("H", np.float32), ("am", np.int32), ("y", np.int32), ("margin", np.float32))}
    out["ids"] = np.empty((n, top_k), np.int64)
    if want_probs:
        out["p"] = np.empty((n, top_k))
    for r in range(n):
        order = np.argsort(-logits[r], kind="stable")[:top_k]       # descending, ties -> lower id
        if forced_ids is not None and forced_ids[r] is not None:
            ids = np.asarray(forced_ids[r], np.int64)
            order = ids[np.lexsort((ids, -logits[r, ids]))]
        z = logits[r, order] * np.float32(inv_t)                        # fp32
        z64 = z.astype(np.float64)
        m = z64.max()
        e = np.exp(z64 - m)
        S = e.sum()
        out["H"][r] = np.float32(np.log(S) - (e * (z64 - m)).sum() / S)
        out["am"][r] = order[0]
        score = z + gumbel_of_ids(seed, canvas, step, int(pos[r]), order)   # fp32
        best = max(range(top_k), key=lambda j: (score[j], -order[j]))   # ties -> lower id
        out["y"][r] = order[best]
        rest = [score[j] for j in range(top_k) if j != best]
        out["margin"][r] = np.float32(score[best] - max(rest)) if rest else np.float32(np.inf)
        out["ids"][r] = order
        if want_probs:
            out["p"][r] = e / S
    return out


def commit(H: np.ndarray, y: np.ndarray, am: np.ndarray, prev_am: Optional[np.ndarray],
           canvas: np.ndarray, step: int, max_steps: int, entropy_bound: float,
           stop_mode: int, stop_tau: float, seed: int, canvas_index: int, vocab: int):
    """One request's commit / re-noise / stop decision.

    Returns (new_canvas int32[n], mask uint8[n], n_committed, done).
    """
    H = np.asarray(H, np.float32)
    n = H.size
    pos = np.arange(n)
    order = np.lexsort((pos, H))              # entropy ascending, then position
    bound = float(np.float32(entropy_bound))
    mask = np.zeros(n, np.uint8)
    total = 0.0
    for i in order:
        total += float(H[i])
        if total <= bound:
            mask[i] = 1
        else:
            break
    mean = 0.0
    for i in range(n):
        mean += float(H[i])
    mean /= n
    tau = float(np.float32(stop_tau))
    stop = False
    if stop_mode == STOP_MEAN:
        stop = mean < tau
    elif stop_mode == STOP_PAGES:
        stop = (mean < tau and prev_am is not None and step > 0
                and bool(np.all(np.asarray(am) == np.asarray(prev_am))))
    final = stop or step >= max_steps - 1
    if final:
        return np.asarray(y, np.int32).copy(), np.ones(n, np.uint8), n, True
    w = philox.words(seed, philox.TAG_RENOISE, canvas_index, step, pos, 0)
    fresh = philox.uniform_token(w, vocab)
    new = np.where(mask == 1, np.asarray(y, np.int32), fresh).astype(np.int32)
    return new, mask, int(mask.sum()), False


def init_canvas(seed: int, canvas_index: int, n: int, vocab: int) -> np.ndarray:
    """Initial canvas: n uniformly random tokens ([mlqm] 一: the canvas starts as random words)."""
    w = philox.words(seed, philox.TAG_INIT, canvas_index, 0, np.arange(n), 0)
    return philox.uniform_token(w, vocab)
