"""Philox4x32-10 counter-based generator, oracle side (numpy, uint64 arithmetic).

Follows the generator's published definition: Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section on Philox.
State: a 4x32-bit counter and a 2x32-bit key.  Each of the ten rounds multiplies
counter words 0 and 2 by the two Philox multipliers, splits each 64-bit product
into high and low halves, and permutes/xors them with words 1 and 3 and the key;
between rounds the key is advanced by the two Weyl constants.

Stream layout (a choice of this project; the pages only say randomness drives
the initial canvas, the sampled tokens and the re-noising, [mlqm] sections 一, 四):
  key     = (low 32 bits of the request seed, high 32 bits of the request seed)
  counter = (j >> 2, position, step, tag << 24 | canvas index), output word j & 3
  tags: INIT (initial canvas, j = 0, step 0), RENOISE (j = 0), GUMBEL (one
        word per vocabulary id v, laid out per aligned group of 64 ids: counter
        word 0 = 16 * (v >> 6) + (v & 15), output word (v >> 4) & 3 -- see
        sampler.gumbel_call_of)
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)

TAG_INIT = 2
TAG_GUMBEL = 3
TAG_RENOISE = 4


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Apply Philox4x32 with 10 rounds.

    ctr: uint32 array [..., 4]; key: uint32 array [..., 2] (broadcast against ctr).
    Returns uint32 [..., 4].
    """
    ctr = np.asarray(ctr, dtype=np.uint32)
    key = np.asarray(key, dtype=np.uint32)
    x = [ctr[..., i].astype(np.uint64) for i in range(4)]
    k0 = key[..., 0].astype(np.uint64)
    k1 = key[..., 1].astype(np.uint64)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    w0, w1 = np.uint64(PHILOX_W0), np.uint64(PHILOX_W1)
    for _ in range(10):
        p0 = x[0] * m0            # exact: both factors < 2**32
        p1 = x[2] * m1
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        x = [hi1 ^ x[1] ^ k0, lo1, hi0 ^ x[3] ^ k1, lo0]
        k0 = (k0 + w0) & _MASK
        k1 = (k1 + w1) & _MASK
    return np.stack([np.broadcast_to(v, np.broadcast(*x).shape) for v in x],
                    axis=-1).astype(np.uint32)


def seed_key(seed: int) -> np.ndarray:
    s = int(seed) & 0xFFFFFFFFFFFFFFFF
    return np.array([s & 0xFFFFFFFF, s >> 32], dtype=np.uint32)


def words(seed: int, tag: int, canvas: int, step: int, pos: np.ndarray,
          j: np.ndarray) -> np.ndarray:
    """Raw 32-bit draws for (position, inner index j) pairs; pos and j broadcast."""
    pos = np.asarray(pos, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    pos, j = np.broadcast_arrays(pos, j)
    ctr = np.empty(pos.shape + (4,), np.uint32)
    ctr[..., 0] = (j >> 2).astype(np.uint32)
    ctr[..., 1] = pos.astype(np.uint32)
    ctr[..., 2] = np.uint32(step)
    ctr[..., 3] = np.uint32(((tag & 0xFF) << 24) | (canvas & 0xFFFFFF))
    out = philox4x32_10(ctr, seed_key(seed))
    return np.take_along_axis(out, (j & 3)[..., None], axis=-1)[..., 0]


def uniform01(x: np.ndarray) -> np.ndarray:
    """float32 uniform in (0, 1): (2 * (x >> 9) + 1) * 2**-24, exact in fp32."""
    k = (np.asarray(x, dtype=np.uint32) >> np.uint32(9)).astype(np.float64)
    return ((2.0 * k + 1.0) * 2.0 ** -24).astype(np.float32)


def gumbel(x: np.ndarray) -> np.ndarray:
    """Standard Gumbel draw -log(-log(u)), evaluated in fp64, rounded to fp32."""
    u = uniform01(x).astype(np.float64)
    return (-np.log(-np.log(u))).astype(np.float32)


def uniform_token(x: np.ndarray, vocab: int) -> np.ndarray:
    """Token id in [0, vocab): floor(x * vocab / 2**32); exactly uniform for power-of-two vocab."""
    return ((np.asarray(x, dtype=np.uint64) * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)
