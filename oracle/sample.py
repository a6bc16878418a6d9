"""Sampling at temperature T (test infrastructure only).

Paper §5.4 (Table 3) and App. D: under sampling the committed token is drawn
from the target's own verified row, so the output distribution is the target's.
Reading used here: every verify row draws one token from softmax(z / T) by the
Gumbel-max rule, y = argmax_v (z_v / T + G_v) with G_v = -ln(-ln U_v), and the
accept walk then runs on the drawn tokens in place of the argmax.  Each row's
draw uses its own counter-based stream, so it is independent of the path that
reaches the row, and the committed tokens are draws from the target's
conditionals.

U_v comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011): key (seed low, seed high 32 bits),
counter (v / 4, row, round low, round high), output word v % 4, and
U = (x / 2^9 (integer part) + 1/2) / 2^23 from the word's top 23 bits.  The
numerator 2 k + 1 has at most 24 bits, so U is exact in float32 as in float64
and never 0 or 1.  (A 24-bit grid is not exact in float32 above 1/2: U there
rounds, 1 - U loses most of its bits where the winning draws live, and the
last grid point rounds to 1, whose noise is infinite.)
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57   # the round multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85   # the key increments (golden ratio, sqrt(3) - 1)
MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds on arrays: ctr [..][4], key [2] (uint32 values).
    Returns [..][4] uint32.  Round: (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0,
    lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key grows by (W0, W1) before
    every round but the first."""
    c = [np.asarray(ctr[..., i], dtype=np.uint64) for i in range(4)]
    k0, k1 = int(key[0]) & MASK, int(key[1]) & MASK
    for r in range(10):
        if r > 0:
            k0, k1 = (k0 + W0) & MASK, (k1 + W1) & MASK
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK)
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return np.stack(c, axis=-1).astype(np.uint32)


def uniforms(seed: int, rnd: int, row: int, V: int) -> np.ndarray:
    """U_v for v < V of one verify row, float64 in (0, 1)."""
    n = (V + 3) // 4
    ctr = np.zeros((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n, dtype=np.uint64)
    ctr[:, 1] = row
    ctr[:, 2] = rnd & MASK
    ctr[:, 3] = (rnd >> 32) & MASK
    x = philox4x32_10(ctr, (seed & MASK, (seed >> 32) & MASK)).reshape(-1)[:V]
    return ((x >> np.uint32(9)).astype(np.float64) + 0.5) / 8388608.0


def sample_rows(z: np.ndarray, T: float, seed: int, rnd: int, rows=None):
    """The drawn token of every row of logits z [n][V] at temperature T, and the
    gap between the best and second-best perturbed score of each row (how far
    the draw is from a tie).  Equal perturbed scores: the lowest token id.
    ``rows``: the verify-row index of each row of z (its stream; default 0..n-1)."""
    z = np.asarray(z, dtype=np.float64)
    rows = np.arange(z.shape[0]) if rows is None else np.asarray(rows)
    tok = np.empty(z.shape[0], dtype=np.int64)
    gap = np.empty(z.shape[0])
    for i in range(z.shape[0]):
        g = -np.log(-np.log(uniforms(seed, rnd, int(rows[i]), z.shape[1])))
        s = z[i] / T + g
        tok[i] = int(np.argmax(s))
        top = np.partition(s, -2)[-2:]
        gap[i] = top[1] - top[0]
    return tok, gap
