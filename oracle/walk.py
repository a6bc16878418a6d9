"""Greedy continuation, accepted length and the accept walk (test infrastructure only).

Paper §3.1: at temperature 0 the target's greedy continuation after the root b is
Y_k = argmax_w p(w | x o b o Y_{1:k-1}); a round commits a + 1 tokens.
Paper §3.2, Def. 1 (and the project page, "Verify pass"): the accepted length is
A(S) = max{k >= 0 : Y_{1:j} in S for all j <= k}; the walk commits Y_{1:A(S)} and
emits the next greedy token, read off the last verified row, as the new root.
Paper App. B.1 (proof of Theorem 1): at a verified prefix y_{1:k} the walk either
descends (y_{1:k} o Y_{k+1} in S: commit Y_{k+1}) or stops and emits Y_{k+1} as
the next root.
"""
from __future__ import annotations

import numpy as np

from .model import Decoder, TargetModel


def greedy_continuation(model: TargetModel, s: int, root: int, tree: set, L: int):
    """Decode Y_1, Y_2, .. from x o b by plain autoregression, stopping at the
    first k with Y_{1:k} not in the tree (k <= L + 1 since depths are <= L).
    Returns (Y as a list, the logits row of every decoded position)."""
    dec = Decoder(model, s)
    z = dec.extend(root)
    Y, rows = [], [z]
    while True:
        y = int(np.argmax(z))
        Y.append(y)
        if tuple(Y) not in tree or len(Y) > L:
            return Y, rows
        z = dec.extend(y)
        rows.append(z)


def accepted_length(Y, tree: set) -> int:
    """A(S) = max{k >= 0 : Y_{1:j} in S for every j <= k}, by set membership."""
    a = 0
    for k in range(1, len(Y) + 1):
        if all(tuple(Y[:j]) in tree for j in range(1, k + 1)):
            a = k
    return a


def walk(parent, token, n_valid: int, argmax_rows, L: int):
    """The accept walk over verify rows (root = row 0): at row r with greedy token
    y = argmax_rows[r], descend to the child of r carrying y and commit y, or stop
    and emit y as the new root.  Returns (a, tokens [a+1], rows [a+1]) where
    tokens[k] is the argmax of rows[k] and tokens[a] is the new root."""
    parent = np.asarray(parent)
    token = np.asarray(token)
    r, out, rows = 0, [], []
    while True:
        y = int(argmax_rows[r])
        out.append(y)
        rows.append(r)
        kids = [c for c in range(1, int(n_valid)) if parent[c] == r and token[c] == y]
        if not kids or len(out) > L:
            return len(out) - 1, out, rows
        r = kids[0]


def greedy_stream(model: TargetModel, s: int, root: int, n: int):
    """Plain autoregressive greedy decoding after x o b (paper §3.1, the
    temperature-0 reference that Theorem 1 says the method reproduces): the n
    tokens Y_1..Y_n, Y_k = argmax p(. | x o b o Y_{1:k-1}), with the top-2 logit
    gap of each step (how far each choice is from a tie)."""
    dec = Decoder(model, s)
    z = dec.extend(root)
    out, gaps = [], []
    for _ in range(n):
        y = int(np.argmax(z))
        top = np.partition(z, -2)[-2:]
        out.append(y)
        gaps.append(float(top[1] - top[0]))
        z = dec.extend(y)
    return out, gaps
