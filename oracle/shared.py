"""Shared-budget width allocation over a batch of rounds (test infrastructure only).

Paper App. B.5 (Proposition 4 and its proof): across rounds under a shared
verifier budget, the allocation that maximises the total expected committed
length is global best-first over node masses, each round's masses indexed by
its value V(H) (Eq. 5), until the marginal mass falls below the exchange rate.

Reading used here.  Round s (one sequence of the batch) gives its prefixes the
key  omega_s + sum_j log q_j(y_j),  with omega_s = ln V(H_s) (``log_value``:
the law's fitted constants b0, b1 and the horizon L are inputs, and the
entropy H_s of each round's root comes with the round), and
  * the budget B is the total number of tree nodes over the batch,
  * every round keeps at most n_max nodes (its verify rows),
  * a node whose key is below tau (the stopping rule, in log units) or -inf is
    never taken.
The batch takes the B highest keys; equal keys go to the lower round index,
and within a round prefixes follow the order of the fixed-width tree (module
doc of oracle.tree), in which every ancestor precedes its descendants.  Within a
round the keys are non-increasing in that order, so each round keeps a prefix
of it: its own top-n_s set, which is prefix-closed.
"""
from __future__ import annotations

import numpy as np

from . import draft, tree as tr
from .numerics import decode


def log_match_probability(H, b0: float, b1: float):
    """ln p_m(H) and ln(1 - p_m(H)) with p_m(H) = sigma(b0 - b1 H): the law's
    affine match logit (paper §6, Eq. 2; project page "An Entropy Law of
    Draftability"), in logs so that no entropy underflows them."""
    x = b0 - b1 * np.asarray(H, dtype=np.float64)
    with np.errstate(invalid="ignore"):  # a NaN entropy stays NaN here
        return -np.logaddexp(0.0, -x), -np.logaddexp(0.0, x)


def log_expected_accept(H, b0: float, b1: float, L: int):
    """ln E[a | H] with E[a | H] ~ sum_{l=1}^{L} p_m^l, the survival sum truncated
    at the block horizon L (paper App. B, the slowly varying step; project page,
    the same sum in closed form)."""
    lnp, _ = log_match_probability(H, b0, b1)
    with np.errstate(invalid="ignore"):  # NaN entropies stay NaN
        return np.logaddexp.reduce(np.stack([l * lnp for l in range(1, L + 1)]), axis=0)


def log_value(H, b0: float, b1: float, L: int):
    """ln V(H) with V(H) = E[a | H] (1 - p_m(H)) (paper App. B.5, Eq. 5: the
    round's marginal value of width, up to a constant factor that is the same
    for every round and so leaves the allocation unchanged).  A NaN entropy
    gives -inf (the round receives no width)."""
    H = np.asarray(H, dtype=np.float64)
    _, ln1mp = log_match_probability(H, b0, b1)
    v = log_expected_accept(H, b0, b1, L) + ln1mp
    return np.where(np.isnan(H), -np.inf, v)


def allocate(logqs, log_weight, B: int, n_max: int, tau: float = -np.inf):
    """Node counts n_s of the batch (logqs: per round [L][V] float64 log q).
    Also returns the boundary gap: the B-th taken key minus the best key left
    out (inf when nothing is left out), and the smallest distance of a
    candidate key to tau (inf without a threshold)."""
    cands = []
    for s, logq in enumerate(logqs):
        top, scores, _ = tr.level_beam_top_n(logq, n_max)
        for i, p in enumerate(top):
            key = float(log_weight[s]) + scores[p]
            cands.append((key, s, i))
    ok = [c for c in cands if c[0] > -np.inf and c[0] >= tau]
    ok.sort(key=lambda c: (-c[0], c[1], c[2]))
    taken = ok[:B]
    n = np.zeros(len(logqs), dtype=np.int64)
    for _, s, _ in taken:
        n[s] += 1
    gap = (taken[-1][0] - ok[B][0]) if (len(ok) > B and B > 0) else np.inf
    tmargin = min((abs(c[0] - tau) for c in cands if c[0] > -np.inf), default=np.inf) \
        if tau > -np.inf else np.inf
    return n, gap, tmargin


def brute_force_allocate(logqs, log_weight, B: int, n_max: int, tau: float = -np.inf):
    """The same counts from the definition on tiny shapes: every prefix of every
    round, ordered by (key desc, round, the round's own prefix order), the first
    B admissible ones, each round capped at n_max."""
    entries = []
    for s, logq in enumerate(logqs):
        top, scores, _ = tr.brute_force_top_n(logq, n_max)
        for i, p in enumerate(top):
            entries.append((float(log_weight[s]) + scores[p], s, i, p))
    entries = [e for e in entries if e[0] > -np.inf and e[0] >= tau]
    entries.sort(key=lambda e: (-e[0], e[1], e[2]))
    chosen = entries[:B]
    sets = [[] for _ in logqs]
    for _, s, _, p in chosen:
        sets[s].append(p)
    return sets


def build_trees(drafts_stored, dtype: str, roots, log_weight, B: int, n_max: int,
                tau: float = -np.inf):
    """Steps 1-2 under the shared budget: every round's tree (its top-n_s set
    laid out as the fixed-width tree with n_max + 1 rows), the counts and the
    boundary gaps of ``allocate``."""
    logqs = [draft.log_softmax(decode(d, dtype)) for d in drafts_stored]
    n, gap, tmargin = allocate(logqs, log_weight, B, n_max, tau)
    trees = []
    for s, logq in enumerate(logqs):
        top, scores, nxt = tr.level_beam_top_n(logq, n_max)
        sel = top[:int(n[s])]
        parent, depth, token, anc, n_valid, order = tr.canonical_layout(sel, int(roots[s]), n_max)
        score = np.full(n_max + 1, -np.inf)
        score[0] = 0.0
        for i, p in enumerate(order[1:], start=1):
            score[i] = scores[p]
        # a round cut at its cap has its own boundary (its n_max-th node against
        # the next one); a cut by the budget or the threshold is the batch's
        own = (scores[top[-1]] - nxt) if (int(n[s]) == n_max and n_max > 0 and len(top) == n_max) \
            else np.inf
        trees.append({"logq": logq, "top": sel, "parent": parent, "depth": depth,
                      "token": token, "anc": anc, "score": score, "n_valid": n_valid,
                      "order": order, "boundary_gap": own})
    return trees, n, gap, tmargin
