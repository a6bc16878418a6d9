"""Top-N prefix-closed candidate tree (test infrastructure only).

Definition (paper §3.2, Def. 1; §4.2; project page "Verify pass"): the candidate
tree S is the set of the N prefixes y_{1:d} (1 <= d <= L) with the highest
plug-in score pi(y_{1:d}) = prod_{j<=d} q_j(y_j) (Assumption 1).  The oracle ranks
by the float64 log score sum_{j<=d} log q_j(y_j), accumulated in depth order.

The pages leave ties open.  The order used here, written >-, compares two
prefixes by
    1. higher score first,
    2. then smaller depth,
    3. then (same depth) the parent that comes first under >-,
    4. then (same parent) the smaller token id.
Every ancestor precedes its descendants (log q <= 0), so the first N prefixes
under >- are prefix-closed even when scores tie.

Two ways to compute the set, which must agree:
  * ``brute_force_top_n`` enumerates every prefix (the definition itself);
  * ``level_beam_top_n`` keeps the top-N prefixes of each depth, extending the
    previous depth's top-N by the N best tokens of q_d.  A depth-d member of the
    top-N of all depth-d prefixes has its parent in the depth-(d-1) top-N and its
    last token in the top-N of q_d, so nothing is lost.

``canonical_layout`` emits the verify rows: row 0 is the root b, rows 1..|S|
sorted by (depth, parent row, token id), which depends only on the set.
"""
from __future__ import annotations

import itertools

import numpy as np

_CHUNK = 1 << 16


def order_prefixes(scores: dict) -> list:
    """Sort a prefix-closed {path tuple: score} dict under >- (module doc)."""
    by_depth: dict = {}
    for p in scores:
        by_depth.setdefault(len(p), []).append(p)
    rank = {(): 0}
    for d in sorted(by_depth):
        items = by_depth[d]
        for p in items:
            if p[:-1] not in rank:
                raise ValueError("candidate set is not prefix-closed")
        items.sort(key=lambda p: (-scores[p], rank[p[:-1]], p[-1]))
        for i, p in enumerate(items):
            rank[p] = i
    return sorted(scores, key=lambda p: (-scores[p], len(p), rank[p]))


def _depth_chunks(logq: np.ndarray, d: int, leads=None):
    """Yield (lead, block) covering every depth-d prefix once: ``lead`` holds the
    first k tokens and ``block`` (a reused buffer) the float64 scores of all
    V**(d-k) completions, each accumulated in depth order
    ((log q_1 + log q_2) + log q_3) + ...; k is the smallest split that keeps a
    block under _CHUNK entries.  ``leads`` restricts the walk to given leads."""
    L, V = logq.shape
    k = 0
    while V ** (d - k) > _CHUNK:
        k += 1
    tail = d - k
    buf = np.empty((V,) * tail, dtype=np.float64)
    if leads is None:
        leads = itertools.product(range(V), repeat=k)
    for lead in leads:
        s = np.float64(0.0)
        for j, t in enumerate(lead):
            s = s + logq[j, t]
        np.copyto(buf, (s + logq[k]).reshape((V,) + (1,) * (tail - 1)))
        for j in range(1, tail):
            sh = [1] * tail
            sh[j] = V
            np.add(buf, logq[k + j].reshape(sh), out=buf)
        yield tuple(lead), buf.reshape(-1)


def brute_force_top_n(logq: np.ndarray, N: int):
    """Top-N prefixes by exhaustive enumeration of all V + V**2 + ... + V**L.

    Returns (paths in >- order, {path: score}, next_score) where next_score is the
    score of the (N+1)-th prefix under >- (-inf if there is none).  Prefixes with
    a -inf score are never selected."""
    logq = np.asarray(logq, dtype=np.float64)
    L, V = logq.shape
    M = N + 1
    # pass 1: the M largest scores (as a multiset of values)
    best = np.empty(0)
    mask = np.empty(min(V ** L, _CHUNK), dtype=bool)
    chunk_max = {}
    for d in range(1, L + 1):
        for lead, blk in _depth_chunks(logq, d):
            chunk_max[(d, lead)] = blk.max()
            m = mask[: blk.size]
            if best.size >= M:
                np.greater(blk, best[-1], out=m)
            else:
                np.isfinite(blk, out=m)
            sel = blk[np.flatnonzero(m)]
            if sel.size:
                if sel.size > M:
                    sel = np.partition(sel, sel.size - M)[sel.size - M:]
                best = np.sort(np.concatenate([best, sel]))[::-1][:M]
    best = best[np.isfinite(best)]
    if best.size == 0:
        return [], {}, -np.inf
    T = best[-1]
    # pass 2: every prefix scoring >= T (a prefix-closed superset of the answer);
    # blocks whose maximum, recorded in pass 1, is below T hold none of them
    cand: dict = {}
    for d in range(1, L + 1):
        keep = [ld for (dd, ld), mx in chunk_max.items() if dd == d and mx >= T]
        for lead, blk in _depth_chunks(logq, d, keep):
            m = mask[: blk.size]
            np.greater_equal(blk, T, out=m)
            idx = np.flatnonzero(m)
            tail = d - len(lead)
            for flat in idx:
                rest = np.unravel_index(int(flat), (V,) * tail) if tail else ()
                p = lead + tuple(int(t) for t in rest)
                cand[p] = float(blk[flat])
    ordered = order_prefixes(cand)
    top = ordered[:N]
    nxt = cand[ordered[N]] if len(ordered) > N else -np.inf
    return top, {p: cand[p] for p in top}, nxt


def token_ranking(logq_row: np.ndarray, n: int) -> np.ndarray:
    """The n best tokens of one marginal, by (log q desc, token id asc),
    finite values only."""
    v = np.arange(logq_row.size)
    order = np.lexsort((v, -logq_row))
    order = order[np.isfinite(logq_row[order])]
    return order[:n]


def level_beam_top_n(logq: np.ndarray, N: int):
    """Top-N prefixes through per-depth top-N beams (same result as the brute
    force; see module doc).  Same return values as ``brute_force_top_n``."""
    logq = np.asarray(logq, dtype=np.float64)
    L, V = logq.shape
    M = N + 1
    levels = []          # per depth: list of (path, score) sorted by >- within depth
    prev = [((), 0.0)]
    for d in range(1, L + 1):
        toks = token_ranking(logq[d - 1], M)
        cands = []
        for pr, (p, s) in enumerate(prev):
            for t in toks:
                cands.append((p + (int(t),), s + logq[d - 1, t], pr))
        cands.sort(key=lambda c: (-c[1], c[2], c[0][-1]))
        cur = [(p, s) for p, s, _ in cands[:M]]
        if not cur:
            break
        levels.append(cur)
        prev = cur
    scores = {p: s for lvl in levels for p, s in lvl}
    ordered = order_prefixes(scores)
    top = ordered[:N]
    nxt = scores[ordered[N]] if len(ordered) > N else -np.inf
    return top, {p: scores[p] for p in top}, nxt


def canonical_layout(paths, root_token: int, N: int):
    """Verify-row layout of a prefix-closed set of paths.

    Row 0 is the root b; rows 1..|S| are the nodes sorted by depth, then by the
    row of their parent, then by token id.  Returns int32 parent, depth, token
    and uint64 anc arrays of N+1 rows plus n_valid = |S| + 1; rows past n_valid
    are padding (parent -1, depth 0, token -1, anc 0).  Bit j of anc[i] is set
    iff row j is row i itself or one of its ancestors; the root is an ancestor of
    every row."""
    paths = list(paths)
    by_depth: dict = {}
    for p in paths:
        by_depth.setdefault(len(p), []).append(p)
    row = {(): 0}
    order = [()]
    for d in sorted(by_depth):
        items = sorted(by_depth[d], key=lambda p: (row[p[:-1]], p[-1]))
        for p in items:
            row[p] = len(order)
            order.append(p)
    R = N + 1
    parent = np.full(R, -1, dtype=np.int32)
    depth = np.zeros(R, dtype=np.int32)
    token = np.full(R, -1, dtype=np.int32)
    anc = np.zeros(R, dtype=np.uint64)
    token[0] = root_token
    anc[0] = np.uint64(1)
    for i, p in enumerate(order[1:], start=1):
        parent[i] = row[p[:-1]]
        depth[i] = len(p)
        token[i] = p[-1]
        anc[i] = anc[parent[i]] | (np.uint64(1) << np.uint64(i))
    return parent, depth, token, anc, len(order), order


def paths_from_layout(parent, token, n_valid):
    """Inverse of canonical_layout: the set of node paths (root excluded)."""
    paths = [()]
    for i in range(1, int(n_valid)):
        paths.append(paths[int(parent[i])] + (int(token[i]),))
    return paths[1:]
