"""Pins of the shared-budget allocation (paper App. B.5, Proposition 4: under a
shared budget the best allocation takes the globally highest node masses, each
round's masses indexed by its V(H)) against its definition written out by
enumeration, the fixed-width tree it reduces to, and the monotone facts the
definition implies."""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import round as orr, shared as sh, tree as tr


def _random_logqs(rng, nseq, L, V):
    return [scipy.special.log_softmax(rng.normal(0, 1.5, (L, V)), axis=1) for _ in range(nseq)]


def _enumerate(logqs, log_weight, B, n_max, tau):
    """The definition: every prefix of every round with its key, best first
    (continuous random inputs have no ties), taken while the round has fewer
    than n_max nodes, the batch fewer than B, and the key is at least tau."""
    entries = []
    for s, logq in enumerate(logqs):
        L, V = logq.shape
        for d in range(1, L + 1):
            for p in itertools.product(range(V), repeat=d):
                sc = sum(logq[j, t] for j, t in enumerate(p))
                entries.append((log_weight[s] + sc, s, p))
    entries.sort(key=lambda e: -e[0])
    sets = [set() for _ in logqs]
    taken = 0
    for key, s, p in entries:
        if taken == B or key < tau:
            break
        if len(sets[s]) < n_max:
            sets[s].add(p)
            taken += 1
    return sets


@pytest.mark.parametrize("seed", range(6))
def test_allocation_matches_enumeration(seed):
    rng = np.random.default_rng(seed)
    nseq, L, V = 3, 3, 4
    logqs = _random_logqs(rng, nseq, L, V)
    w = rng.normal(0, 1.0, nseq)
    for B, n_max, tau in [(10, 6, -np.inf), (7, 10, -np.inf), (20, 8, -np.inf), (12, 9, -4.0)]:
        n, gap, _ = sh.allocate(logqs, w, B, n_max, tau)
        want = _enumerate(logqs, w, B, n_max, tau)
        assert n.tolist() == [len(x) for x in want], (B, n_max, tau)
        assert gap > 0
        for s, logq in enumerate(logqs):
            top, _, _ = tr.level_beam_top_n(logq, n_max)
            assert set(top[:n[s]]) == want[s]
            # and the brute-force variant of the oracle agrees
        bf = sh.brute_force_allocate(logqs, w, B, n_max, tau)
        assert [set(x) for x in bf] == want


def test_equal_weights_and_full_budget_give_fixed_width_trees():
    rng = np.random.default_rng(7)
    nseq, L, V, N = 4, 4, 6, 9
    stored = [rng.normal(0, 2.0, (L, V)).astype(np.float32) for _ in range(nseq)]
    roots = [11, 12, 13, 14]
    trees, n, _, _ = sh.build_trees(stored, "f32", roots, np.zeros(nseq), nseq * N, N)
    assert n.tolist() == [N] * nseq
    for s in range(nseq):
        ref = orr.build_tree(stored[s], "f32", roots[s], N)
        for k in ("parent", "depth", "token", "anc"):
            assert np.array_equal(trees[s][k], ref[k]), k
        assert trees[s]["n_valid"] == ref["n_valid"]


def test_weights_move_the_budget_monotonically():
    rng = np.random.default_rng(3)
    logqs = _random_logqs(rng, 3, 3, 5)
    base = np.zeros(3)
    n0, _, _ = sh.allocate(logqs, base, 15, 12)
    for delta in (0.5, 1.0, 3.0):
        w = base.copy()
        w[1] += delta
        n1, _, _ = sh.allocate(logqs, w, 15, 12)
        assert n1[1] >= n0[1] and n1[0] <= n0[0] and n1[2] <= n0[2]
        assert n1.sum() == n0.sum() == 15
    # a round of zero value gets nothing; the others share the whole budget
    w = np.array([0.0, -np.inf, 0.0])
    n2, _, _ = sh.allocate(logqs, w, 15, 12)
    assert n2[1] == 0 and n2.sum() == 15


def test_threshold_stops_allocation():
    rng = np.random.default_rng(5)
    logqs = _random_logqs(rng, 2, 3, 4)
    n, _, _ = sh.allocate(logqs, np.zeros(2), 30, 20, tau=1.0)   # every key is <= 0
    assert n.tolist() == [0, 0]
    n_all, _, _ = sh.allocate(logqs, np.zeros(2), 30, 20)
    n_cut, _, _ = sh.allocate(logqs, np.zeros(2), 30, 20, tau=-3.0)
    assert np.all(n_cut <= n_all) and n_cut.sum() < n_all.sum()
    trees, n0, _, _ = sh.build_trees([np.zeros((3, 4), np.float32)] * 2, "f32", [1, 2],
                                     np.zeros(2), 10, 8, tau=1.0)
    assert n0.tolist() == [0, 0]
    for t in trees:   # the root alone
        assert t["n_valid"] == 1 and t["parent"][0] == -1 and np.all(t["token"][1:] == -1)


def test_equal_keys_go_to_the_lower_round():
    rng = np.random.default_rng(9)
    logq = _random_logqs(rng, 1, 3, 4)[0]
    n, _, _ = sh.allocate([logq, logq.copy()], np.zeros(2), 5, 10)
    assert n.tolist() == [3, 2]
