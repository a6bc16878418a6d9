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


# --------------------------------------------------------------- entropy keying
# ln V(H) of the entropy law (paper §6 Eq. 2, App. B and B.5 Eq. 5), pinned to
# closed forms that a dropped term, a sign or a wrong horizon breaks.

def test_log_value_at_half_match_probability():
    # H = b0 / b1 gives p_m = 1/2: E[a|H] = 1 - 2^-L, V = (1 - 2^-L) / 2
    b0, b1 = 0.96, 0.63
    for L in (1, 2, 15):
        got = sh.log_value(b0 / b1, b0, b1, L)
        assert got == pytest.approx(np.log((1 - 2.0 ** -L) / 2), abs=1e-13)


def test_log_value_one_offset_and_infinite_horizon():
    rng = np.random.default_rng(3)
    b0, b1 = 1.226, 0.95
    H = rng.uniform(0.0, 8.0, 50)
    x = b0 - b1 * H
    # L = 1: V = p (1 - p) = sigma(x) sigma(-x)
    want1 = -np.logaddexp(0.0, -x) - np.logaddexp(0.0, x)
    assert np.allclose(sh.log_value(H, b0, b1, 1), want1, atol=1e-12)
    # long horizon: E[a|H] -> p / (1 - p), so V -> p = sigma(x)
    want_inf = -np.logaddexp(0.0, -x)
    assert np.allclose(sh.log_value(H, b0, b1, 400), want_inf, atol=1e-9)


def test_log_value_peaks_at_intermediate_entropy():
    # Prop. 4: small when acceptance is hopeless (large H) or already deep
    # (H -> 0, with a horizon long enough that 1 - p_m dominates), largest in
    # between; the truncated value p (1 - p^L) peaks where p = (L + 1)^(-1/L)
    b0, b1, L = 6.0, 1.0, 15
    H = np.linspace(0.0, 12.0, 4801)
    v = sh.log_value(H, b0, b1, L)
    i = int(np.argmax(v))
    assert 0 < i < len(H) - 1
    p_star = (L + 1.0) ** (-1.0 / L)
    H_star = (b0 - np.log(p_star / (1 - p_star))) / b1
    assert abs(H[i] - H_star) < 2 * (H[1] - H[0])
    assert np.all(np.diff(v[:i]) >= 0) and np.all(np.diff(v[i:]) <= 0)
    # large H: ln V ~ ln p ~ b0 - b1 H
    assert sh.log_value(40.0, b0, b1, L) == pytest.approx(b0 - b1 * 40.0, abs=1e-9)


def test_log_value_special_inputs():
    assert sh.log_value(np.nan, 0.96, 0.63, 15) == -np.inf
    assert np.isfinite(sh.log_value(0.0, 0.96, 0.63, 15))
    # a huge entropy: p itself would underflow, ln V still follows b0 - b1 H
    assert sh.log_value(1e4, 0.96, 0.63, 15) == pytest.approx(0.96 - 0.63e4, abs=1e-9)


def test_log_value_matches_the_plain_product_where_it_is_representable():
    # the log-domain steps equal ln( (sum_l p^l) (1 - p) ) computed directly
    rng = np.random.default_rng(9)
    b0, b1, L = 0.96, 0.63, 15
    H = rng.uniform(0.0, 20.0, 200)
    p = 1.0 / (1.0 + np.exp(-(b0 - b1 * H)))
    plain = np.log(sum(p ** l for l in range(1, L + 1)) * (1.0 - p))
    assert np.allclose(sh.log_value(H, b0, b1, L), plain, rtol=1e-12, atol=1e-12)
