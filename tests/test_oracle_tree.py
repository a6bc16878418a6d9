"""Pins of the oracle's top-N tree (steps 1-2) against hand-worked cases, brute
force, an independent best-first search, and the structural facts the pages fix
(paper §3.2 Assumption 1 and Def. 1; project page "Verify pass")."""
import heapq
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import draft, round as orr, tree as tr
from synth import gen_round, make_config
from tests.golden import parse_paths, read_cases


def _logq_from_probs(rows):
    with np.errstate(divide="ignore"):
        z = np.log(np.array(rows, dtype=np.float64))
    return draft.log_softmax(z)


# ------------------------------------------------------------------ golden cases
@pytest.mark.parametrize("case", read_cases("tree_cases.txt"), ids=lambda c: c["name"])
@pytest.mark.parametrize("how", ["brute", "beam"])
def test_hand_worked_trees(case, how):
    logq = _logq_from_probs(case["q"])
    N = int(case["N"][0])
    fn = tr.brute_force_top_n if how == "brute" else tr.level_beam_top_n
    top, scores, nxt = fn(logq, N)
    assert set(top) == set(parse_paths(case["set"]))
    parent, depth, token, anc, n_valid, order = tr.canonical_layout(top, 77, N)
    exp_tok = [77 if t == "R" else int(t) for t in case["token"]]
    assert parent.tolist() == [int(x) for x in case["parent"]]
    assert depth.tolist() == [int(x) for x in case["depth"]]
    assert token.tolist() == exp_tok
    assert n_valid == len(top) + 1
    want_next = float(case["next"][0])
    if want_next == 0.0:
        assert nxt == -np.inf
    else:
        assert np.exp(nxt) == pytest.approx(want_next, rel=1e-12)


# ------------------------------------------------------------ structural facts
def _check_tree_facts(top, scores, logq, N):
    L, V = logq.shape
    S = set(top)
    assert len(S) == len(top)
    n_finite = sum(int(np.isfinite(logq[:d]).all(axis=1).prod()) for d in range(1, L + 1))
    assert len(top) == N or len(top) < N
    for p in top:
        assert 1 <= len(p) <= L
        assert p[:-1] == () or p[:-1] in S          # prefix-closed (Def. 1)
        # Lemma T: a depth-d member's token ranks within the top N-d+1 of q_d
        d = len(p)
        order = tr.token_ranking(logq[d - 1], V)
        rank = int(np.flatnonzero(order == p[-1])[0]) + 1
        assert rank <= N - d + 1
        # score is the depth-order log-sum of the marginals (plug-in score)
        assert np.exp(scores[p]) == pytest.approx(np.prod([np.exp(logq[j, t]) for j, t in enumerate(p)]),
                                                  rel=1e-9)
    del n_finite


def _micro_logq(rng, L, V, kind):
    if kind == "normal":
        z = rng.standard_normal((L, V)) * 2.0
    elif kind == "uniform":
        z = np.zeros((L, V))
    elif kind == "ties":
        z = rng.integers(0, 3, size=(L, V)).astype(np.float64)
    elif kind == "spiky":
        z = rng.standard_normal((L, V))
        z[np.arange(L), rng.integers(0, V, L)] += 40.0
    elif kind == "neginf":
        z = rng.standard_normal((L, V))
        z[rng.random((L, V)) < 0.4] = -np.inf
        z[:, 0] = np.where(np.isfinite(z[:, 0]), z[:, 0], 0.0)
    return draft.log_softmax(z)


@pytest.mark.parametrize("V,L", [(2, 4), (3, 3), (8, 3), (8, 4), (16, 3), (16, 4)])
@pytest.mark.parametrize("kind", ["normal", "uniform", "ties", "spiky", "neginf"])
def test_brute_force_equals_beam_micro(V, L, kind):
    rng = np.random.default_rng(V * 100 + L * 10 + len(kind))
    for N in (1, 5, 15, 31, 63):
        logq = _micro_logq(rng, L, V, kind)
        a = tr.brute_force_top_n(logq, N)
        b = tr.level_beam_top_n(logq, N)
        assert a[0] == b[0]                       # same members in the same >- order
        assert a[2] == b[2] or (np.isinf(a[2]) and np.isinf(b[2]))
        _check_tree_facts(a[0], a[1], logq, N)


def test_brute_force_counts_every_prefix():
    # V=3, L=3: 3 + 9 + 27 = 39 prefixes, all finite; N = 39 keeps every one and
    # N = 40 cannot exceed them.
    logq = draft.log_softmax(np.random.default_rng(5).standard_normal((3, 3)))
    top, _, nxt = tr.brute_force_top_n(logq, 39)
    assert set(top) == set(p for d in (1, 2, 3) for p in itertools.product(range(3), repeat=d))
    assert nxt == -np.inf
    top40, _, _ = tr.brute_force_top_n(logq, 40)
    assert len(top40) == 39


def _heap_top_n(logq, N):
    """Independent best-first search (test only): pop the best frontier prefix,
    push its next sibling and its first child.  Key: (-score, depth, pop index of
    the parent, token rank), which orders prefixes like >- on the oracle side."""
    L, V = logq.shape
    ranks = [tr.token_ranking(logq[j], V) for j in range(L)]
    out = []
    heap = []
    if len(ranks[0]):
        heap.append((-logq[0, ranks[0][0]], 1, -1, 0, (), 0.0))
    while heap and len(out) < N:
        negs, d, ppop, r, ppath, pscore = heapq.heappop(heap)
        path = ppath + (int(ranks[d - 1][r]),)
        me = len(out)
        out.append(path)
        if r + 1 < len(ranks[d - 1]):
            sib = pscore + logq[d - 1, ranks[d - 1][r + 1]]
            heapq.heappush(heap, (-sib, d, ppop, r + 1, ppath, pscore))
        if d < L and len(ranks[d]):
            kid = -negs + logq[d, ranks[d][0]]
            heapq.heappush(heap, (-kid, d + 1, me, 0, path, -negs))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_beam_equals_best_first_large(seed):
    rng = np.random.default_rng(seed)
    V, L = 3000, 15
    z = rng.standard_normal((L, V)) * [0.5, 1, 2, 3, 4, 6][seed]
    logq = draft.log_softmax(z)
    for N in (15, 31, 63):
        top, scores, _ = tr.level_beam_top_n(logq, N)
        assert set(top) == set(_heap_top_n(logq, N))
        _check_tree_facts(top, scores, logq, N)


@pytest.mark.parametrize("seed", [1000, 1001])
def test_tiny_config_brute_force(seed):
    """The tiny workload (V=256, L=4, N=15): enumeration of all 4,311,810,304
    prefixes agrees with the beam."""
    inp = gen_round(make_config("tiny"), seed, with_model=False)
    z = inp["rounds"][0]["draft_logits"][0]
    a = orr.build_tree(z, "f32", 0, 15, "brute")
    b = orr.build_tree(z, "f32", 0, 15, "beam")
    assert a["top"] == b["top"]
    assert a["next_score"] == b["next_score"]
    for k in ("parent", "depth", "token", "anc"):
        assert np.array_equal(a[k], b[k])


# ------------------------------------------------------------- layout facts
@pytest.mark.parametrize("seed", range(5))
def test_canonical_layout_facts(seed):
    rng = np.random.default_rng(seed)
    logq = draft.log_softmax(rng.standard_normal((15, 500)) * 3)
    top, _, _ = tr.level_beam_top_n(logq, 63)
    parent, depth, token, anc, n_valid, order = tr.canonical_layout(top, 9, 63)
    assert n_valid == 64 and parent[0] == -1 and anc[0] == 1
    for i in range(1, 64):
        assert parent[i] < i                                   # parents first
        assert depth[i] == depth[parent[i]] + 1
        assert anc[i] == anc[parent[i]] | (np.uint64(1) << np.uint64(i))
        if i > 1:  # rows sorted by (depth, parent row, token)
            assert (depth[i - 1], parent[i - 1], token[i - 1]) < (depth[i], parent[i], token[i])
    # bit j of anc[i] <=> row j's path is a prefix of row i's path
    for i in range(64):
        for j in range(64):
            bit = bool(int(anc[i]) >> j & 1)
            assert bit == (order[i][:len(order[j])] == order[j])
    assert tr.paths_from_layout(parent, token, n_valid) == order[1:]


# ------------------------------------------------------------- log-softmax pins
def test_log_softmax_matches_scipy():
    rng = np.random.default_rng(3)
    for scale in (1e-3, 1.0, 30.0, 1e4):
        z = rng.standard_normal((7, 1001)) * scale
        np.testing.assert_allclose(draft.log_softmax(z), scipy.special.log_softmax(z, axis=-1),
                                   rtol=1e-12, atol=1e-12)
    z = rng.standard_normal((3, 50))
    z[0, :10] = -np.inf
    a, b = draft.log_softmax(z), scipy.special.log_softmax(z, axis=-1)
    assert np.array_equal(np.isinf(a), np.isinf(b))
    np.testing.assert_allclose(a[np.isfinite(a)], b[np.isfinite(b)], rtol=1e-12)


def test_log_softmax_closed_forms():
    V = 151936
    lq = draft.log_softmax(np.zeros((1, V)))
    assert np.allclose(lq, -np.log(V), rtol=0, atol=1e-12)
    assert draft.entropy_nats(lq)[0] == pytest.approx(np.log(V), abs=1e-9)  # 11.9312
    assert np.log(V) == pytest.approx(11.9312, abs=1e-4)
    lq = draft.log_softmax(np.array([[0.0, 0.0, -1e4, -1e4]]))
    assert draft.entropy_nats(lq)[0] == pytest.approx(np.log(2), abs=1e-12)
    lq = draft.log_softmax(np.array([[50.0, -50.0, -50.0]]))
    assert draft.entropy_nats(lq)[0] == pytest.approx(0.0, abs=1e-40)
    rng = np.random.default_rng(0)
    lq = draft.log_softmax(rng.standard_normal((5, 100)) * 4)
    np.testing.assert_allclose(np.exp(lq).sum(axis=1), 1.0, rtol=1e-13)


def test_c2_scales_span_draft_entropy_range():
    """The single-layer 8B sweep's draft scales give mean draft entropies that
    fall monotonically from about 6 nats to about 0.1 (the workload recipe)."""
    from synth.gen import C2_SCALES
    rng = np.random.default_rng(11)
    g = rng.standard_normal((15, 151936))
    H = [draft.entropy_nats(draft.log_softmax(g * s)).mean() for s in C2_SCALES]
    assert 5.5 < H[0] < 6.5
    assert H[-1] < 0.3
    assert all(a > b for a, b in zip(H, H[1:]))
