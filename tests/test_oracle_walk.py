"""Pins of the oracle's walk and accepted length (step 5) against hand-worked
cases, Definition 1 itself, and whole rounds whose answer is fixed by
construction (paper §3.1-§3.2 Def. 1, Eq. (1); App. B.1)."""
import numpy as np
import pytest

from oracle import round as orr, tree as tr, walk as wk
from synth import gen_round, make_config
from tests.golden import parse_paths, read_cases


@pytest.mark.parametrize("case", read_cases("walk_cases.txt"), ids=lambda c: c["name"])
def test_hand_worked_walks(case):
    parent = [int(x) for x in case["parent"]]
    token = [int(x) for x in case["token"]]
    argmax = [int(x) for x in case["argmax"]]
    a, toks, rows = wk.walk(parent, token, len(parent), argmax, int(case["L"][0]))
    assert a == int(case["a"][0])
    assert toks == [int(x) for x in case["tokens"]]
    assert rows == [int(x) for x in case["rows"]]
    assert all(argmax[r] == t for r, t in zip(rows, toks))  # each token is a row argmax


@pytest.mark.parametrize("case", read_cases("accept_cases.txt"), ids=lambda c: c["name"])
def test_accepted_length_definition(case):
    S = set(parse_paths(case.get("set", [])))
    Y = [int(x) for x in case["Y"]]
    assert wk.accepted_length(Y, S) == int(case["A"][0])


@pytest.mark.parametrize("seed", range(40))
def test_walk_equals_definition_on_random_trees(seed):
    """For any prefix-closed tree and any greedy target (a function from prefixes
    to tokens), the walk over rows commits exactly Y_{1:A(S)} plus Y_{A+1}."""
    rng = np.random.default_rng(seed)
    V, L = int(rng.integers(2, 6)), int(rng.integers(1, 6))
    N = int(rng.integers(0, 20))
    root = 0
    parent, depth, token, anc = _random_tree(rng, N, L, V)
    n_valid = len(parent)
    order = [()] + tr.paths_from_layout(parent, token, n_valid)
    table = {}

    def target(prefix):  # greedy token after root o prefix (fixed at random)
        if prefix not in table:
            table[prefix] = int(rng.integers(0, V))
        return table[prefix]

    argmax = [target(p) for p in order]
    a, toks, rows = wk.walk(parent, token, n_valid, argmax, L)
    Y = []
    while True:
        Y.append(target(tuple(Y)))
        if tuple(Y) not in set(order[1:]):
            break
    A = wk.accepted_length(Y, set(order[1:]))
    assert a == A and toks == Y[:A + 1]
    assert [order[r] for r in rows] == [tuple(Y[:k]) for k in range(A + 1)]


def _random_tree(rng, N, L, V):
    from synth.gen import random_tree
    maxn = sum(V ** d for d in range(1, L + 1))
    return random_tree(rng, min(N, maxn), L, V, 0)


def test_empty_tree_commits_one_token():
    """N = 0: the tree is the root alone, A = 0 and the one committed token is
    the root row's argmax, so tau = 1 (paper Eq. (1))."""
    inp = gen_round(make_config("tiny", N=0), 1000)
    res = orr.oracle_round(inp, 0)[0]
    assert res["tree"]["n_valid"] == 1
    assert res["walk"]["a"] == 0 and res["greedy"]["A"] == 0
    assert res["walk"]["tokens"] == [int(res["rows"]["argmax"][0])]
    assert res["greedy"]["Y"] == res["walk"]["tokens"]


@pytest.mark.parametrize("name,seed", [("tiny", 1000), ("tiny", 1001), ("tiny_widehead", 1000),
                                       ("tiny_widehead", 1001), ("tiny_widehead", 1002)])
def test_walk_over_rows_equals_independent_decode(name, seed):
    """The walk over the verify rows and the independent greedy decode give the
    same A(S) and tokens on every round whose visited rows are not near-ties."""
    inp = gen_round(make_config(name), seed)
    res = orr.oracle_round(inp, 0)[0]
    w, g = res["walk"], res["greedy"]
    if not (w["flagged"] or g["flagged"]):
        assert w["a"] == g["A"]
        assert w["tokens"] == g["Y"][:g["A"] + 1]
    # every committed token is the argmax of its row, on every round
    assert all(res["rows"]["argmax"][r] == t for r, t in zip(w["rows"], w["tokens"]))


def test_widehead_rounds_are_mostly_unflagged():
    flagged = 0
    for seed in range(1000, 1006):
        res = orr.oracle_round(gen_round(make_config("tiny_widehead"), seed), 0)[0]
        flagged += res["walk"]["flagged"]
    assert flagged <= 2


def test_copy_regime_accepts_planted_run():
    """Copy regime: the head is biased so that the greedy continuation follows a
    planted run of G tokens and then breaks; the draft puts >= 0.9 mass on the
    run, so A(S) = G and the new root is the break token."""
    inp = gen_round(make_config("mini_bf16_copy"), 3)
    for r, rd in enumerate(inp["rounds"]):
        res = orr.oracle_round(inp, r)[0]
        G = rd["G"]
        chain = tuple(int(t) for t in rd["planted"][:G])
        assert chain == () or chain in set(res["tree"]["top"])
        assert res["greedy"]["A"] == G
        assert res["greedy"]["new_root"] == rd["break_token"]
        assert res["walk"]["a"] == G
