"""Theorem 1 of the paper (App. B.1), end to end on the oracle: rounds chained by
committing each round's accepted path reproduce plain autoregressive greedy
decoding token for token, whatever the drafts (here drafts that favour the
greedy stream, so that most rounds accept several tokens)."""
import numpy as np

from oracle import model as mdl, round as orr, walk as wk
from tests.chain import chained_workload, favoured_draft


def test_chained_oracle_rounds_equal_greedy_decoding():
    R = 8
    cfg, inp = chained_workload("tiny_widehead", 11, R)
    model = mdl.TargetModel(inp)
    b = int(inp["rounds"][0]["root"][0])
    G, gaps = wk.greedy_stream(model, 0, b, R * (cfg.L + 1))
    assert min(gaps) > 1e-6  # wide head: no near-tie in the reference stream
    rng = np.random.default_rng(5)
    stream, rounds = orr.multi_round(
        model, 0, b, lambda r, st: favoured_draft(cfg, G, len(st) - 1, rng)[0], R, cfg.dtype,
        cfg.N, cfg.L)
    assert stream[0] == b
    assert stream[1:] == G[:len(stream) - 1]
    accepted = [a for a, _ in rounds]
    assert len(stream) - 1 == sum(a + 1 for a in accepted)
    assert max(accepted) >= 2 and sum(accepted) > R  # several tokens per round


def test_chained_rounds_with_adversarial_drafts_commit_one_token_each():
    """Drafts that never contain the greedy token: every round accepts nothing and
    emits exactly the next greedy token (A = 0, one token per round)."""
    R = 4
    cfg, inp = chained_workload("tiny_widehead", 12, R)
    model = mdl.TargetModel(inp)
    b = int(inp["rounds"][0]["root"][0])
    G, _ = wk.greedy_stream(model, 0, b, R + 1)

    def draft(r, stream):
        z = np.zeros((cfg.L, cfg.V), dtype=np.float32)
        z[:, G[len(stream) - 1]] = -1e4  # the greedy token is never drafted at any offset
        return z

    stream, rounds = orr.multi_round(model, 0, b, draft, R, cfg.dtype, cfg.N, cfg.L)
    assert [a for a, _ in rounds] == [0] * R
    assert stream[1:] == G[:R]
