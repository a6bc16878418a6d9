"""Chained rounds on the device (commit + advance after every walk) against the
oracle's plain autoregressive greedy decoding (paper Theorem 1, App. B.1): the
committed token stream must equal the greedy stream, compared up to the
reference's first near-tie (top-2 gap <= 1e-3, where bf16 arithmetic may pick
the other token).  Drafts favour the greedy stream so rounds accept several
tokens; the device keeps the prefix length and the root itself between rounds."""
import numpy as np
import pytest
import torch

from oracle import model as mdl, walk as wk
from tests.chain import agreed_prefix, chained_workload, favoured_draft

pytestmark = pytest.mark.gpu

GAP = 1e-3


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,seed,R,over,packed", [
    ("tiny_widehead", 11, 8, {}, False),
    ("mini_bf16", 6, 6, {"head_std": 4.0}, False),  # smallest top-2 gap of the reference: 0.69
    # the 8B shapes with the packed head and attention weights, as the benchmark
    # runs them; the reference's 48 greedy tokens all have top-2 gaps >= 0.0126.
    # At these random weights the greedy stream settles on one repeated token
    # after two, so this case pins the chained path at full size, and
    # test_commit_appends_the_path_rows pins the committed cache rows exactly
    ("qwen8b_1layer", 8, 3, {}, True),
])
def test_device_rounds_equal_greedy_decoding(name, seed, R, over, packed):
    from tree_verified_block_amd.round import DeviceRound
    cfg, inp = chained_workload(name, seed, R, **over)
    model = mdl.TargetModel(inp, cache_head=cfg.V > 100000)
    b = int(inp["rounds"][0]["root"][0])
    G, gaps = wk.greedy_stream(model, 0, b, R * (cfg.L + 1))
    P = int(inp["prefix_len"][0])
    dev = DeviceRound(inp, capacity=P + (R + 1) * (cfg.L + 1), packed_head=packed)
    rng = np.random.default_rng(seed + 100)
    stream = [b]
    dev.set_draft(favoured_draft(cfg, G, 0, rng), root=b)
    accepted = []
    for r in range(R):
        dev.run()
        dev.commit()
        torch.cuda.synchronize()
        a = int(dev.n_accept[0])
        toks = dev.out_tokens[0, :a + 1].cpu().tolist()
        accepted.append(a)
        stream += [int(x) for x in toks]
        print(f"[chain] {name} round {r}: A={a} tokens={toks}", flush=True)
        # the device advanced its own prefix end and root
        assert int(dev.kv_offsets[1]) == P + len(stream) - 1
        assert int(dev.root[0]) == stream[-1]
        dev.set_draft(favoured_draft(cfg, G, len(stream) - 1, rng))
    n = min(len(stream) - 1, agreed_prefix(gaps, GAP))
    print(f"[chain] {name}: {len(stream) - 1} tokens committed, {n} compared, accepted {accepted}", flush=True)
    assert n >= 2 * (cfg.L + 1) or n == len(stream) - 1
    assert stream[1:n + 1] == G[:n]
    assert sum(accepted) > R


@pytest.mark.parametrize("name,over", [("mini_bf16", {"n_layers": 3, "head_std": 4.0}),
                                       ("tiny_widehead", {})])
def test_commit_appends_the_path_rows(name, over):
    """glance_commit_kv, checked bit for bit: after a round, cache rows P .. P + A
    of every layer hold the K and V entries that the verify pass wrote for the
    walk's path rows (the root, then the accepted nodes in path order), the rows
    after them are untouched, and the next round's prefix starts past them."""
    from tree_verified_block_amd.round import DeviceRound
    seed, R = 6, 2
    cfg, inp = chained_workload(name, seed, R, **over)
    model = mdl.TargetModel(inp)
    b = int(inp["rounds"][0]["root"][0])
    G, _ = wk.greedy_stream(model, 0, b, R * (cfg.L + 1))
    P0 = int(inp["prefix_len"][0])
    dev = DeviceRound(inp, capacity=P0 + (R + 1) * (cfg.L + 1))
    rng = np.random.default_rng(seed + 7)
    dev.set_draft(favoured_draft(cfg, G, 0, rng), root=b)
    n_done = 0
    for r in range(R):
        P = int(dev.kv_offsets[1])
        dev.run()
        torch.cuda.synchronize()
        a = int(dev.n_accept[0])
        path = dev.path_rows[0, :a + 1].cpu().numpy()
        assert path[0] == 0 and np.all(np.diff(path) > 0)
        before = [(lw["k_cache"].clone(), lw["v_cache"].clone()) for lw in dev.layers]
        tk = [t.clone() for t in dev.tree_ks]
        tv = [t.clone() for t in dev.tree_vs]
        dev.commit()
        torch.cuda.synchronize()
        for li, lw in enumerate(dev.layers):
            kc, vc = lw["k_cache"], lw["v_cache"]
            idx = torch.as_tensor(path, dtype=torch.long, device=kc.device)
            assert torch.equal(kc[P:P + a + 1], tk[li][idx]), (r, li)
            assert torch.equal(vc[P:P + a + 1], tv[li][idx]), (r, li)
            assert torch.equal(kc[:P], before[li][0][:P]) and torch.equal(vc[:P], before[li][1][:P])
            assert torch.equal(kc[P + a + 1:], before[li][0][P + a + 1:])
            assert torch.equal(vc[P + a + 1:], before[li][1][P + a + 1:])
        assert int(dev.kv_offsets[1]) == P + a + 1
        n_done += a + 1
        dev.set_draft(favoured_draft(cfg, G, n_done, rng))
