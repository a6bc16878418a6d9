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
@pytest.mark.parametrize("name,seed,R,over", [
    ("tiny_widehead", 11, 8, {}),
    ("mini_bf16", 6, 6, {"head_std": 4.0}),  # smallest top-2 gap of the reference: 0.69
])
def test_device_rounds_equal_greedy_decoding(name, seed, R, over):
    from tree_verified_block_amd.round import DeviceRound
    cfg, inp = chained_workload(name, seed, R, **over)
    model = mdl.TargetModel(inp)
    b = int(inp["rounds"][0]["root"][0])
    G, gaps = wk.greedy_stream(model, 0, b, R * (cfg.L + 1))
    P = int(inp["prefix_len"][0])
    dev = DeviceRound(inp, capacity=P + (R + 1) * (cfg.L + 1))
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
