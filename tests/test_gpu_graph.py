"""A whole verify round captured once into a HIP graph and replayed: every replay
(with eager rounds of another draft and host synchronisations between them)
returns exactly the outputs of the eager round of the same draft.  The library
allocates nothing and records no memset inside a call, and its arrival counters
reset themselves, so the captured launches are replayable."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


# mini_bf16 merges its attention splits inside the attention kernel (arrival
# counters that must return to zero between replays); mini_bf16_ragged has 123
# rows, so its projections and head take two 64-row tiles per work-group.
@pytest.mark.parametrize("name,seed,packed,kw", [("mini_bf16_copy", 5, True, {}),
                                                 ("mini_bf16", 6, True, dict(n_rounds=2, draft_scales=(3.0, 4.0))),
                                                 ("mini_bf16_ragged", 8, True, dict(n_rounds=2)),
                                                 ("qwen8b_1layer", 2000, True, {}),
                                                 ("tiny", 7, False, dict(n_rounds=2))])
def test_graph_replay_equals_eager(name, seed, packed, kw):
    from synth import gen_round, make_config
    from tree_verified_block_amd.round import DeviceRound, to_device
    cfg = make_config(name, **kw)
    inp = gen_round(cfg, seed)
    dev = DeviceRound(inp, packed_head=packed and cfg.dtype == "bf16")
    dev.set_round(0)
    drafts = [to_device(rd["draft_logits"], cfg.dtype, "cuda") for rd in inp["rounds"]]
    assert len(drafts) >= 2

    def eager(i):
        dev.draft = drafts[i]
        dev.run()
        return dev.fetch()

    want = [eager(i) for i in range(2)]
    # capture the round of draft 0 (its tensor is the one the graph reads)
    dev.draft = drafts[0]
    dev.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev.run()
    for rep in range(4):
        eager(1)                 # eager work of another draft between replays
        g.replay()
        got = dev.fetch()        # synchronises
        for k in want[0]:
            assert np.array_equal(np.asarray(got[k]), np.asarray(want[0][k])), (rep, k)
