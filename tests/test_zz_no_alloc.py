"""The allocation-free packed LM head: two calls in a row (the second with fewer
rows, so stale scratch from the first would show) return exactly what the
workspace call returns, greedy and sampled, at the 8B head shape."""
import numpy as np
import pytest
import torch

from tree_verified_block_amd import api

pytestmark = pytest.mark.gpu


def _outs(R, V):
    o = {k: torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
         for k in ("top1", "gap", "H", "sgap")}
    o["am"] = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    o["tok"] = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    o["logits"] = torch.full((R, V), float("nan"), dtype=torch.float32, device="cuda")
    return o


def _call(h, packed, V, sample, noalloc):
    R = h.shape[0]
    o = _outs(R, V)
    kw = {}
    if sample:
        kw = dict(temperature=sample[0], seed=sample[1], round_id=sample[2],
                  sample_tok=o["tok"], sample_gap=o["sgap"])
    if noalloc:
        api.glance_verify_head_packed_noalloc(h, packed, V, o["am"], o["top1"], o["gap"], o["H"],
                                              logits=o["logits"], **kw)
    else:
        ws = api.workspace(api.verify_head_ws_bytes(R, V, h.shape[1], 1), "cuda")
        api.glance_verify_head_packed(h, packed, V, o["am"], o["top1"], o["gap"], o["H"], ws,
                                      logits=o["logits"], **kw)
    torch.cuda.synchronize()
    keys = ["am", "top1", "gap", "H", "logits"] + (["tok", "sgap"] if sample else [])
    return {k: o[k].cpu().numpy() for k in keys}


@pytest.mark.parametrize("sample", [None, (0.8, (1 << 40) + 7, 123)])
def test_noalloc_head_equals_workspace_head(sample):
    V, d = 151936, 4096
    g = torch.Generator(device="cuda").manual_seed(77)
    w = (torch.randn((V, d), generator=g, device="cuda") * 0.05).to(torch.bfloat16)
    packed = api.glance_head_pack(w)
    del w
    for R in (200, 37):
        print(f"noalloc head: R={R} sample={sample is not None}", flush=True)
        h = (torch.randn((R, d), generator=g, device="cuda")).to(torch.bfloat16)
        ref = _call(h, packed, V, sample, noalloc=False)
        got = _call(h, packed, V, sample, noalloc=True)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (R, k)


def test_noalloc_head_rejects_rows_beyond_its_scratch():
    V, d = 151936, 4096
    limit = 8 << 20
    R = 1
    while api.verify_head_ws_bytes(R + 1, V, d, 1) <= limit:
        R += 1
    h = torch.zeros((R + 1, d), dtype=torch.bfloat16, device="cuda")
    packed = torch.zeros(api.head_pack_bytes(V, d), dtype=torch.uint8, device="cuda")
    o = _outs(R + 1, V)
    with pytest.raises(RuntimeError, match="scratch"):
        api.glance_verify_head_packed_noalloc(h, packed, V, o["am"], o["top1"], o["gap"], o["H"])
