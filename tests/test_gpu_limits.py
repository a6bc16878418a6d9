"""Steps 1-2 at the limits the C ABI documents: L = GLANCE_MAX_L (16) offsets,
vocabularies of 2^18 (bf16) and 2^17 (fp32) logits, N + 1 = GLANCE_MAX_ROWS
rows, and a shared-budget batch of GLANCE_MAX_SHARED (16) sequences; every tree
against the oracle's exact tree (exact layout unless its boundary is a
near-tie)."""
import numpy as np
import pytest
import torch

from oracle import round as orr, shared as sh
from synth import gen_round, make_config
from synth.gen import bf16_bits, bf16_bits_to_f32
from tests import parity

pytestmark = pytest.mark.gpu


def _build(drafts, dtype, roots, N):
    from tree_verified_block_amd import api
    from tree_verified_block_amd.round import to_device
    nseq, L, V = drafts.shape
    out = api.tree_outputs(nseq, N, "cuda")
    ws = api.workspace(api.build_tree_ws_bytes(nseq, L, V, N), "cuda")
    api.glance_build_tree(to_device(drafts, dtype, "cuda"),
                          torch.tensor(np.asarray(roots, np.int32), device="cuda"), N, out, ws)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["anc"] = res["anc"].view(np.uint64)
    return res


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,V,draft", [("bf16", 1 << 18, "mixed"), ("f32", 1 << 17, "scaled")])
def test_tree_at_the_size_limits(dtype, V, draft):
    cfg = make_config("mini_bf16", dtype=dtype, V=V, L=16, N=63, nseq=2, draft=draft)
    inp = gen_round(cfg, 17, with_model=False)
    rd = inp["rounds"][0]
    gpu = _build(rd["draft_logits"], dtype, rd["root"], cfg.N)
    report = {}
    for s in range(cfg.nseq):
        ot = orr.build_tree(rd["draft_logits"][s], dtype, int(rd["root"][s]), cfg.N)
        parity.check_tree(gpu, s, ot, ot["logq"], cfg.N, cfg.L, report)
        assert int(gpu["depth"][s].max()) <= 16
    print(f"[limits] {dtype} V={V} L=16: {report}", flush=True)


@pytest.mark.timeout(300)
def test_shared_budget_with_the_most_sequences():
    from tree_verified_block_amd import api
    from tree_verified_block_amd.round import to_device
    cfg = make_config("mini_bf16", V=4099, L=8, nseq=16, draft="mixed")
    inp = gen_round(cfg, 18, with_model=False)
    rd = inp["rounds"][0]
    w = np.random.default_rng(18).normal(0.0, 1.0, 16).astype(np.float32)
    B, n_max = 16 * 20, 63
    out = api.tree_outputs(16, n_max, "cuda")
    ws = api.workspace(api.build_tree_ws_bytes(16, cfg.L, cfg.V, n_max), "cuda")
    api.glance_build_tree_shared(to_device(rd["draft_logits"], cfg.dtype, "cuda"),
                                 torch.tensor(rd["root"].astype(np.int32), device="cuda"),
                                 torch.tensor(w, device="cuda"), n_max, B, out, ws)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in out.items()}
    gpu["anc"] = gpu["anc"].view(np.uint64)
    trees, n, gap, tm = sh.build_trees([rd["draft_logits"][s] for s in range(16)], cfg.dtype,
                                       rd["root"], w.astype(np.float64), B, n_max)
    got = gpu["n_valid"] - 1
    assert got.sum() <= B
    report = {}
    if gap > parity.GAP:
        assert got.tolist() == n.tolist()
    for s in range(16):
        if got[s] == n[s]:
            parity.check_tree(gpu, s, trees[s], trees[s]["logq"], n_max, cfg.L, report)
    print(f"[limits] shared 16 sequences: n={got.tolist()} gap={gap:.3g} {report}", flush=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 1 << 17)])
def test_tree_when_every_chunk_ends_in_ties(dtype, V):
    """Rows of equal logits (0) with 100 spikes in [1, 7): the K best keys of
    every chunk of a row end in a run of equal logits, ranked by token id (the
    exact radix select), while each merged row keeps only spikes (in bf16 some
    spikes are equal too, again ranked by token id)."""
    rng = np.random.default_rng(19)
    nseq, L, N = 2, 4, 63
    z = np.zeros((nseq, L, V), np.float32)
    for s in range(nseq):
        for j in range(L):
            z[s, j, rng.choice(V, 100, replace=False)] = rng.uniform(1.0, 7.0, 100)
    if dtype == "bf16":   # the values the device sees
        z = bf16_bits_to_f32(bf16_bits(z))
    stored = z if dtype == "f32" else bf16_bits(z)
    roots = np.array([3, 4], np.int64)
    gpu = _build(stored, dtype, roots, N)
    report = {}
    for s in range(nseq):
        ot = orr.build_tree(stored[s], dtype, int(roots[s]), N)
        parity.check_tree(gpu, s, ot, ot["logq"], N, L, report)
        # every node's token is one of its offset's spikes
        nv = int(gpu["n_valid"][s])
        for i in range(1, nv):
            assert z[s, int(gpu["depth"][s][i]) - 1, int(gpu["token"][s][i])] >= 1.0
    print(f"[limits] ties {dtype} V={V}: {report}", flush=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,V,L,N", [
    ("bf16", 151936, 1, 63),   # one offset: the tree is the root's 63 best children
    ("bf16", 151936, 16, 1),   # a single node
    ("bf16", 4099, 2, 5),      # V not a multiple of the 8-logit vector (scalar loads)
    ("f32", 20011, 7, 40),     # V not a multiple of the 4-logit vector
    ("f32", 3, 4, 63),         # fewer tokens than K: lists end early
])
def test_tree_at_edge_shapes(dtype, V, L, N):
    rng = np.random.default_rng(20 + L + N)
    nseq = 2
    z = rng.normal(0.0, 2.0, (nseq, L, V)).astype(np.float32)
    stored = z if dtype == "f32" else bf16_bits(z)
    roots = np.array([5 % V, 7 % V], np.int64)
    gpu = _build(stored, dtype, roots, N)
    report = {}
    for s in range(nseq):
        ot = orr.build_tree(stored[s], dtype, int(roots[s]), N)
        parity.check_tree(gpu, s, ot, ot["logq"], N, L, report)
    print(f"[limits] edge {dtype} V={V} L={L} N={N}: {report}", flush=True)


@pytest.mark.timeout(300)
def test_nonfinite_logits_set_the_flag_word():
    """The workspace's flag word reports NaN (bit 0) and +inf (bit 1) draft
    logits; -inf logits are legal (probability 0) and leave it clear, and the
    word is sticky until the caller clears it."""
    from tree_verified_block_amd import api
    from tree_verified_block_amd.round import to_device
    cfg = make_config("mini_bf16", V=4099, L=4, N=15, nseq=2)
    inp = gen_round(cfg, 19, with_model=False)
    z = bf16_bits_to_f32(inp["rounds"][0]["draft_logits"]).copy()
    roots = torch.tensor(inp["rounds"][0]["root"].astype(np.int32), device="cuda")
    out = api.tree_outputs(cfg.nseq, cfg.N, "cuda")
    ws = api.workspace(api.build_tree_ws_bytes(cfg.nseq, cfg.L, cfg.V, cfg.N), "cuda")

    def build(zz):
        api.glance_build_tree(to_device(bf16_bits(zz), "bf16", "cuda"), roots, cfg.N, out, ws)
        return api.build_tree_flags(ws, cfg.nseq, cfg.L, cfg.V, cfg.N)

    zi = z.copy()
    zi[0, 1, 7] = -np.inf
    zi[1, 3, 100:200] = -np.inf
    assert build(zi) == 0
    zn = z.copy()
    zn[1, 2, 4000] = np.nan
    assert build(zn) == 1
    assert build(z) == 1                 # sticky
    off = api._lib.load().glance_build_tree_flag_offset(cfg.nseq, cfg.L, cfg.V, cfg.N)
    ws[off:off + 4].zero_()
    zp = z.copy()
    zp[0, 0, 3] = np.inf
    assert build(zp) == 2
    zp[1, 0, 9] = np.nan
    assert build(zp) == 3
