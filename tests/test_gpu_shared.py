"""The shared-budget tree build on the GPU against the oracle's allocation
(paper App. B.5, Proposition 4): the node counts of every sequence are exact and
every tree is the oracle's (exact layout) unless the batch's cut, the
threshold or a sequence's own cap boundary is a near-tie (<= 1e-3 in log
units), where the counts still sum to at most the budget and every tree is a
valid top set.  With a budget that binds nowhere the trees equal the fixed-width
build's."""
import numpy as np
import pytest
import torch

from oracle import shared as sh
from synth import gen_round, make_config
from tests import parity

pytestmark = pytest.mark.gpu


def _device_draft(x, dtype):
    from tree_verified_block_amd.round import to_device
    return to_device(x, dtype, "cuda")


def _run(drafts, dtype, roots, w, B, n_max, tau=float("-inf")):
    from tree_verified_block_amd import api
    nseq, L, V = drafts.shape
    out = api.tree_outputs(nseq, n_max, "cuda")
    for v in out.values():
        v.fill_(7)  # a value the kernel must overwrite everywhere
    ws = api.workspace(api.build_tree_ws_bytes(nseq, L, V, n_max), "cuda")
    wd = w if torch.is_tensor(w) else torch.tensor(np.asarray(w, np.float32), device="cuda")
    api.glance_build_tree_shared(_device_draft(drafts, dtype),
                                 torch.tensor(np.asarray(roots, np.int32), device="cuda"),
                                 wd, n_max, B, out, ws, min_log_value=tau)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["anc"] = res["anc"].view(np.uint64)
    return res


def _case(name, seed, B, n_max, tau=float("-inf"), w=None, w_gpu=None, **over):
    """w: the oracle's weights (rounded to float32, the boundary's type); w_gpu:
    the device's own weights when they come from a device computation."""
    cfg = make_config(name, **over)
    inp = gen_round(cfg, seed, with_model=False)
    rd = inp["rounds"][0]
    drafts, roots = rd["draft_logits"], rd["root"]
    rng = np.random.default_rng(seed)
    if w is None:
        w = rng.normal(0.0, 1.0, cfg.nseq)
    w = np.asarray(w, np.float32).astype(np.float64)   # the key adds the float32 weight
    gpu = _run(drafts, cfg.dtype, roots, w if w_gpu is None else w_gpu, B, n_max, tau)
    trees, n, gap, tmargin = sh.build_trees([drafts[s] for s in range(cfg.nseq)], cfg.dtype, roots,
                                            w, B, n_max, tau)
    report = {}
    got_n = gpu["n_valid"] - 1
    assert got_n.sum() <= B and np.all(got_n <= n_max)
    if gap > parity.GAP and tmargin > parity.GAP:
        assert got_n.tolist() == n.tolist()
        report["cut_exact"] = 1
    else:
        report["cut_flagged"] = 1
        assert abs(int(got_n.sum()) - int(n.sum())) <= 1
    for s in range(cfg.nseq):
        if got_n[s] == n[s]:
            parity.check_tree(gpu, s, trees[s], trees[s]["logq"], n_max, cfg.L, report)
    print(f"[shared] {name} nseq={cfg.nseq} B={B} n_max={n_max} tau={tau}: n={got_n.tolist()} "
          f"gap={gap:.3g} {report}", flush=True)
    return gpu, n, cfg, drafts, roots, w


@pytest.mark.parametrize("name,seed,B,n_max,over", [
    ("tiny", 1, 20, 15, dict(nseq=3)),
    ("mini_bf16", 2, 124, 63, dict(nseq=4, draft="mixed")),
    ("mini_bf16", 3, 40, 31, dict(nseq=6, draft="mixed")),
    ("qwen8b_ragged8", 4, 248, 63, {}),
])
def test_shared_budget_matches_oracle(name, seed, B, n_max, over):
    _case(name, seed, B, n_max, **over)


def test_threshold_and_zero_value_sequences():
    gpu, n, *_ = _case("mini_bf16", 5, 200, 63, tau=-9.0, w=[0.0, -np.inf, 0.5, -1.0],
                       nseq=4, draft="mixed")
    assert gpu["n_valid"][1] == 1 and n[1] == 0


def test_zero_budget_gives_roots_alone():
    gpu, n, cfg, *_ = _case("mini_bf16", 6, 0, 63, nseq=3, draft="mixed")
    assert np.all(gpu["n_valid"] == 1) and np.all(n == 0)
    assert np.all(gpu["parent"][:, 0] == -1) and np.all(gpu["token"][:, 1:] == -1)


def test_unbinding_budget_equals_fixed_width():
    from tree_verified_block_amd import api
    gpu, n, cfg, drafts, roots, _ = _case("mini_bf16", 7, 10 ** 6, 40, nseq=5, draft="mixed")
    nseq, L, V = drafts.shape
    out = api.tree_outputs(nseq, 40, "cuda")
    ws = api.workspace(api.build_tree_ws_bytes(nseq, L, V, 40), "cuda")
    api.glance_build_tree(_device_draft(drafts, cfg.dtype),
                          torch.tensor(np.asarray(roots, np.int32), device="cuda"), 40, out, ws)
    torch.cuda.synchronize()
    for k, v in out.items():
        assert np.array_equal(v.cpu().numpy().view(gpu[k].dtype) if k == "anc" else v.cpu().numpy(),
                              gpu[k]), k


# ------------------------------------------------- entropy-keyed weights (f2)
# paper §6 Eq. 2, App. B and B.5 Eq. 5: ln V(H) from each round's root entropy
LAW = [(0.96, 0.63, 15), (1.226, 0.95, 15), (0.96, 1.71, 1), (2.0, 0.46, 7)]


def _log_value_gpu(H, b0, b1, L, stride=1):
    from tree_verified_block_amd import api
    Ht = torch.tensor(np.asarray(H, np.float32), device="cuda")
    n = Ht.numel() // stride
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    api.glance_entropy_log_value(Ht, b0, b1, L, out, stride=stride)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("b0,b1,L", LAW)
def test_entropy_log_value_matches_oracle(b0, b1, L):
    rng = np.random.default_rng(int(b1 * 100) + L)
    H = np.concatenate([[0.0, 1e-6, b0 / b1, 6.0, 30.0, 1e4, np.nan, -1e-7],
                        rng.uniform(0.0, 8.0, 300)]).astype(np.float32)
    got = _log_value_gpu(H, b0, b1, L).cpu().numpy().astype(np.float64)
    want = sh.log_value(H.astype(np.float64), b0, b1, L)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(got[~fin] == want[~fin])
    err = np.abs(got[fin] - want[fin]) / np.maximum(1.0, np.abs(want[fin]))
    assert err.max() <= 1e-5, err.max()
    # strided input: every n_rows-th entry (row 0 of each sequence)
    n_rows = 64
    Hs = np.full((len(H), n_rows), 99.0, np.float32)
    Hs[:, 0] = H
    got_s = _log_value_gpu(Hs.reshape(-1), b0, b1, L, stride=n_rows).cpu().numpy()
    assert np.array_equal(got_s, got.astype(np.float32), equal_nan=True)


@pytest.mark.parametrize("name,seed,B,n_max,over", [
    ("mini_bf16", 11, 120, 63, dict(nseq=6, draft="mixed")),
    ("qwen8b_ragged8", 12, 248, 63, {}),
])
def test_entropy_keyed_shared_budget(name, seed, B, n_max, over):
    """Root entropies over the pages' span (0.1-6 nats) -> ln V on the device ->
    the shared build, against the oracle's ln V and allocation."""
    b0, b1, L = 0.96, 0.63, 15
    nseq = make_config(name, **over).nseq
    H = np.random.default_rng(seed).uniform(0.1, 6.0, nseq).astype(np.float32)
    lw_gpu = _log_value_gpu(H, b0, b1, L)
    lw = sh.log_value(H.astype(np.float64), b0, b1, L)
    gpu, n, cfg, *_ = _case(name, seed, B, n_max, w=lw, w_gpu=lw_gpu, **over)
    # the intermediate-entropy rounds get the width: V peaks at intermediate H
    assert int(np.argmax(lw)) == int(np.argmax(lw_gpu.cpu().numpy()))
