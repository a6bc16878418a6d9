"""Parity at the full 8B-shaped sizes, in the launch configuration the benchmark
times (the same DeviceRound path: one C-ABI call per step, bf16 storage).

  single layer  d_model 4096, 32q/8kv heads x 128, V 151936, L 15, N 63, a
                1024-token prefix; six draft temperatures (one round each);
                every row checked against the oracle's full float64 head
  copy regime   the same shapes with a 4096-token prefix and N 31; the planted
                run must be accepted whole (A = G) and the break token emitted
  ragged batch  8 rounds in one call, prefixes uniform in 512..6144; rows on
                the walk plus a seeded sample per round, with their ancestors
  full layer    the single-layer shapes with RMSNorm, QK-norm and a SwiGLU MLP
                (intermediate 12288); sampled rows as for the ragged batch
  deep stack    36 layers over an 8192-token prefix, a given random topology;
                a sampled set of rows (and their ancestors) evaluated
                free-running by the oracle (every layer's attention output and
                hidden rows, the logits, argmax and walk), and beside it each
                layer on the inputs the GPU fed it (the per-call contract)

The oracle evaluates each sampled row on its own explicit token sequence
(unpacked), so a sample needs only the row and its ancestors."""
import gc

import numpy as np
import pytest

from oracle import model as mdl, round as orr
from synth import gen_round, make_config
from tests import parity

pytestmark = pytest.mark.gpu

_CACHE: dict = {}


def _workload(name, seed, cache_head):
    """Inputs, oracle model and device round of one configuration (one at a time:
    switching configurations frees the previous one)."""
    key = (name, seed)
    if key not in _CACHE:
        _CACHE.clear()
        gc.collect()
        import torch
        torch.cuda.empty_cache()
        from tree_verified_block_amd.round import DeviceRound
        inp = gen_round(make_config(name), seed)
        print(f"[full] generated {name} seed {seed}", flush=True)
        model = mdl.TargetModel(inp, cache_head=cache_head)
        dev = DeviceRound(inp, keep_layers=True, want_logits=True)
        _CACHE[key] = (inp, model, dev)
    return _CACHE[key]


def _closure(parent, rows):
    keep = set()
    for r in rows:
        r = int(r)
        while r >= 0 and r not in keep:
            keep.add(r)
            r = int(parent[r])
    return sorted(keep)


def _check_walk_on_rows(gpu, s, n_rows, am_rows, gap_rows, rows, L, report):
    """The GPU walk of round s against the oracle's argmax on the rows it visits:
    where none of them is a near-tie, the oracle's walk takes the same steps (the
    argmax token's child, or the stop) and so commits the same tokens."""
    a = int(gpu["n_accept"][s])
    path = [int(x) for x in gpu["path_rows"][s][:a + 1]]
    toks = gpu["out_tokens"][s]
    parent, token = gpu["parent"][s], gpu["token"][s]
    nv = int(gpu["n_valid"][s])
    pos = {r: i for i, r in enumerate(rows)}
    if any(gap_rows[pos[r]] <= report["threshold"] for r in path):
        report["walk_flagged"] = report.get("walk_flagged", 0) + 1
        return
    for k, r in enumerate(path):
        y = int(am_rows[pos[r]])
        assert int(toks[k]) == y
        kids = [c for c in range(1, nv) if int(parent[c]) == r and int(token[c]) == y]
        # the argmax token's child continues the walk; at the stop there is none
        assert kids == ([path[k + 1]] if k < a else [])
    report["walk_exact"] = report.get("walk_exact", 0) + 1


def _sampled_round(inp, model, dev, r, per_seq, seed, teacher_forced=False):
    """Round r with a seeded sample of rows per sequence (and their ancestors)
    compared free-running; ``teacher_forced`` adds the per-layer comparison on
    the GPU's own layer inputs."""
    cfg = inp["cfg"]
    dev.set_round(r)
    dev.run()
    gpu = dev.fetch()
    rd = inp["rounds"][r]
    rng = np.random.default_rng(seed + 7919 * r)
    report = {}
    n_rows = cfg.N + 1
    for s in range(cfg.nseq):
        root = int(rd["root"][s])
        if "draft_logits" in rd:
            ot = orr.build_tree(rd["draft_logits"][s], cfg.dtype, root, cfg.N, "beam")
            parity.check_tree(gpu, s, ot, ot["logq"], cfg.N, cfg.L, report)
        paths = parity.gpu_paths(gpu["parent"][s], gpu["token"][s], gpu["n_valid"][s])
        nv = int(gpu["n_valid"][s])
        a = int(gpu["n_accept"][s])
        want = list(gpu["path_rows"][s][:a + 1]) + list(rng.choice(nv, size=min(per_seq, nv),
                                                                   replace=False))
        rows = _closure(gpu["parent"][s], want)
        sel = [paths[i] for i in rows]
        g_rows = [s * n_rows + i for i in rows]
        ev = mdl.evaluate_paths(model, s, root, sel)
        z = model.logits(ev["final"])
        am, gap = parity.check_rows(gpu, ev, z, s, n_rows, cfg, report, rows=rows)
        _check_walk_on_rows(gpu, s, n_rows, am, gap, rows, cfg.L, report)
        if teacher_forced:
            feeds = [None] + [gpu["h_layers"][li - 1][g_rows] for li in range(1, cfg.n_layers)]
            tf = mdl.evaluate_paths(model, s, root, sel, layer_inputs=feeds)
            tol = parity.tol_for(cfg.dtype)
            for li in range(cfg.n_layers):
                ea = parity.rel_err(gpu["attn_out"][li][g_rows], tf["attn"][li])
                eh = parity.rel_err(gpu["h_layers"][li][g_rows], tf["h"][li])
                report["tf_attn_err"] = max(report.get("tf_attn_err", 0.0), ea)
                report["tf_h_err"] = max(report.get("tf_h_err", 0.0), eh)
                assert ea <= tol and eh <= tol, ("teacher-forced layer", li, ea, eh)
    parity.record(f"{cfg.name} seed={inp['seed']} round={r}", report)
    return gpu, report


# ------------------------------------------------------------- single layer
@pytest.mark.timeout(300)
@pytest.mark.parametrize("r", range(6))
def test_single_layer_8b_round(r):
    """Every row of the round, the tree, the walk and the independent greedy
    decode, at one of six draft temperatures."""
    inp, model, dev = _workload("qwen8b_1layer", 2000, cache_head=True)
    cfg = inp["cfg"]
    dev.set_round(r)
    dev.run()
    gpu = dev.fetch()
    rd = inp["rounds"][r]
    root = int(rd["root"][0])
    report = {}
    ot = orr.build_tree(rd["draft_logits"][0], cfg.dtype, root, cfg.N, "beam")
    paths = parity.check_tree(gpu, 0, ot, ot["logq"], cfg.N, cfg.L, report)
    ev = mdl.evaluate_paths(model, 0, root, paths)
    z = model.logits(ev["final"])
    am, gap = parity.check_rows(gpu, ev, z, 0, cfg.N + 1, cfg, report)
    g = orr.continuation(model, 0, root, paths[1:], cfg.L)
    parity.check_walk(gpu, 0, paths, am, gap, cfg.L, report, g)
    parity.record(f"{cfg.name} scale={rd['scale']} round={r}", report)


@pytest.mark.timeout(300)
def test_partial_tree_8b_round():
    """Draft logits that are -inf off two tokens at the first offset and one at
    every later one: 30 finite prefixes, so 31 live rows of 64.  The padding
    rows pass through the attention (zeroed), the head and the walk; the live
    rows, the walk and the greedy decode match the oracle."""
    from tests.test_gpu_parity import _sparse_draft
    from tree_verified_block_amd.round import to_device
    inp, model, dev = _workload("qwen8b_1layer", 2000, cache_head=True)
    cfg = inp["cfg"]
    dev.set_round(0)
    rd = inp["rounds"][0]
    draft = _sparse_draft(rd["draft_logits"], cfg.dtype, [2] + [1] * (cfg.L - 1))
    dev.draft = to_device(draft, cfg.dtype, "cuda")
    dev.run()
    gpu = dev.fetch()
    root = int(rd["root"][0])
    report = {}
    ot = orr.build_tree(draft[0], cfg.dtype, root, cfg.N, "beam")
    paths = parity.check_tree(gpu, 0, ot, ot["logq"], cfg.N, cfg.L, report)
    assert int(gpu["n_valid"][0]) == 31 == len(paths)
    assert np.all(gpu["h_final"][31:] == 0) and np.all(gpu["attn_out"][0][31:] == 0)
    ev = mdl.evaluate_paths(model, 0, root, paths)
    z = model.logits(ev["final"])
    am, gap = parity.check_rows(gpu, ev, z, 0, cfg.N + 1, cfg, report)
    g = orr.continuation(model, 0, root, paths[1:], cfg.L)
    parity.check_walk(gpu, 0, paths, am, gap, cfg.L, report, g)
    parity.record(f"{cfg.name} partial tree (31 of 64 rows)", report)


# --------------------------------------------------------------- copy regime
@pytest.mark.timeout(300)
@pytest.mark.parametrize("r", range(4))
def test_copy_regime_8b_accepts_planted_run(r):
    inp, model, dev = _workload("qwen8b_copy", 3000, cache_head=True)
    cfg = inp["cfg"]
    dev.set_round(r)
    dev.run()
    gpu = dev.fetch()
    rd = inp["rounds"][r]
    root = int(rd["root"][0])
    report = {}
    ot = orr.build_tree(rd["draft_logits"][0], cfg.dtype, root, cfg.N, "beam")
    paths = parity.check_tree(gpu, 0, ot, ot["logq"], cfg.N, cfg.L, report)
    ev = mdl.evaluate_paths(model, 0, root, paths)
    z = model.logits(ev["final"])
    am, gap = parity.check_rows(gpu, ev, z, 0, cfg.N + 1, cfg, report)
    g = orr.continuation(model, 0, root, paths[1:], cfg.L)
    parity.check_walk(gpu, 0, paths, am, gap, cfg.L, report, g)
    assert int(gpu["n_accept"][0]) == rd["G"]
    assert int(gpu["out_tokens"][0][rd["G"]]) == rd["break_token"]
    parity.record(f"{cfg.name} round={r} G={rd['G']}", report)


# -------------------------------------------------------------- ragged batch
@pytest.mark.timeout(300)
def test_ragged_batch_8b_sampled_rows():
    inp, model, dev = _workload("qwen8b_ragged8", 5000, cache_head=False)
    _sampled_round(inp, model, dev, 0, per_seq=4, seed=5000)


# ---------------------------------------------------------------- full layer
@pytest.mark.timeout(300)
def test_full_layer_8b_sampled_rows():
    """A full decoder layer (RMSNorm, QK-norm, SwiGLU MLP with intermediate
    size 12288) at the 8B shapes: the attention output and hidden rows of a
    seeded sample of rows (with their ancestors), their logits and the walk."""
    inp, model, dev = _workload("qwen8b_full", 6000, cache_head=False)
    _sampled_round(inp, model, dev, 0, per_seq=4, seed=6000)


# ---------------------------------------------------------------- deep stack
@pytest.mark.timeout(900)
def test_deep_36_layers_sampled_rows():
    """The 36-layer round free-running against the oracle (every layer's
    attention output and hidden rows, logits, argmax and walk of the sampled
    rows), and each layer on the inputs the GPU fed it (the per-call contract
    of the attention entry point)."""
    inp, model, dev = _workload("qwen8b_deep36", 4000, cache_head=False)
    _sampled_round(inp, model, dev, 0, per_seq=3, seed=4000, teacher_forced=True)
