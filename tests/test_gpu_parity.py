"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
synthetic rounds.  Every test needs an MI355X."""
import numpy as np
import pytest

from oracle import model as mdl, round as orr, tree as tr
from synth import gen_round, make_config
from tests import parity

pytestmark = pytest.mark.gpu


def _run(inp, r=0, logits=True):
    from tree_verified_block_amd.round import DeviceRound
    dev = DeviceRound(inp, keep_layers=True, want_logits=logits)
    dev.set_round(r)
    dev.run()
    return dev.fetch()


def _round_parity(inp, r, exact="beam", greedy=True):
    cfg = inp["cfg"]
    gpu = _run(inp, r)
    model = inp.setdefault("_oracle_model", mdl.TargetModel(inp))
    rd = inp["rounds"][r]
    report = {}
    for s in range(cfg.nseq):
        root = int(rd["root"][s])
        if "draft_logits" in rd:
            ot = orr.build_tree(rd["draft_logits"][s], cfg.dtype, root, cfg.N, exact)
            paths = parity.check_tree(gpu, s, ot, ot["logq"], cfg.N, cfg.L, report)
        else:
            paths = parity.gpu_paths(gpu["parent"][s], gpu["token"][s], gpu["n_valid"][s])
        ev = mdl.evaluate_paths(model, s, root, paths)
        z = model.logits(ev["final"])
        am, gap = parity.check_rows(gpu, ev, z, s, cfg.N + 1, cfg, report)
        g = orr.continuation(model, s, root, paths[1:], cfg.L) if greedy else None
        parity.check_walk(gpu, s, paths, am, gap, cfg.L, report, g)
    parity.record(f"{cfg.name} seed={inp['seed']} round={r}", report)
    return gpu, report


@pytest.mark.parametrize("seed", [1000, 1001, 1002])
def test_tiny_round_brute_force(seed):
    """Tiny fp32 round; the oracle's tree is the full enumeration."""
    _round_parity(gen_round(make_config("tiny"), seed), 0, exact="brute")


@pytest.mark.parametrize("seed", range(1000, 1006))
def test_tiny_widehead_round(seed):
    _round_parity(gen_round(make_config("tiny_widehead"), seed), 0)


def test_tiny_empty_tree():
    inp = gen_round(make_config("tiny_widehead", N=0), 1000)
    gpu, _ = _round_parity(inp, 0)
    assert gpu["n_valid"][0] == 1 and gpu["n_accept"][0] == 0
    assert gpu["out_tokens"][0][0] == gpu["argmax"][0]


@pytest.mark.parametrize("name,seed", [("mini_bf16", 1), ("mini_bf16", 2),
                                       ("mini_bf16_ragged", 3), ("mini_bf16_ragged", 4)])
def test_mini_bf16_round(name, seed):
    _round_parity(gen_round(make_config(name), seed), 0)


def test_eight_query_heads_per_kv_head():
    """Eight query heads share one KV head (G = 8): 8 x 41 queries per round
    and KV head, query blocks that straddle rows; two ragged rounds."""
    cfg = make_config("mini_bf16_ragged", Hq=8, Hkv=1, d_model=512, nseq=2)
    _round_parity(gen_round(cfg, 33), 0)


@pytest.mark.parametrize("Hq,Hkv,seed", [(2, 2, 41), (6, 2, 42)])
def test_query_heads_not_a_multiple_of_four(Hq, Hkv, seed):
    """One query head per KV head (plain multi-head attention) and three per KV
    head: query counts that leave the last query block partly empty, and split
    records merged by the one-dimension-per-thread merge kernel (the 16-byte
    merge needs a multiple of four query heads); a 600-token prefix gives
    several splits."""
    cfg = make_config("mini_bf16_copy", Hq=Hq, Hkv=Hkv, prefix=("fixed", 600), n_rounds=1)
    _round_parity(gen_round(cfg, seed), 0)


@pytest.mark.parametrize("nseq,seed", [(4, 31), (7, 32)])
def test_projection_row_tiles(nseq, seed):
    """More rows than one 64-row tile: the projections take several tiles per
    work-group, and 164 or 287 rows leave the last group of tiles partly empty;
    every round output against the oracle."""
    _round_parity(gen_round(make_config("mini_bf16_ragged", nseq=nseq), seed), 0)


@pytest.mark.parametrize("seed", [1, 2])
def test_mini_full_layer_round(seed):
    """Two full decoder layers (RMSNorm, QK-norm, SwiGLU MLP): every layer's
    attention output and hidden rows, the logits, the statistics and the walk."""
    _round_parity(gen_round(make_config("mini_bf16_full"), seed), 0)


def test_mini_copy_regime_accepts_planted_run():
    inp = gen_round(make_config("mini_bf16_copy"), 3)
    for r, rd in enumerate(inp["rounds"]):
        gpu, _ = _round_parity(inp, r)
        assert int(gpu["n_accept"][0]) == rd["G"]
        assert int(gpu["out_tokens"][0][rd["G"]]) == rd["break_token"]


@pytest.mark.parametrize("prefix,seed", [(300, 21), (600, 22), (1500, 23), (20000, 24)])
def test_attention_split_paths(prefix, seed):
    """Two query blocks per KV head and longer prefixes: four-wave tile groups
    with two key splits merged inside the attention kernel (prefix 300), with
    four splits merged by the separate merge kernel (600), with more than
    eight (1500), and at the cap of sixteen splits of about forty 32-key
    blocks each (20000); every output against the oracle, and a second and
    third launch give the same bits (the merge's arrival counters return to
    zero)."""
    from tree_verified_block_amd.round import DeviceRound
    inp = gen_round(make_config("mini_bf16_copy", prefix=("fixed", prefix), n_rounds=1), seed)
    first, _ = _round_parity(inp, 0)
    dev = DeviceRound(inp, keep_layers=True, want_logits=True)
    dev.set_round(0)
    for _ in range(2):
        dev.run()
        again = dev.fetch()
        for k in ("attn_out", "h_final", "logits", "argmax", "n_accept", "out_tokens"):
            assert np.array_equal(np.asarray(again[k]), np.asarray(first[k])), k


@pytest.mark.parametrize("prefix", [300, 600, 1500])
@pytest.mark.parametrize("excess", [40.0, 200.0])
def test_attention_score_far_above_first_block(prefix, excess):
    """One prefix key (position 40, the second 32-key block of the first key
    split) is set along the root row's first query head, so that its score for
    that query lies `excess` (base-2 units) above every score of the split's
    first block: the running maximum jumps by far more than the kernel's
    rescaling threshold, and a weight taken against the old maximum would
    overflow float32 at 200.  Every round output matches the oracle."""
    from synth import bf16_bits, bf16_bits_to_f32
    inp = gen_round(make_config("mini_bf16_copy", prefix=("fixed", prefix), n_rounds=1), 21)
    cfg = inp["cfg"]
    probe = mdl.TargetModel(inp)
    root = int(inp["rounds"][0]["root"][0])
    q, _, _ = probe.project(0, probe.embed_rows([root]), np.array([prefix]))
    qh = q[0, 0]
    K, _ = probe.prefix_kv(0, 0)
    to_log2 = np.log2(np.e) / np.sqrt(cfg.D)
    first = float((K[:32, 0, :] @ qh).max()) * to_log2
    key = (first + excess) / to_log2 * qh / float(qh @ qh)
    kc = inp["layers"][0]["k_cache"]
    kc[int(inp["kv_offsets"][0]) + 40, 0] = bf16_bits(key.astype(np.float32))
    planted = float(bf16_bits_to_f32(kc[int(inp["kv_offsets"][0]) + 40, 0]) @ qh) * to_log2
    assert planted - first > excess - 1.0
    _round_parity(inp, 0)


@pytest.mark.parametrize("name", ["mini_bf16", "tiny"])
def test_layer_before_any_tree_build(name):
    """A round whose drafts are loaded but whose tree was never built: its tree
    outputs are the binding's empty tree, so the attention layer sees only
    padding rows and writes them as zeros."""
    from tree_verified_block_amd.round import DeviceRound
    inp = gen_round(make_config(name), 3)
    dev = DeviceRound(inp, keep_layers=True)
    dev.set_round(0)
    dev.step_attn()
    out = dev.fetch()
    assert np.all(out["token"] == -1)
    assert np.all(out["h_final"] == 0.0)
    assert all(np.all(a == 0.0) for a in out["attn_out"])


def test_mini_given_topology_multilayer():
    """Random prefix-closed topology (no draft), three stacked layers."""
    cfg = make_config("mini_bf16_ragged", draft="topology", n_layers=3, nseq=2, N=63, L=15)
    _round_parity(gen_round(cfg, 9), 0)


def test_determinism():
    """Two launches give identical bits (also a race check of the LDS code)."""
    from tree_verified_block_amd.round import DeviceRound
    inp = gen_round(make_config("mini_bf16_ragged"), 5)
    dev = DeviceRound(inp, keep_layers=True, want_logits=True)
    dev.set_round(0)
    dev.run()
    a = dev.fetch()
    dev.run()
    b = dev.fetch()
    for k in ("parent", "token", "anc", "score", "argmax", "top1", "gap", "entropy", "logits",
              "n_accept", "out_tokens", "h_final"):
        assert np.array_equal(a[k], b[k]), k


def test_non_ancestor_rows_do_not_leak():
    """Changing the token of a leaf changes no other row's output bits."""
    from tree_verified_block_amd.round import DeviceRound
    cfg = make_config("mini_bf16_ragged", draft="topology", nseq=1, N=40, L=7)
    inp = gen_round(cfg, 11)
    dev = DeviceRound(inp, keep_layers=True)
    dev.set_round(0)
    dev.run()
    a = dev.fetch()
    rd = inp["rounds"][0]
    parent = rd["parent"][0]
    leaf = max(i for i in range(1, cfg.N + 1) if i not in set(parent.tolist()))
    tok = dev.tree["token"].clone()
    tok[0, leaf] = (tok[0, leaf] + 1) % cfg.V
    dev.tree["token"].copy_(tok)
    dev.step_attn()
    dev.step_head()
    b = dev.fetch()
    keep = [i for i in range(cfg.N + 1) if i != leaf]
    assert np.array_equal(a["h_final"][keep], b["h_final"][keep])
    assert not np.array_equal(a["h_final"][leaf], b["h_final"][leaf])


def _sparse_draft(draft, dtype, keep):
    """Draft logits with every token of offset j but its keep[j] largest set to
    -inf: only prod_{j<=d} keep[j] prefixes of depth d have a finite score."""
    from synth.gen import as_f32, bf16_bits
    z = as_f32(np.array(draft), dtype).astype(np.float32).copy()
    for s in range(z.shape[0]):
        for j in range(z.shape[1]):
            top = np.argsort(-z[s, j], kind="stable")[:keep[j]]
            row = np.full(z.shape[2], -np.inf, dtype=np.float32)
            row[top] = z[s, j, top]
            z[s, j] = row
    return bf16_bits(z) if dtype == "bf16" else z


@pytest.mark.parametrize("name,seed,exact", [("tiny", 1003, "brute"), ("tiny_widehead", 1004, "beam"),
                                             ("mini_bf16_ragged", 6, "beam")])
def test_partial_tree_round(name, seed, exact):
    """Draft marginals that are zero off a few tokens per offset (logits -inf):
    fewer finite prefixes than N, so the tree has padding rows (token -1), which
    the attention zeroes and the walk never reaches; every live row, the walk and
    the greedy decode still match the oracle (paper §3.2 Def. 1: S need not fill
    the budget)."""
    inp = gen_round(make_config(name), seed)
    cfg = inp["cfg"]
    rd = dict(inp["rounds"][0])
    keep = [2] + [1] * (cfg.L - 1)
    rd["draft_logits"] = _sparse_draft(rd["draft_logits"], cfg.dtype, keep)
    inp = dict(inp, rounds=[rd])
    gpu, _ = _round_parity(inp, 0, exact=exact)
    n_live = 1 + 2 * cfg.L
    assert n_live < cfg.N + 1
    for s in range(cfg.nseq):
        assert int(gpu["n_valid"][s]) == n_live
        rows = slice(s * (cfg.N + 1) + n_live, (s + 1) * (cfg.N + 1))
        assert np.all(gpu["h_final"][rows] == 0)
        for li in range(cfg.n_layers):
            assert np.all(gpu["attn_out"][li][rows] == 0)
