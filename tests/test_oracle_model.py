"""Pins of the oracle's verify rows (steps 3-4): an independent chain evaluation
through torch's scaled_dot_product_attention, a complex-number statement of the
rotary embedding, token-by-token decoding, closed forms of the row statistics,
and the bf16 storage rounding against torch's conversion."""
import numpy as np
import pytest
import scipy.stats
import torch

from oracle import model as mdl, numerics, round as orr, tree as tr
from synth import gen_round, make_config
from synth.gen import as_f32


# ----------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.02, 1.0, 300.0)])
    x = x.astype(np.float32).astype(np.float64)  # torch rounds f32 -> bf16 exactly once
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(numerics.round_bf16(x), want)


def test_round_bf16_ties_to_even():
    u = 2.0 ** -7                       # bf16 spacing just above 1.0
    assert numerics.round_bf16(np.array([1 + u / 2]))[0] == 1.0          # tie -> even
    assert numerics.round_bf16(np.array([1 + 3 * u / 2]))[0] == 1 + 2 * u  # tie -> even
    assert numerics.round_bf16(np.array([1 + u / 2 + 1e-12]))[0] == 1 + u
    assert numerics.round_bf16(np.array([-(1 + u / 2)]))[0] == -1.0
    assert numerics.round_bf16(np.array([0.0]))[0] == 0.0


# ------------------------------------------------------------------------- RoPE
def _rope_complex(x, pos, cos, sin):
    """x [n][H][D] viewed as D/2 complex numbers x_i + i x_{i+D/2}, each
    multiplied by exp(i * angle(pos, i)) with cos/sin of that angle."""
    half = x.shape[-1] // 2
    zc = x[..., :half] + 1j * x[..., half:]
    rot = (cos[pos] + 1j * sin[pos])[:, None, :]
    w = zc * rot
    return np.concatenate([w.real, w.imag], axis=-1)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(1)
    from synth.gen import rope_tables
    cos, sin = (t.astype(np.float64) for t in rope_tables(600, 128, 1e6))
    x = rng.standard_normal((9, 4, 128))
    pos = rng.integers(0, 600, 9)
    np.testing.assert_allclose(mdl.rope(x, pos, cos, sin), _rope_complex(x, pos, cos, sin),
                               rtol=1e-14, atol=1e-14)
    # position 0 is the identity; rotations keep norms; scores depend on m - n only
    # (the tables are float32, so cos^2 + sin^2 = 1 only to about 1e-7)
    np.testing.assert_allclose(mdl.rope(x, np.zeros(9, int), cos, sin), x, atol=0)
    np.testing.assert_allclose(np.linalg.norm(mdl.rope(x, pos, cos, sin), axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-7)
    q, k = x[:1], x[1:2]
    s1 = (mdl.rope(q, np.array([100]), cos, sin) * mdl.rope(k, np.array([90]), cos, sin)).sum()
    s2 = (mdl.rope(q, np.array([310]), cos, sin) * mdl.rope(k, np.array([300]), cos, sin)).sum()
    assert s1 == pytest.approx(s2, rel=1e-6)


# -------------------------------------------------------- chain vs library SDPA
def _chain_reference(inp, s, tokens):
    """Independent evaluation of one explicit token sequence (root first) after
    sequence s's prefix: numpy projections, complex-form RoPE, and torch's
    scaled_dot_product_attention with a causal-after-prefix boolean mask."""
    cfg = inp["cfg"]
    dt = cfg.dtype

    def f64(x):
        return torch.from_numpy(as_f32(np.asarray(x), dt).astype(np.float64))

    def st(x):  # storage rounding of bf16 runs, via torch's converter
        return x.to(torch.float32).to(torch.bfloat16).to(torch.float64) if dt == "bf16" else x

    n = len(tokens)
    P = int(inp["prefix_len"][s])
    a0, a1 = int(inp["kv_offsets"][s]), int(inp["kv_offsets"][s + 1])
    pos = P + np.arange(n)
    cos, sin = inp["rope_cos"].astype(np.float64), inp["rope_sin"].astype(np.float64)
    h = f64(inp["embed"][np.asarray(tokens)])
    attn, hs = [], []
    for lw in inp["layers"]:
        q = (h @ f64(lw["wq"]).T).numpy().reshape(n, cfg.Hq, cfg.D)
        k = (h @ f64(lw["wk"]).T).numpy().reshape(n, cfg.Hkv, cfg.D)
        v = (h @ f64(lw["wv"]).T).reshape(n, cfg.Hkv, cfg.D)
        q = torch.from_numpy(_rope_complex(q, pos, cos, sin))
        k = st(torch.from_numpy(_rope_complex(k, pos, cos, sin)))
        v = st(v)
        K = torch.cat([f64(lw["k_cache"][a0:a1]), k], 0)
        Vv = torch.cat([f64(lw["v_cache"][a0:a1]), v], 0)
        mask = torch.arange(P + n)[None, :] < (P + 1 + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(0, 1), K.transpose(0, 1), Vv.transpose(0, 1),
            attn_mask=mask, enable_gqa=True)
        a = o.transpose(0, 1).reshape(n, -1)
        h = st(h + a @ f64(lw["wo"]).T)
        attn.append(a.numpy())
        hs.append(h.numpy())
    return attn, hs


def _chain_paths(tokens):
    return [tuple(tokens[1:k + 1]) for k in range(len(tokens))]


@pytest.mark.parametrize("name,seed,tol", [("tiny", 1000, 1e-12), ("tiny_widehead", 1003, 1e-12),
                                           ("mini_bf16_ragged", 7, 2e-3)])
def test_chain_rows_match_sdpa(name, seed, tol):
    inp = gen_round(make_config(name), seed)
    cfg = inp["cfg"]
    model = mdl.TargetModel(inp)
    rng = np.random.default_rng(seed)
    for s in range(cfg.nseq):
        tokens = [int(t) for t in rng.integers(0, cfg.V, cfg.L + 1)]
        paths = _chain_paths(tokens)
        ev = mdl.evaluate_paths(model, s, tokens[0], paths)
        ra, rh = _chain_reference(inp, s, tokens)
        for li in range(cfg.n_layers):
            for got, want in ((ev["attn"][li], ra[li]), (ev["h"][li], rh[li])):
                err = np.abs(got - want).max() / np.abs(want).max()
                assert err <= tol, (li, err)


def test_single_position_hand_attention():
    """One query over a handful of keys: the softmax-weighted sum written out."""
    inp = gen_round(make_config("tiny"), 1002)
    m = mdl.TargetModel(inp)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((m.Hq, m.D))
    keys = rng.standard_normal((5, m.Hkv, m.D))
    vals = rng.standard_normal((5, m.Hkv, m.D))
    got = m.attend(q, keys, vals)
    for g in range(m.Hq):
        kv = g * m.Hkv // m.Hq
        w = [np.exp(sum(q[g][i] * keys[t, kv, i] for i in range(m.D)) / m.D ** 0.5) for t in range(5)]
        tot = sum(w)
        want = [sum(w[t] / tot * vals[t, kv, i] for t in range(5)) for i in range(m.D)]
        np.testing.assert_allclose(got[g], want, rtol=1e-12)


@pytest.mark.parametrize("name,seed", [("tiny", 1000), ("mini_bf16_ragged", 3)])
def test_tree_rows_equal_token_by_token_decoding(name, seed):
    """Every node of a round's tree, evaluated layer by layer over the whole
    tree, equals plain decoding of its own path one token at a time."""
    inp = gen_round(make_config(name), seed)
    cfg = inp["cfg"]
    model = mdl.TargetModel(inp)
    s = cfg.nseq - 1
    root = int(inp["rounds"][0]["root"][s])
    t = orr.build_tree(inp["rounds"][0]["draft_logits"][s], cfg.dtype, root, cfg.N)
    ev = mdl.evaluate_paths(model, s, root, t["order"])
    z_tree = model.logits(ev["final"])
    for i in list(range(0, len(t["order"]), 7)) + [len(t["order"]) - 1]:
        dec = mdl.Decoder(model, s)
        z = dec.extend(root)
        for y in t["order"][i]:
            z = dec.extend(y)
        np.testing.assert_allclose(z, z_tree[i], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dec.final, ev["final"][i], rtol=1e-12, atol=1e-14)


def test_teacher_forced_layers_reproduce_free_running():
    """Feeding every layer the rows the oracle itself produced before it gives
    back the free-running result exactly; feeding a perturbed layer input moves
    that layer and the ones after it, and no earlier one."""
    inp = gen_round(make_config("mini_bf16_ragged", n_layers=3), 3)
    cfg = inp["cfg"]
    model = mdl.TargetModel(inp)
    root = int(inp["rounds"][0]["root"][0])
    t = orr.build_tree(inp["rounds"][0]["draft_logits"][0], cfg.dtype, root, cfg.N)
    free = mdl.evaluate_paths(model, 0, root, t["order"])
    feeds = [None] + [free["h"][li - 1] for li in range(1, cfg.n_layers)]
    tf = mdl.evaluate_paths(model, 0, root, t["order"], layer_inputs=feeds)
    for li in range(cfg.n_layers):
        assert np.array_equal(tf["h"][li], free["h"][li])
        assert np.array_equal(tf["attn"][li], free["attn"][li])
    feeds[2] = free["h"][1] * 1.01
    moved = mdl.evaluate_paths(model, 0, root, t["order"], layer_inputs=feeds)
    assert np.array_equal(moved["h"][1], free["h"][1])
    assert not np.allclose(moved["attn"][2], free["attn"][2])


def test_rows_ignore_non_ancestors():
    """A row depends on its own path only: changing the other nodes leaves it
    unchanged (paper App. B.1: masking changes the layout, not the conditioning)."""
    inp = gen_round(make_config("tiny"), 1004)
    model = mdl.TargetModel(inp)
    a = [(), (3,), (3, 4), (5,), (5, 6), (5, 6, 7)]
    b = [(), (3,), (3, 4), (9,), (9, 1)]
    ea = mdl.evaluate_paths(model, 0, 11, a)
    eb = mdl.evaluate_paths(model, 0, 11, b)
    for i in range(3):
        assert np.array_equal(ea["final"][i], eb["final"][i])
    assert not np.allclose(ea["final"][3], eb["final"][3])


# -------------------------------------------------------------- LM head + stats
def test_logits_with_basis_head():
    """With W_head rows equal to unit vectors e_{v mod d}, z_v = h_{v mod d}."""
    inp = gen_round(make_config("tiny"), 1000)
    cfg = inp["cfg"]
    eye = np.zeros((cfg.V, cfg.d_model), dtype=np.float32)
    eye[np.arange(cfg.V), np.arange(cfg.V) % cfg.d_model] = 1.0
    inp2 = dict(inp, w_head=eye)
    m = mdl.TargetModel(inp2)
    h = np.random.default_rng(2).standard_normal((3, cfg.d_model))
    z = m.logits(h, chunk=100)
    np.testing.assert_array_equal(z, h[:, np.arange(cfg.V) % cfg.d_model])


def test_row_stats_closed_forms():
    V = 151936
    am, top1, gap, H = mdl.row_stats(np.zeros((1, V)))
    assert am[0] == 0 and gap[0] == 0 and H[0] == pytest.approx(np.log(V), abs=1e-9)
    am, top1, gap, H = mdl.row_stats(np.array([[-1e4, 3.0, 3.0, -1e4]]))
    assert am[0] == 1 and gap[0] == 0.0 and H[0] == pytest.approx(np.log(2), abs=1e-12)
    am, top1, gap, H = mdl.row_stats(np.array([[-5.0, 1.0, 0.75, 0.9]]))
    assert am[0] == 1 and top1[0] == 1.0 and gap[0] == pytest.approx(0.1, abs=1e-15)
    am, top1, gap, H = mdl.row_stats(np.array([[1e3, 0.0, 0.0]]))
    assert H[0] == pytest.approx(0.0, abs=1e-300)
    rng = np.random.default_rng(0)
    z = rng.standard_normal((6, 5000)) * [[0.05], [1], [3], [10], [30], [100]]
    am, top1, gap, H = mdl.row_stats(z)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(H, scipy.stats.entropy(p, axis=1), rtol=1e-9, atol=1e-12)
    srt = np.sort(z, axis=1)
    np.testing.assert_array_equal(gap, srt[:, -1] - srt[:, -2])
    np.testing.assert_array_equal(top1, srt[:, -1])
