"""Pins of the oracle's full layer (RMSNorm, per-head QK-norm, SwiGLU MLP; the
public decoder-layer shape of the target family the paper names): the norm's
invariants, SiLU against SciPy's logistic function, unit-RMS q/k heads, an MLP
that vanishes with a zero gate or up projection, bf16 storage points, and tree
rows that equal token-by-token decoding through full layers."""
import numpy as np
import pytest
import scipy.special

from oracle import model as mdl, round as orr
from oracle.numerics import round_bf16
from synth import gen_round, make_config


def test_rmsnorm_invariants():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 3.0, (5, 64))
    g = np.ones(64)
    y = mdl.rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)   # unit RMS
    np.testing.assert_allclose(mdl.rmsnorm(7.5 * x, g, 0.0), y, rtol=1e-13)  # scale-free
    gg = rng.normal(1, 0.2, 64)
    np.testing.assert_allclose(mdl.rmsnorm(x, gg, 0.0), y * gg, rtol=1e-13)  # gain per feature
    c = np.full((1, 16), -2.0)
    np.testing.assert_allclose(mdl.rmsnorm(c, np.arange(16.0), 0.0), -np.arange(16.0)[None], atol=1e-15)
    # eps only matters for small rows
    small = np.full((1, 8), 1e-4)
    assert mdl.rmsnorm(small, np.ones(8), 1e-6)[0, 0] < 0.1


def test_silu_against_logistic():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(mdl.silu(z), z * scipy.special.expit(z), rtol=1e-12, atol=1e-300)
    assert mdl.silu(np.array([0.0]))[0] == 0.0


@pytest.fixture(scope="module")
def tiny_full():
    return gen_round(make_config("tiny", mlp=96, n_layers=2), 11)


def test_full_layer_tensors_and_storage_points(tiny_full):
    inp = gen_round(make_config("mini_bf16_full"), 2)
    model = mdl.TargetModel(inp)
    assert model.full
    w = model.layer(0)
    assert w["w_gate"].shape == (1536, 512) and w["w_down"].shape == (512, 1536)
    rng = np.random.default_rng(1)
    h = round_bf16(rng.normal(0, 1, (3, 512)))
    a = rng.normal(0, 1, (3, 4, 128))
    out = model.residual(0, h, a)
    assert np.array_equal(round_bf16(out), out)   # the layer output is a storage point


def test_qk_heads_have_unit_rms_with_unit_gains(tiny_full):
    inp = dict(tiny_full)
    inp["layers"] = [dict(lw) for lw in inp["layers"]]
    for lw in inp["layers"]:
        lw["g_q"] = np.ones_like(lw["g_q"])
        lw["g_k"] = np.ones_like(lw["g_k"])
    model = mdl.TargetModel(inp)
    cfg = inp["cfg"]
    rng = np.random.default_rng(2)
    h = rng.normal(0, 1, (4, cfg.d_model))
    q, k, v = model.project(0, h, np.array([3, 4, 5, 6]))
    # RoPE is a rotation, so the normalised heads keep RMS 1 up to eps / mean(x^2)
    # (about 4e-5 here; the raw heads have a mean square near 0.03)
    np.testing.assert_allclose(np.mean(q * q, axis=-1), 1.0, rtol=1e-3)
    np.testing.assert_allclose(np.mean(k * k, axis=-1), 1.0, rtol=1e-3)
    # v is not normalised: it is the plain projection of the normalised input
    w = model.layer(0)
    x = mdl.rmsnorm(h, w["g_attn"], cfg.norm_eps)
    np.testing.assert_allclose(v.reshape(4, -1), x @ w["wv"].T, rtol=1e-12)


@pytest.mark.parametrize("zero", ["w_gate", "w_up"])
def test_mlp_vanishes_with_a_zero_branch(tiny_full, zero):
    inp = dict(tiny_full)
    inp["layers"] = [dict(lw) for lw in inp["layers"]]
    inp["layers"][0][zero] = np.zeros_like(inp["layers"][0][zero])
    full = mdl.TargetModel(inp)
    rng = np.random.default_rng(3)
    cfg = inp["cfg"]
    h = rng.normal(0, 1, (2, cfg.d_model))
    a = rng.normal(0, 1, (2, cfg.Hq, cfg.D))
    w = full.layer(0)
    h1 = h + a.reshape(2, -1) @ w["wo"].T
    np.testing.assert_allclose(full.residual(0, h, a), h1, rtol=1e-12)


@pytest.mark.parametrize("name,seed,over", [("tiny", 5, dict(mlp=96, n_layers=2)),
                                            ("mini_bf16_full", 6, {})])
def test_full_tree_rows_equal_token_by_token_decoding(name, seed, over):
    inp = gen_round(make_config(name, **over), seed)
    cfg = inp["cfg"]
    model = mdl.TargetModel(inp)
    root = int(inp["rounds"][0]["root"][0])
    t = orr.build_tree(inp["rounds"][0]["draft_logits"][0], cfg.dtype, root, cfg.N)
    ev = mdl.evaluate_paths(model, 0, root, t["order"])
    z_tree = model.logits(ev["final"])
    for i in list(range(0, len(t["order"]), 9)) + [len(t["order"]) - 1]:
        dec = mdl.Decoder(model, 0)
        z = dec.extend(root)
        for y in t["order"][i]:
            z = dec.extend(y)
        np.testing.assert_allclose(z, z_tree[i], rtol=1e-12, atol=1e-14)
