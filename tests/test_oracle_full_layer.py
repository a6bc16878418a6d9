"""Pins of the oracle's full layer (RMSNorm, per-head QK-norm, SwiGLU MLP; the
public decoder-layer shape of the target family the paper names): the norm's
invariants, SiLU against SciPy's logistic function, unit-RMS q/k heads, an MLP
that vanishes with a zero gate or up projection, bf16 storage points, tree
rows that equal token-by-token decoding through full layers, and chains equal
to an independent torch float64 evaluation with non-unit gains (which a
gate/up swap, the q/k norm after the rotation or a mis-wired residual fail)."""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import model as mdl, round as orr
from oracle.numerics import round_bf16
from synth import gen_round, make_config
from synth.gen import as_f32


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


# ------------------------------------------- full layers vs an independent chain
def _full_chain_reference(inp, s, tokens):
    """Independent torch float64 evaluation of one explicit token sequence (root
    first) after sequence s's prefix through full decoder layers: RMSNorm written
    out as x * rsqrt(mean(x^2) + eps) * g, per-head q/k norm before the rotary
    embedding (complex-number form), torch's scaled_dot_product_attention with
    grouped heads and a causal-after-prefix mask, torch's SiLU, and the two
    residual additions (attention, then MLP on the attention's output)."""
    cfg = inp["cfg"]
    dt = cfg.dtype
    F = torch.nn.functional

    def f64(x):
        return torch.from_numpy(as_f32(np.asarray(x), dt).astype(np.float64))

    def st(x):  # bf16 storage point through torch's converter (identity for fp32)
        return x.to(torch.float32).to(torch.bfloat16).to(torch.float64) if dt == "bf16" else x

    def norm(x, g):
        return x * torch.rsqrt((x * x).mean(dim=-1, keepdim=True) + cfg.norm_eps) * g

    def rot(x, pos):  # x [n][H][D]: pairs (i, i + D/2) as complex numbers
        half = x.shape[-1] // 2
        c = torch.from_numpy(inp["rope_cos"][pos].astype(np.float64))[:, None, :]
        sn = torch.from_numpy(inp["rope_sin"][pos].astype(np.float64))[:, None, :]
        z = torch.complex(x[..., :half], x[..., half:]) * torch.complex(c, sn)
        return torch.cat([z.real, z.imag], dim=-1)

    n = len(tokens)
    P = int(inp["prefix_len"][s])
    a0, a1 = int(inp["kv_offsets"][s]), int(inp["kv_offsets"][s + 1])
    pos = P + np.arange(n)
    h = f64(inp["embed"][np.asarray(tokens)])
    mask = torch.arange(P + n)[None, :] < (P + 1 + torch.arange(n))[:, None]
    hs = []
    for lw in inp["layers"]:
        x = st(norm(h, f64(lw["g_attn"])))
        q = norm((x @ f64(lw["wq"]).T).reshape(n, cfg.Hq, cfg.D), f64(lw["g_q"]))
        k = norm((x @ f64(lw["wk"]).T).reshape(n, cfg.Hkv, cfg.D), f64(lw["g_k"]))
        v = st((x @ f64(lw["wv"]).T).reshape(n, cfg.Hkv, cfg.D))
        q, k = rot(q, pos), st(rot(k, pos))
        K = torch.cat([f64(lw["k_cache"][a0:a1]), k], 0)
        Vv = torch.cat([f64(lw["v_cache"][a0:a1]), v], 0)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), K.transpose(0, 1), Vv.transpose(0, 1),
                                           attn_mask=mask, enable_gqa=True)
        h1 = st(h + o.transpose(0, 1).reshape(n, -1) @ f64(lw["wo"]).T)
        x2 = st(norm(h1, f64(lw["g_mlp"])))
        act = st(F.silu(x2 @ f64(lw["w_gate"]).T) * (x2 @ f64(lw["w_up"]).T))
        h = st(h1 + act @ f64(lw["w_down"]).T)
        hs.append(h.numpy())
    return hs


def _full_chain_error(inp, model, seed):
    """Largest norm-wise difference between the oracle's rows and the chain
    reference's, over every layer of one random chain per sequence."""
    cfg = inp["cfg"]
    rng = np.random.default_rng(seed)
    worst = 0.0
    for s in range(cfg.nseq):
        tokens = [int(t) for t in rng.integers(0, cfg.V, cfg.L + 1)]
        paths = [tuple(tokens[1:k + 1]) for k in range(len(tokens))]
        ev = mdl.evaluate_paths(model, s, tokens[0], paths)
        ref = _full_chain_reference(inp, s, tokens)
        for li in range(cfg.n_layers):
            worst = max(worst, float(np.abs(ev["h"][li] - ref[li]).max() / np.abs(ref[li]).max()))
    return worst


# tiny fp32 full layers agree to rounding; the bf16 run differs only where
# torch's two-step conversion (float64 -> float32 -> bf16) and the oracle's
# direct rounding disagree on a near-halfway value (one bf16 ulp of an element)
_FULL_CASES = [("tiny", dict(mlp=96, n_layers=2), 21, 1e-12), ("mini_bf16_full", {}, 22, 1e-2)]


@pytest.mark.parametrize("name,over,seed,tol", _FULL_CASES)
def test_full_layer_rows_match_independent_chain(name, over, seed, tol):
    inp = gen_round(make_config(name, **over), seed)
    gains = inp["layers"][0]["g_q"]
    assert np.abs(as_f32(gains, inp["cfg"].dtype) - 1.0).max() > 0.05   # gains are not unit
    assert _full_chain_error(inp, mdl.TargetModel(inp), seed) <= tol


class _GateUpSwapped(mdl.TargetModel):
    def residual(self, li, h, a):
        w = self.layer(li)
        h1 = self._store(h + a.reshape(a.shape[0], -1) @ w["wo"].T)
        x2 = self._store(mdl.rmsnorm(h1, w["g_mlp"], self.eps))
        act = self._store(mdl.silu(x2 @ w["w_up"].T) * (x2 @ w["w_gate"].T))
        return self._store(h1 + act @ w["w_down"].T)


class _NormAfterRope(mdl.TargetModel):
    def project(self, li, h, pos):
        w = self.layer(li)
        n = h.shape[0]
        x = self._store(mdl.rmsnorm(h, w["g_attn"], self.eps))
        q = (x @ w["wq"].T).reshape(n, self.Hq, self.D)
        k = (x @ w["wk"].T).reshape(n, self.Hkv, self.D)
        v = (x @ w["wv"].T).reshape(n, self.Hkv, self.D)
        q = mdl.rmsnorm(mdl.rope(q, pos, self.cos, self.sin), w["g_q"], self.eps)
        k = self._store(mdl.rmsnorm(mdl.rope(k, pos, self.cos, self.sin), w["g_k"], self.eps))
        return q, k, self._store(v)


class _MlpOnLayerInput(mdl.TargetModel):
    def residual(self, li, h, a):
        w = self.layer(li)
        h1 = self._store(h + a.reshape(a.shape[0], -1) @ w["wo"].T)
        x2 = self._store(mdl.rmsnorm(h, w["g_mlp"], self.eps))   # wired to h, not h1
        act = self._store(mdl.silu(x2 @ w["w_gate"].T) * (x2 @ w["w_up"].T))
        return self._store(h1 + act @ w["w_down"].T)


@pytest.mark.parametrize("name,over,seed,tol", _FULL_CASES)
@pytest.mark.parametrize("mutant", [_GateUpSwapped, _NormAfterRope, _MlpOnLayerInput])
def test_chain_pin_catches_planted_mistakes(name, over, seed, tol, mutant):
    """The chain pin is sharp: an oracle with the gate and up projections
    swapped, the q/k norm applied after the rotation, or the MLP reading the
    layer input instead of the attention's output fails it by far."""
    inp = gen_round(make_config(name, **over), seed)
    assert _full_chain_error(inp, mutant(inp), seed) > max(10 * tol, 1e-3)
