"""Seeded synthetic workloads for one verify round.

Every tensor is drawn from its own NumPy ``Generator(PCG64)`` stream, spawned from
``SeedSequence(seed)`` in a fixed order (see ``_STREAMS``).  Values are drawn in
float32 and, for bf16 workloads, rounded to bfloat16 with round-to-nearest-even;
bf16 tensors are returned as ``uint16`` bit patterns.

Shapes follow the draft interface of the paper "Vision Is Not Overhead: One-Pass
Block Drafting for Lossless Speculative Decoding in Vision-Language Models"
(§3.2, Assumption 1: one marginal per offset j = 1..L; §4.1: block size B = 16,
so L = 15) and the verify budget of its project page ("Verify pass": N = 63, or
31 nodes plus the root).  The target shapes (d_model 4096, 32 query / 8 KV
heads, head_dim 128, vocabulary 151936) are those of an 8B Qwen3-family target.

Layouts (row-major, C order):
  draft_logits  [nseq][L][V]            f32 or bf16 bits
  root          [nseq]                  int32
  embed         [V][d_model]            token embedding, layer-0 input of every row
  w_head        [V][d_model]            LM head (out x in)
  layer i:  wq [Hq*D][d_model], wk/wv [Hkv*D][d_model], wo [d_model][Hq*D]
            k_cache/v_cache [sum P][Hkv][D] (already rotated; packed over sequences)
  kv_offsets    [nseq+1]                int64 prefix offsets into the packed cache
  rope_cos/sin  [n_pos][D/2]            float32 tables, angle = pos * theta**(-2i/D)
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Fixed order in which child streams are spawned from SeedSequence(seed).
_STREAMS = ("draft", "root", "embed", "head", "layers", "kv", "prefix", "extra", "mlp")
_CHUNK = 1 << 22  # elements per generation chunk (bounded temporaries)


# --------------------------------------------------------------------------- bf16
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.
    Inputs here are always finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_b = b.reshape(-1)
    flat_o = out.reshape(-1)
    tmp = np.empty(min(flat_b.size, _CHUNK), dtype=np.uint32)
    for s in range(0, flat_b.size, _CHUNK):
        e = min(s + _CHUNK, flat_b.size)
        t = tmp[: e - s]
        np.right_shift(flat_b[s:e], 16, out=t)
        np.bitwise_and(t, 1, out=t)
        np.add(t, 0x7FFF, out=t)
        np.add(t, flat_b[s:e], out=t)
        np.right_shift(t, 16, out=t)
        flat_o[s:e] = t
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------------ configs
@dataclass(frozen=True)
class RoundConfig:
    name: str
    dtype: str                      # "f32" or "bf16" storage of every tensor
    V: int
    L: int
    N: int
    d_model: int
    Hq: int
    Hkv: int
    D: int
    n_layers: int = 1
    nseq: int = 1
    prefix: tuple = ("fixed", 48)   # ("fixed", P) or ("uniform", lo, hi)
    draft: str = "spike"            # spike | scaled | planted | mixed | topology
    draft_scales: tuple = (1.0,)    # per-round scale for "scaled"
    n_rounds: int = 1
    w_std: float = 0.02             # Wq/Wk/Wv/Wo
    head_std: float = 0.02          # LM head
    embed_std: float = 0.02
    kv_std: float = 0.02
    rope_theta: float = 1.0e6
    spike: float = 6.0              # "spike": +spike on one token per position
    spike_sigma: float = 3.0        # "spike": z = spike_sigma * N(0,1) + spike
    planted_alpha: float = 4.0      # "planted": strength of the head's bigram bias
    planted_rho: float = 0.852      # "planted": P(G >= l) = rho**l, G <= L
    mixed_top: float = 50.0         # "mixed": spike on the last sequence
    mlp: int = 0                    # intermediate size of a full layer (0: attention only)
    mlp_std: float = 0.02           # W_gate / W_up / W_down
    gain_std: float = 0.1           # RMSNorm gains 1 + gain_std * N(0, 1)
    norm_eps: float = 1e-6

    @property
    def rows(self) -> int:          # verify rows per sequence: root + N nodes
        return self.N + 1

    def replace(self, **kw) -> "RoundConfig":
        return dataclasses.replace(self, **kw)


# Draft-logit scales of the single-layer 8B sweep.  The mean over offsets of the
# draft entropy H(softmax(s * N(0,1))) at V = 151936 is about 6, 4, 2, 1, 0.5 and
# 0.1 nats for these s (the low end varies with the draw, since there the gap
# between the two largest logits sets H); the CPU tests check the span.
C2_SCALES = (3.67, 4.61, 6.28, 8.44, 11.6, 45.0)

CONFIGS = {
    # Tiny fp32 round, brute-forceable tree (V=256, L=4, N=15, one layer).
    "tiny": RoundConfig(
        name="tiny", dtype="f32", V=256, L=4, N=15, d_model=64, Hq=2, Hkv=1,
        D=32, prefix=("fixed", 48), draft="spike", kv_std=0.02),
    # Same, with an N(0,1) LM head so that target top-2 gaps are large.
    "tiny_widehead": RoundConfig(
        name="tiny_widehead", dtype="f32", V=256, L=4, N=15, d_model=64, Hq=2,
        Hkv=1, D=32, prefix=("fixed", 48), draft="spike", head_std=1.0),
    # Single-layer 8B-shaped round, bf16 storage, draft-temperature sweep.
    "qwen8b_1layer": RoundConfig(
        name="qwen8b_1layer", dtype="bf16", V=151936, L=15, N=63, d_model=4096,
        Hq=32, Hkv=8, D=128, prefix=("fixed", 1024), draft="scaled",
        draft_scales=C2_SCALES, n_rounds=len(C2_SCALES), kv_std=1.0),
    # Grounded copy regime: planted draft run and a head biased to follow it.
    "qwen8b_copy": RoundConfig(
        name="qwen8b_copy", dtype="bf16", V=151936, L=15, N=31, d_model=4096,
        Hq=32, Hkv=8, D=128, prefix=("fixed", 4096), draft="planted",
        n_rounds=8, kv_std=1.0),
    # 36 stacked attention layers over an 8192-token prefix, given topology.
    "qwen8b_deep36": RoundConfig(
        name="qwen8b_deep36", dtype="bf16", V=151936, L=15, N=63, d_model=4096,
        Hq=32, Hkv=8, D=128, n_layers=36, prefix=("fixed", 8192),
        draft="topology", kv_std=1.0),
    # Ragged batch of 8 rounds, prefixes uniform in 512..6144.
    "qwen8b_ragged8": RoundConfig(
        name="qwen8b_ragged8", dtype="bf16", V=151936, L=15, N=63, d_model=4096,
        Hq=32, Hkv=8, D=128, nseq=8, prefix=("uniform", 512, 6144),
        draft="mixed", kv_std=1.0),
    # Reduced bf16 shapes that the CPU oracle evaluates in seconds while still
    # spanning several vocabulary tiles, prefix tiles and a ragged tail.
    "mini_bf16": RoundConfig(
        name="mini_bf16", dtype="bf16", V=20011, L=15, N=63, d_model=512,
        Hq=8, Hkv=2, D=128, prefix=("fixed", 333), draft="scaled",
        draft_scales=(3.0,), kv_std=1.0),
    # a full layer (RMSNorm, QK-norm, SwiGLU MLP) at reduced and at 8B shapes
    "mini_bf16_full": RoundConfig(
        name="mini_bf16_full", dtype="bf16", V=20011, L=15, N=63, d_model=512,
        Hq=4, Hkv=2, D=128, n_layers=2, mlp=1536, prefix=("fixed", 300), draft="scaled",
        draft_scales=(3.0,), kv_std=1.0, w_std=0.05, mlp_std=0.05),
    "qwen8b_full": RoundConfig(
        name="qwen8b_full", dtype="bf16", V=151936, L=15, N=63, d_model=4096,
        Hq=32, Hkv=8, D=128, mlp=12288, prefix=("fixed", 1024), draft="scaled",
        draft_scales=C2_SCALES, n_rounds=len(C2_SCALES), kv_std=1.0),
    "mini_bf16_ragged": RoundConfig(
        name="mini_bf16_ragged", dtype="bf16", V=9001, L=7, N=40, d_model=256,
        Hq=4, Hkv=1, D=128, n_layers=2, nseq=3, prefix=("uniform", 1, 700),
        draft="mixed", kv_std=1.0),
    "mini_bf16_copy": RoundConfig(
        name="mini_bf16_copy", dtype="bf16", V=4099, L=15, N=31, d_model=256,
        Hq=4, Hkv=2, D=128, prefix=("fixed", 200), draft="planted", n_rounds=4,
        kv_std=1.0),
}


def make_config(name: str, **overrides) -> RoundConfig:
    return CONFIGS[name].replace(**overrides)


# ---------------------------------------------------------------------- helpers
class _Streams:
    def __init__(self, seed: int):
        kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
        self._seq = dict(zip(_STREAMS, kids))

    def rng(self, name: str, *sub: int) -> np.random.Generator:
        ss = self._seq[name]
        for i in sub:
            ss = np.random.SeedSequence(ss.entropy, spawn_key=ss.spawn_key + (i,))
        return np.random.Generator(np.random.PCG64(ss))


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    """std * N(0,1) drawn in float32 chunks; bf16 storage returns bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    buf = np.empty(min(n, _CHUNK), dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(s + _CHUNK, n)
        t = buf[: e - s]
        rng.standard_normal(out=t, dtype=np.float32)
        if std != 1.0:
            np.multiply(t, np.float32(std), out=t)
        out[s:e] = bf16_bits(t) if dtype == "bf16" else t
    return out.reshape(shape)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float32 values."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else x


def rope_tables(n_pos: int, D: int, theta: float):
    """cos/sin of pos * theta**(-2i/D), i < D/2, built in float64, stored float32."""
    half = D // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / D)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _prefix_lengths(cfg: RoundConfig, st: _Streams) -> np.ndarray:
    kind = cfg.prefix[0]
    if kind == "fixed":
        return np.full(cfg.nseq, int(cfg.prefix[1]), dtype=np.int64)
    lo, hi = int(cfg.prefix[1]), int(cfg.prefix[2])
    return st.rng("prefix").integers(lo, hi + 1, size=cfg.nseq).astype(np.int64)


# ------------------------------------------------------------------- draft logits
def _draft_spike(cfg, rng):
    z = rng.standard_normal((cfg.nseq, cfg.L, cfg.V)).astype(np.float32)
    z *= np.float32(cfg.spike_sigma)
    hot = rng.integers(0, cfg.V, size=(cfg.nseq, cfg.L))
    for s in range(cfg.nseq):
        for j in range(cfg.L):
            z[s, j, hot[s, j]] += np.float32(cfg.spike)
    return z


def _draft_scaled(cfg, rng, scale):
    z = np.empty((cfg.nseq, cfg.L, cfg.V), dtype=np.float32)
    rng.standard_normal(out=z, dtype=np.float32)
    z *= np.float32(scale)
    return z


def _draft_mixed(cfg, rng):
    """Per-sequence scales log-spaced from near-uniform (0.1) up to 6, and a
    one-hot spike (+mixed_top over N(0,1)) on the last sequence."""
    z = np.empty((cfg.nseq, cfg.L, cfg.V), dtype=np.float32)
    rng.standard_normal(out=z, dtype=np.float32)
    n_scaled = max(cfg.nseq - 1, 1)
    scales = np.geomspace(0.1, 6.0, n_scaled)
    for s in range(cfg.nseq):
        if s < cfg.nseq - 1 or cfg.nseq == 1:
            z[s] *= np.float32(scales[min(s, n_scaled - 1)])
        else:
            hot = rng.integers(0, cfg.V, size=cfg.L)
            for j in range(cfg.L):
                z[s, j, hot[j]] += np.float32(cfg.mixed_top)
    return z


def _draft_planted(cfg, rng, tokens, mu):
    """Position j puts mass mu_j on planted token tokens[j]; the remaining mass
    1 - mu_j follows softmax of N(0,1) logits over the other tokens.  Stored as
    logits: z_t = ln(mu/(1-mu)) + ln(sum_{v != t} exp(g_v)), z_v = g_v."""
    z = np.empty((cfg.L, cfg.V), dtype=np.float32)
    for j in range(cfg.L):
        g = rng.standard_normal(cfg.V)
        t = int(tokens[j])
        rest = np.delete(g, t)
        mx = rest.max()
        lse = mx + np.log(np.exp(rest - mx).sum())
        g[t] = np.log(mu[j] / (1.0 - mu[j])) + lse
        z[j] = g.astype(np.float32)
    return z


# --------------------------------------------------------------------- topology
def random_tree(rng: np.random.Generator, N: int, L: int, V: int, root: int):
    """Random prefix-closed tree of N nodes and depth <= L, laid out breadth-first
    with rows sorted by (depth, parent row, token); row 0 is the root.  Returns
    parent, depth, token (int32 [N+1]) and anc (uint64 [N+1], bit j of row i set
    iff row j is row i or one of its ancestors)."""
    paths = [()]
    kids = {(): set()}
    for _ in range(N):
        cand = [p for p in paths if len(p) < L and len(kids[p]) < V]
        if not cand:
            raise ValueError("no room for another node")
        par = cand[int(rng.integers(0, len(cand)))]
        while True:
            t = int(rng.integers(0, V))
            if t not in kids[par]:
                break
        kids[par].add(t)
        child = par + (t,)
        paths.append(child)
        kids[child] = set()
    order = sorted(paths, key=lambda p: (len(p), p))
    row = {p: i for i, p in enumerate(order)}
    parent = np.array([-1] + [row[p[:-1]] for p in order[1:]], dtype=np.int32)
    depth = np.array([len(p) for p in order], dtype=np.int32)
    token = np.array([root] + [p[-1] for p in order[1:]], dtype=np.int32)
    anc = np.zeros(N + 1, dtype=np.uint64)
    anc[0] = np.uint64(1)
    for i in range(1, N + 1):
        anc[i] = anc[parent[i]] | np.uint64(1 << i)
    return parent, depth, token, anc


# ------------------------------------------------------------------------ rounds
def gen_round(cfg: RoundConfig, seed: int, with_model: bool = True, model: dict | None = None) -> dict:
    """Draw every input of ``cfg.n_rounds`` verify rounds that share one model.

    Returns a dict with the model tensors (``embed``, ``w_head``, ``layers``,
    ``kv_offsets``, ``prefix_len``, ``rope_cos``, ``rope_sin``) and a list
    ``rounds`` of per-round dicts (``draft_logits`` or a given tree, ``root``,
    plus recipe metadata such as the draft scale or the planted run).

    ``model``: the output of an earlier call for a config of the same shapes and
    weight distributions; its embedding, head and layer weights are reused (the
    layers cyclically) instead of drawn again, and only the prefix caches, the
    rounds and, in the copy regime, the biased head rows (on a copy) are new."""
    st = _Streams(seed)
    dt = cfg.dtype
    out: dict = {"cfg": cfg, "seed": seed}

    P = _prefix_lengths(cfg, st)
    kv_off = np.zeros(cfg.nseq + 1, dtype=np.int64)
    kv_off[1:] = np.cumsum(P)
    out["prefix_len"] = P
    out["kv_offsets"] = kv_off

    rounds = []
    r_draft = st.rng("draft")
    r_root = st.rng("root")
    r_extra = st.rng("extra")
    used_tokens: set = set()
    plant_bias = []  # (row, source_row, alpha)
    for r in range(cfg.n_rounds):
        rd: dict = {}
        if cfg.draft == "planted":
            assert cfg.nseq == 1
            # root, L planted tokens and one break token, all distinct across rounds
            toks = []
            while len(toks) < cfg.L + 2:
                t = int(r_extra.integers(0, cfg.V))
                if t not in used_tokens:
                    used_tokens.add(t)
                    toks.append(t)
            root, planted, brk = toks[0], toks[1:cfg.L + 1], toks[cfg.L + 1]
            mu = r_extra.uniform(0.9, 0.99, size=cfg.L)
            G = 0
            while G < cfg.L and r_extra.uniform() < cfg.planted_rho:
                G += 1
            z = _draft_planted(cfg, r_draft, planted, mu)[None]
            chain = [root] + planted[:G]
            for k in range(G):
                plant_bias.append((planted[k], chain[k]))
            plant_bias.append((brk, chain[G]))
            rd.update(root=np.array([root], dtype=np.int32), planted=np.array(planted),
                      mu=mu, G=G, break_token=brk)
            rd["draft_logits"] = _store(z, dt)
        elif cfg.draft == "topology":
            roots = r_root.integers(0, cfg.V, size=cfg.nseq).astype(np.int32)
            trees = [random_tree(r_extra, cfg.N, cfg.L, cfg.V, int(roots[s]))
                     for s in range(cfg.nseq)]
            rd["root"] = roots
            rd["parent"] = np.stack([t[0] for t in trees])
            rd["depth"] = np.stack([t[1] for t in trees])
            rd["token"] = np.stack([t[2] for t in trees])
            rd["anc"] = np.stack([t[3] for t in trees])
        else:
            rd["root"] = r_root.integers(0, cfg.V, size=cfg.nseq).astype(np.int32)
            if cfg.draft == "spike":
                z = _draft_spike(cfg, r_draft)
            elif cfg.draft == "scaled":
                scale = cfg.draft_scales[r % len(cfg.draft_scales)]
                rd["scale"] = scale
                z = _draft_scaled(cfg, r_draft, scale)
            elif cfg.draft == "mixed":
                z = _draft_mixed(cfg, r_draft)
            else:
                raise ValueError(cfg.draft)
            rd["draft_logits"] = _store(z, dt)
        rounds.append(rd)
    out["rounds"] = rounds

    if not with_model:
        return out

    if model is not None:
        assert model["embed"].shape == (cfg.V, cfg.d_model) and model["embed"].dtype == _store(
            np.zeros((1, 1), np.float32), dt).dtype, "the reused model has other shapes"
        out["embed"] = model["embed"]
        w_head = model["w_head"].copy() if plant_bias else model["w_head"]
    else:
        out["embed"] = _normal(st.rng("embed"), (cfg.V, cfg.d_model), cfg.embed_std, dt)
        w_head = _normal(st.rng("head"), (cfg.V, cfg.d_model), cfg.head_std, dt)
    if plant_bias:
        # Bigram bias of the copy regime: row t_{k+1} of the head gains
        # alpha * E[t_k] / |E[t_k]|^2, so the greedy continuation follows the run.
        emb32 = as_f32(out["embed"], dt)
        for row, src in plant_bias:
            e = emb32[src].astype(np.float64)
            w = as_f32(w_head[row:row + 1], dt)[0].astype(np.float64)
            w = w + cfg.planted_alpha * e / float(e @ e)
            w_head[row] = _store(w.astype(np.float32)[None], dt)[0]
    out["w_head"] = w_head

    layers = []
    qd, kd = cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    sumP = int(kv_off[-1])
    for li in range(cfg.n_layers):
        rw = st.rng("layers", li)
        rk = st.rng("kv", li)
        if model is not None:
            src = model["layers"][li % len(model["layers"])]
            assert src["wq"].shape == (qd, cfg.d_model), "the reused model has other shapes"
            layers.append({k: v for k, v in src.items() if k not in ("k_cache", "v_cache")})
            layers[-1]["k_cache"] = _normal(rk, (sumP, cfg.Hkv, cfg.D), cfg.kv_std, dt)
            layers[-1]["v_cache"] = _normal(rk, (sumP, cfg.Hkv, cfg.D), cfg.kv_std, dt)
            continue
        layers.append({
            "wq": _normal(rw, (qd, cfg.d_model), cfg.w_std, dt),
            "wk": _normal(rw, (kd, cfg.d_model), cfg.w_std, dt),
            "wv": _normal(rw, (kd, cfg.d_model), cfg.w_std, dt),
            "wo": _normal(rw, (cfg.d_model, qd), cfg.w_std, dt),
            "k_cache": _normal(rk, (sumP, cfg.Hkv, cfg.D), cfg.kv_std, dt),
            "v_cache": _normal(rk, (sumP, cfg.Hkv, cfg.D), cfg.kv_std, dt),
        })
        if cfg.mlp > 0:
            # full layer: RMSNorm gains (input, per q/k head, before the MLP) and
            # the gate/up/down projections, from a stream of their own
            rm = st.rng("mlp", li)
            gain = lambda n: _store((1.0 + cfg.gain_std * rm.standard_normal(n)).astype(np.float32), dt)
            layers[-1].update({
                "g_attn": gain(cfg.d_model), "g_q": gain(cfg.D), "g_k": gain(cfg.D),
                "g_mlp": gain(cfg.d_model),
                "w_gate": _normal(rm, (cfg.mlp, cfg.d_model), cfg.mlp_std, dt),
                "w_up": _normal(rm, (cfg.mlp, cfg.d_model), cfg.mlp_std, dt),
                "w_down": _normal(rm, (cfg.d_model, cfg.mlp), cfg.mlp_std, dt),
            })
    out["layers"] = layers
    # a row of the table for every position P + depth a verify row can take
    # (depth < N + 1 rows), so that tables cover max prefix + rows
    n_pos = int(P.max()) + max(cfg.L, cfg.N) + 1
    out["rope_cos"], out["rope_sin"] = rope_tables(n_pos, cfg.D, cfg.rope_theta)
    return out
