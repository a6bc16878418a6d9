"""Unpacked evaluation of verify rows and the head's row statistics
(test infrastructure only).

What a verify row must equal (paper §3.2, Def. 1; App. B.1 proof; project page
"Verify pass"): the row of a depth-d node y_{1:d} is the target's next-token
distribution p(. | x o b o y_{1:d}); packing and ancestor-only masking change
the layout of the pass, never a row's conditioning.  So the oracle evaluates
every node on its own explicit token sequence b, y_1, .., y_d placed after the
cached prefix x, causally, with no tree and no mask matrix.

The pages do not define the target's layers.  The reading used here is an
attention-only residual stack over the given shapes:
  layer input   h = E[token] at the first layer (one embedding row per token)
  per layer     q = h Wq^T, k = h Wk^T, v = h Wv^T, split into heads of size D
                q and k rotated by rotate-half RoPE at absolute position
                P + (index in the sequence), from the given cos/sin tables
                query head g reads KV head floor(g / (Hq / Hkv))
                a = softmax(q k^T / sqrt(D)) v over [prefix keys, own keys <= pos]
                h' = h + concat_g(a_g) Wo^T
  logits        z = h_last W_head^T
Storage points of bf16 runs (values that a real engine keeps in bf16): the
K/V entry of every sequence position and each layer's output h'.  The oracle
rounds there and computes in float64 everywhere else.

Full layer (configs with an MLP; the pages name the target, Qwen3-VL-8B, but
not its layer internals, so this is the public decoder-layer shape of that
family):
  x   = RMSNorm(h) * g_attn                       (stored)
  q, k, v = x Wq^T, x Wk^T, x Wv^T; every q and k head normalised,
        RMSNorm(q_head) * g_q, RMSNorm(k_head) * g_k, then rotated (k stored)
  h1  = h + concat_g(a_g) Wo^T                    (stored)
  x2  = RMSNorm(h1) * g_mlp                       (stored)
  act = silu(x2 W_gate^T) * (x2 W_up^T)           (stored)
  h'  = h1 + act W_down^T                         (stored)
with RMSNorm(x) = x / sqrt(mean(x^2) + eps) and silu(z) = z / (1 + e^-z).

Row statistics (paper §3.1 greedy argmax; App. B.1 top-2 gap; §6 and the
project page's entropy law: next-token entropy H at the round root, in nats):
argmax (lowest token id on exact ties), top-1 logit, gap = top-1 minus the best
logit of any other token, and H = -sum_v p(v) ln p(v) with p = softmax(z).
"""
from __future__ import annotations

import numpy as np

from .numerics import decode, store


def rope(x: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half rotary embedding of x [..., n, H, D] at positions pos [n]:
    for i < D/2, (x_i, x_{i+D/2}) -> (x_i c - x_{i+D/2} s, x_{i+D/2} c + x_i s)
    with c, s = cos/sin tables at (pos, i)."""
    half = x.shape[-1] // 2
    c = cos[pos][:, None, :]
    s = sin[pos][:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (in float32 when x is
    float32, else float64)."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        x = x.astype(np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + x.dtype.type(eps)) * g.astype(x.dtype)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (z.dtype.type(1) + np.exp(-z))


class TargetModel:
    """Float64 view of the synthetic target's tensors, decoded on demand.

    ``compute="f32"`` evaluates the same definition with every operation between
    two storage points in float32 instead of float64 (the storage points, and the
    order of operations, are unchanged).  It is a second valid evaluation of the
    same model, used only to measure how far two correct implementations of a
    bf16 stack can drift apart from rounding alone; the tolerances of the
    comparisons are derived from that drift."""

    def __init__(self, inp: dict, cache_head: bool = False, compute: str = "f64"):
        if compute not in ("f64", "f32"):
            raise ValueError(compute)
        self.ft = np.float64 if compute == "f64" else np.float32
        cfg = inp["cfg"]
        self.cfg = cfg
        self.dtype = cfg.dtype
        self.V, self.d = cfg.V, cfg.d_model
        self.Hq, self.Hkv, self.D = cfg.Hq, cfg.Hkv, cfg.D
        self.n_layers = cfg.n_layers
        self.full = getattr(cfg, "mlp", 0) > 0
        self.eps = getattr(cfg, "norm_eps", 1e-6)
        self._inp = inp
        self.kv_offsets = np.asarray(inp["kv_offsets"], dtype=np.int64)
        self.prefix_len = np.asarray(inp["prefix_len"], dtype=np.int64)
        self.cos = np.asarray(inp["rope_cos"], dtype=self.ft)
        self.sin = np.asarray(inp["rope_sin"], dtype=self.ft)
        self._head64 = self._dec(inp["w_head"]) if cache_head else None
        self._layer_cache: dict = {}

    # ---------------------------------------------------------------- tensors
    def _dec(self, x) -> np.ndarray:
        """Stored tensor -> exact values in the compute type."""
        return decode(x, self.dtype).astype(self.ft, copy=False)

    def _store(self, x) -> np.ndarray:
        """Storage point: round to the storage format, back in the compute type."""
        return store(x, self.dtype).astype(self.ft, copy=False)

    def embed_rows(self, tokens) -> np.ndarray:
        return self._dec(self._inp["embed"][np.asarray(tokens, dtype=np.int64)])

    def layer(self, li: int) -> dict:
        if li not in self._layer_cache:
            lw = self._inp["layers"][li]
            names = ("wq", "wk", "wv", "wo")
            if self.full:
                names += ("g_attn", "g_q", "g_k", "g_mlp", "w_gate", "w_up", "w_down")
            self._layer_cache = {li: {k: self._dec(lw[k]) for k in names}}
        return self._layer_cache[li]

    def prefix_kv(self, li: int, s: int):
        lw = self._inp["layers"][li]
        a, b = int(self.kv_offsets[s]), int(self.kv_offsets[s + 1])
        return self._dec(lw["k_cache"][a:b]), self._dec(lw["v_cache"][a:b])

    def logits(self, h: np.ndarray, chunk: int = 8192) -> np.ndarray:
        """z = h W_head^T (float64, or float32 in the float32 mode; returned as
        float64), over vocabulary chunks."""
        h = np.atleast_2d(np.asarray(h, dtype=self.ft))
        z = np.empty((h.shape[0], self.V), dtype=np.float64)
        for a in range(0, self.V, chunk):
            b = min(a + chunk, self.V)
            w = self._head64[a:b] if self._head64 is not None else \
                self._dec(self._inp["w_head"][a:b])
            z[:, a:b] = h @ w.T
        return z

    # ------------------------------------------------------------- one layer
    def project(self, li: int, h: np.ndarray, pos: np.ndarray):
        """q (rotated), k (rotated, stored), v (stored) of rows h at positions pos."""
        w = self.layer(li)
        h = np.asarray(h, dtype=self.ft)
        n = h.shape[0]
        x = self._store(rmsnorm(h, w["g_attn"], self.eps)) if self.full else h
        q = (x @ w["wq"].T).reshape(n, self.Hq, self.D)
        k = (x @ w["wk"].T).reshape(n, self.Hkv, self.D)
        v = (x @ w["wv"].T).reshape(n, self.Hkv, self.D)
        if self.full:
            q = rmsnorm(q, w["g_q"], self.eps)
            k = rmsnorm(k, w["g_k"], self.eps)
        q = rope(q, pos, self.cos, self.sin)
        k = self._store(rope(k, pos, self.cos, self.sin))
        v = self._store(v)
        return q, k, v

    def attend(self, q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
        """Softmax attention of one position's query heads q [Hq][D] over an
        explicit key/value sequence [T][Hkv][D]; returns [Hq][D]."""
        G = self.Hq // self.Hkv
        out = np.empty((self.Hq, self.D), dtype=self.ft)
        for g in range(self.Hq):
            kv = g // G
            sc = keys[:, kv, :] @ q[g] / self.ft(np.sqrt(self.D))
            p = np.exp(sc - sc.max())
            p /= p.sum()
            out[g] = p @ vals[:, kv, :]
        return out

    def residual(self, li: int, h: np.ndarray, a: np.ndarray) -> np.ndarray:
        w = self.layer(li)
        h = np.asarray(h, dtype=self.ft)
        a = np.asarray(a, dtype=self.ft)
        h1 = self._store(h + a.reshape(a.shape[0], -1) @ w["wo"].T)
        if not self.full:
            return h1
        x2 = self._store(rmsnorm(h1, w["g_mlp"], self.eps))
        act = self._store(silu(x2 @ w["w_gate"].T) * (x2 @ w["w_up"].T))
        return self._store(h1 + act @ w["w_down"].T)


def evaluate_paths(model: TargetModel, s: int, root: int, paths: list,
                   layer_inputs: list | None = None) -> dict:
    """Evaluate every node of a prefix-closed set of token paths (the root is the
    empty path ()) on its own explicit sequence after sequence s's prefix.

    Layer by layer, every node's query attends to the prefix keys followed by the
    keys of its own path (root, y_1, .., y_d), i.e. exactly the causal sequence
    x o b o y_{1:d}; no other node is visible.  Returns per-layer attention
    outputs ``attn[l]`` [n][Hq*D], per-layer outputs ``h[l]`` [n][d] and the
    final hidden rows ``final`` [n][d], all float64, in the order of ``paths``.

    ``layer_inputs[l]`` (l >= 1), when given, replaces the rows entering layer l
    (in the order of ``paths``): each layer is then evaluated on exactly the
    inputs another implementation fed to it, which isolates that layer's error
    from the drift that bf16 storage accumulates over a deep stack."""
    index = {p: i for i, p in enumerate(paths)}
    if () not in index:
        raise ValueError("paths must contain the root ()")
    n = len(paths)
    tokens = [root if p == () else p[-1] for p in paths]
    P = int(model.prefix_len[s])
    pos = np.array([P + len(p) for p in paths], dtype=np.int64)
    chains = [[index[p[:j]] for j in range(len(p) + 1)] for p in paths]
    h = model.embed_rows(tokens)
    attn_all, h_all = [], []
    for li in range(model.n_layers):
        if layer_inputs is not None and li > 0 and layer_inputs[li] is not None:
            h = np.asarray(layer_inputs[li], dtype=model.ft)
        q, k, v = model.project(li, h, pos)
        Kp, Vp = model.prefix_kv(li, s)
        a = np.empty((n, model.Hq, model.D), dtype=model.ft)
        for i in range(n):
            keys = np.concatenate([Kp, k[chains[i]]], axis=0)
            vals = np.concatenate([Vp, v[chains[i]]], axis=0)
            a[i] = model.attend(q[i], keys, vals)
        attn_all.append(a.reshape(n, -1).astype(np.float64))
        h = model.residual(li, h, a)
        h_all.append(h.astype(np.float64))
    return {"attn": attn_all, "h": h_all, "final": h.astype(np.float64)}


class Decoder:
    """Plain autoregressive decoding of one sequence after its cached prefix:
    each ``extend(token)`` appends one position, evaluates it through every layer
    against the prefix and the sequence's own earlier positions, and returns the
    position's logits."""

    def __init__(self, model: TargetModel, s: int):
        self.m = model
        self.s = s
        self.P = int(model.prefix_len[s])
        self.keys = [[] for _ in range(model.n_layers)]
        self.vals = [[] for _ in range(model.n_layers)]
        self.kv = [model.prefix_kv(li, s) for li in range(model.n_layers)]
        self.final = None

    def extend(self, token: int) -> np.ndarray:
        m = self.m
        pos = np.array([self.P + len(self.keys[0])], dtype=np.int64)
        h = m.embed_rows([token])
        for li in range(m.n_layers):
            q, k, v = m.project(li, h, pos)
            self.keys[li].append(k[0])
            self.vals[li].append(v[0])
            Kp, Vp = self.kv[li]
            keys = np.concatenate([Kp, np.stack(self.keys[li])], axis=0)
            vals = np.concatenate([Vp, np.stack(self.vals[li])], axis=0)
            a = m.attend(q[0], keys, vals)[None]
            h = m.residual(li, h, a)
        self.final = h[0]
        return m.logits(h)[0]


def row_stats(z: np.ndarray):
    """argmax (lowest id on exact ties), top-1 logit, top-2 gap and entropy (nats)
    of every row of logits z [n][V]."""
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    am = np.argmax(z, axis=1)
    rows = np.arange(z.shape[0])
    top1 = z[rows, am]
    other = z.copy()
    other[rows, am] = -np.inf
    second = other.max(axis=1)
    gap = top1 - second
    lse = top1 + np.log(np.exp(z - top1[:, None]).sum(axis=1))
    lp = z - lse[:, None]
    p = np.exp(lp)
    H = -np.where(p > 0, p * lp, 0.0).sum(axis=1)
    return am.astype(np.int64), top1, gap, H
