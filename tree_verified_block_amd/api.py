"""Torch-tensor front end of the C ABI: the same four calls, argument
marshalling only (device pointers, sizes, the current HIP stream).  Every step
runs in libglance's HIP kernels; PyTorch only provides memory and streams."""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import GLANCE_BF16, GLANCE_F32, GlanceAttnLayer, GlanceFullLayer, GlanceWalk


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GLANCE_F32
    if t.dtype == torch.bfloat16:
        return GLANCE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace (the library's arrival counters start at zero and
    every call leaves them at zero)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ step 1 + 2
def build_tree_ws_bytes(nseq: int, L: int, V: int, N: int) -> int:
    return _lib.load().glance_build_tree_ws(nseq, L, V, N)


def build_tree_flags(ws: torch.Tensor, nseq: int, L: int, V: int, N: int) -> int:
    """The workspace's sticky non-finite flag word (bit 0: a NaN draft logit was
    read, bit 1: a +inf one) as a Python int; synchronises with the device."""
    off = _lib.load().glance_build_tree_flag_offset(nseq, L, V, N)
    if off == 0:
        raise ValueError("invalid tree sizes")
    return int(ws[off:off + 4].view(torch.int32).item()) & 0xFFFFFFFF


def tree_outputs(nseq: int, N: int, device) -> dict:
    """The tree outputs, allocated as an empty tree (every row padding), so that
    a layer call before the first tree build reads only valid tokens."""
    R = N + 1
    return {
        "parent": torch.full((nseq, R), -1, dtype=torch.int32, device=device),
        "depth": torch.zeros((nseq, R), dtype=torch.int32, device=device),
        "token": torch.full((nseq, R), -1, dtype=torch.int32, device=device),
        "anc": torch.zeros((nseq, R), dtype=torch.int64, device=device),
        "score": torch.zeros((nseq, R), dtype=torch.float32, device=device),
        "n_valid": torch.zeros((nseq,), dtype=torch.int32, device=device),
    }


def glance_build_tree(draft_logits, root_token, N, out, ws, stream=None):
    nseq, L, V = draft_logits.shape
    _lib.call("glance_build_tree", _ptr(draft_logits), dtype_code(draft_logits),
              _ptr(root_token), nseq, L, V, N, _ptr(out["parent"]), _ptr(out["depth"]),
              _ptr(out["token"]), _ptr(out["anc"]), _ptr(out["score"]), _ptr(out["n_valid"]),
              _ptr(ws), ws.numel(), _stream(stream))
    return out


def glance_build_tree_shared(draft_logits, root_token, log_weight, n_max, budget, out, ws,
                             min_log_value=float("-inf"), stream=None):
    """Trees of a batch of rounds under one shared node budget (out as from
    tree_outputs(nseq, n_max))."""
    nseq, L, V = draft_logits.shape
    _lib.call("glance_build_tree_shared", _ptr(draft_logits), dtype_code(draft_logits),
              _ptr(root_token), _ptr(log_weight), nseq, L, V, n_max, budget, float(min_log_value),
              _ptr(out["parent"]), _ptr(out["depth"]), _ptr(out["token"]), _ptr(out["anc"]),
              _ptr(out["score"]), _ptr(out["n_valid"]), _ptr(ws), ws.numel(), _stream(stream))
    return out


def glance_entropy_log_value(entropy, b0: float, b1: float, L: int, log_weight, nseq=None,
                             stride: int = 1, stream=None):
    """ln V(H) of the entropy law for each round's root entropy (float32 device
    tensors; H_s = entropy.flatten()[s * stride])."""
    n = log_weight.numel() if nseq is None else nseq
    _lib.call("glance_entropy_log_value", _ptr(entropy), n, stride, float(b0), float(b1), int(L),
              _ptr(log_weight), _stream(stream))


# ---------------------------------------------------------------------- step 3
def tree_attn_ws_bytes(nseq, n_rows, max_prefix, d_model, Hq, Hkv, D) -> int:
    return _lib.load().glance_tree_attn_ws(nseq, n_rows, max_prefix, d_model, Hq, Hkv, D)


def glance_tree_attn(layer: dict, dtype: int, embed, token, h_in, h_out, kv_offsets,
                     max_prefix: int, depth, anc, rope_cos, rope_sin, nseq: int, n_rows: int,
                     d_model: int, Hq: int, Hkv: int, D: int, ws, attn_out=None, tree_k=None,
                     tree_v=None, stream=None):
    lay = GlanceAttnLayer(_ptr(layer["wq"]), _ptr(layer["wk"]), _ptr(layer["wv"]),
                          _ptr(layer["wo"]), _ptr(layer["k_cache"]), _ptr(layer["v_cache"]),
                          _ptr(layer.get("attn_packed")))
    _lib.call("glance_tree_attn", ctypes.byref(lay), dtype, _ptr(embed), _ptr(token),
              _ptr(h_in), _ptr(h_out), _ptr(kv_offsets), int(max_prefix), _ptr(depth),
              _ptr(anc), _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], nseq, n_rows,
              d_model, Hq, Hkv, D, _ptr(attn_out), _ptr(tree_k), _ptr(tree_v), _ptr(ws),
              ws.numel(), _stream(stream))


def tree_layer_ws_bytes(nseq, n_rows, max_prefix, d_model, Hq, Hkv, D, inter) -> int:
    return _lib.load().glance_tree_layer_ws(nseq, n_rows, max_prefix, d_model, Hq, Hkv, D, inter)


def glance_tree_layer(layer: dict, eps: float, embed, token, h_in, h_out, kv_offsets,
                      max_prefix: int, depth, anc, rope_cos, rope_sin, nseq: int, n_rows: int,
                      d_model: int, Hq: int, Hkv: int, D: int, ws, attn_out=None, tree_k=None,
                      tree_v=None, stream=None):
    """One full decoder layer (RMSNorm, QK-norm, attention, SwiGLU MLP) over the
    verify rows; ``layer`` holds wq/wk/wv/wo, the caches, g_attn/g_q/g_k/g_mlp and
    w_gate/w_up/w_down (bf16)."""
    attn = GlanceAttnLayer(_ptr(layer["wq"]), _ptr(layer["wk"]), _ptr(layer["wv"]),
                           _ptr(layer["wo"]), _ptr(layer["k_cache"]), _ptr(layer["v_cache"]),
                           _ptr(layer.get("attn_packed")))
    full = GlanceFullLayer(attn, _ptr(layer["g_attn"]), _ptr(layer["g_q"]), _ptr(layer["g_k"]),
                           _ptr(layer["g_mlp"]), _ptr(layer["w_gate"]), _ptr(layer["w_up"]),
                           _ptr(layer["w_down"]), layer["w_gate"].shape[0], float(eps),
                           _ptr(layer.get("mlp_packed")))
    _lib.call("glance_tree_layer", ctypes.byref(full), _ptr(embed), _ptr(token), _ptr(h_in),
              _ptr(h_out), _ptr(kv_offsets), int(max_prefix), _ptr(depth), _ptr(anc),
              _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], nseq, n_rows, d_model, Hq, Hkv,
              D, _ptr(attn_out), _ptr(tree_k), _ptr(tree_v), _ptr(ws), ws.numel(),
              _stream(stream))


def glance_attn_pack(layer: dict, Hq: int, Hkv: int, stream=None):
    """bf16 attention weights (wq/wk/wv/wo) -> the projection kernel's packed tile
    order (a new uint8 device tensor; done once, when the weights are loaded)."""
    qd, d_model = layer["wq"].shape
    D = qd // Hq
    n = _lib.load().glance_attn_pack_bytes(d_model, Hq, Hkv, D)
    if n == 0:
        raise ValueError(f"no packed layout for d_model={d_model}, Hq={Hq}, Hkv={Hkv}, D={D}")
    out = torch.empty(n, dtype=torch.uint8, device=layer["wq"].device)
    _lib.call("glance_attn_pack", _ptr(layer["wq"]), _ptr(layer["wk"]), _ptr(layer["wv"]),
              _ptr(layer["wo"]), d_model, Hq, Hkv, D, _ptr(out), _stream(stream))
    return out


def glance_mlp_pack(layer: dict, stream=None):
    """bf16 MLP weights of a full layer -> the projection kernel's packed tile
    order (a new uint8 device tensor; done once, when the weights are loaded)."""
    inter, d_model = layer["w_gate"].shape
    n = _lib.load().glance_mlp_pack_bytes(d_model, inter)
    if n == 0:
        raise ValueError(f"no packed layout for d_model={d_model}, inter={inter}")
    out = torch.empty(n, dtype=torch.uint8, device=layer["w_gate"].device)
    _lib.call("glance_mlp_pack", _ptr(layer["w_gate"]), _ptr(layer["w_up"]), _ptr(layer["w_down"]),
              d_model, inter, _ptr(out), _stream(stream))
    return out


# ---------------------------------------------------------------------- step 4
def verify_head_ws_bytes(R, V, d_model, dtype) -> int:
    return _lib.load().glance_verify_head_ws(R, V, d_model, dtype)


def glance_verify_head(h, w_head, argmax, top1, gap, entropy, ws, logits=None, stream=None):
    R, d_model = h.shape
    V = w_head.shape[0]
    _lib.call("glance_verify_head", _ptr(h), _ptr(w_head), dtype_code(w_head), R, d_model, V,
              _ptr(argmax), _ptr(top1), _ptr(gap), _ptr(entropy), _ptr(logits), _ptr(ws),
              ws.numel(), _stream(stream))


def glance_verify_head_sampled(h, w_head, temperature, seed, round_id, argmax, top1, gap,
                               entropy, sample_tok, sample_gap, ws, logits=None, stream=None):
    """The head with one token per row drawn from softmax(z / temperature)."""
    R, d_model = h.shape
    V = w_head.shape[0]
    _lib.call("glance_verify_head_sampled", _ptr(h), _ptr(w_head), dtype_code(w_head), R,
              d_model, V, float(temperature), int(seed), int(round_id), _ptr(argmax), _ptr(top1),
              _ptr(gap), _ptr(entropy), _ptr(sample_tok), _ptr(sample_gap), _ptr(logits),
              _ptr(ws), ws.numel(), _stream(stream))


def head_pack_bytes(V: int, d_model: int) -> int:
    return _lib.load().glance_head_pack_bytes(V, d_model)


def glance_head_pack(w_head, stream=None):
    """bf16 LM-head weights [V][d_model] -> the head kernel's packed tile order
    (a new uint8 device tensor; done once, when the weights are loaded)."""
    V, d_model = w_head.shape
    n = head_pack_bytes(V, d_model)
    if n == 0:
        raise ValueError(f"no packed layout for V={V}, d_model={d_model}")
    out = torch.empty(n, dtype=torch.uint8, device=w_head.device)
    _lib.call("glance_head_pack", _ptr(w_head), V, d_model, _ptr(out), _stream(stream))
    return out


def glance_verify_head_packed(h, w_packed, V, argmax, top1, gap, entropy, ws, logits=None,
                              temperature=1.0, seed=0, round_id=0, sample_tok=None,
                              sample_gap=None, stream=None):
    R, d_model = h.shape
    _lib.call("glance_verify_head_packed", _ptr(h), _ptr(w_packed), R, d_model, V,
              float(temperature), int(seed), int(round_id), _ptr(argmax), _ptr(top1), _ptr(gap),
              _ptr(entropy), _ptr(sample_tok), _ptr(sample_gap), _ptr(logits), _ptr(ws),
              ws.numel(), _stream(stream))


def glance_verify_head_walk(h, w_packed, V, argmax, top1, gap, entropy, ws, parent, token, n_valid,
                            nseq, n_rows, L, gap_flag, n_accept, out_tokens, path_rows, flagged,
                            logits=None, temperature=1.0, seed=0, round_id=0, sample_tok=None,
                            sample_gap=None, stream=None):
    """The packed head and the accept walk of every round in one call (the
    head's last row to finish walks)."""
    R, d_model = h.shape
    walk = GlanceWalk(_ptr(parent), _ptr(token), _ptr(n_valid), nseq, n_rows, L, float(gap_flag),
                      _ptr(n_accept), _ptr(out_tokens), _ptr(path_rows), _ptr(flagged))
    _lib.call("glance_verify_head_walk", _ptr(h), _ptr(w_packed), R, d_model, V, float(temperature),
              int(seed), int(round_id), _ptr(argmax), _ptr(top1), _ptr(gap), _ptr(entropy),
              _ptr(sample_tok), _ptr(sample_gap), _ptr(logits), ctypes.byref(walk), _ptr(ws),
              ws.numel(), _stream(stream))


def glance_verify_head_packed_noalloc(h, w_packed, V, argmax, top1, gap, entropy, logits=None,
                                      temperature=1.0, seed=0, round_id=0, sample_tok=None,
                                      sample_gap=None, stream=None):
    """The packed head with the library's fixed device scratch in place of a
    workspace (no allocation); calls that overlap on one GPU race."""
    R, d_model = h.shape
    _lib.call("glance_verify_head_packed_noalloc", _ptr(h), _ptr(w_packed), R, d_model, V,
              float(temperature), int(seed), int(round_id), _ptr(argmax), _ptr(top1), _ptr(gap),
              _ptr(entropy), _ptr(sample_tok), _ptr(sample_gap), _ptr(logits), _stream(stream))


# ---------------------------------------------------------------------- step 5
def glance_read_probe(buf, out, n_wg: int, stream=None):
    """One calibration read of every byte of ``buf`` (XOR per work-group into ``out``)."""
    _lib.call("glance_read_probe", _ptr(buf), buf.numel() * buf.element_size(), n_wg, _ptr(out),
              _stream(stream))


def glance_head_timing(start=None, stop=None):
    """Record two torch.cuda.Event objects around the LM-head GEMM of every later
    verify-head call (both None: stop recording)."""
    if (start is None) != (stop is None):
        raise ValueError("start and stop must both be events or both be None")
    if start is None:
        _lib.call("glance_head_timing", None, None)
        return
    if not start.cuda_event or not stop.cuda_event:
        raise ValueError("record each event once before handing it over (torch creates it lazily)")
    _lib.call("glance_head_timing", ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event))


def glance_accept_walk(parent, token, n_valid, argmax, gap, nseq, n_rows, L, gap_flag,
                       n_accept, out_tokens, path_rows, flagged, stream=None):
    _lib.call("glance_accept_walk", _ptr(parent), _ptr(token), _ptr(n_valid), _ptr(argmax),
              _ptr(gap), nseq, n_rows, L, float(gap_flag), _ptr(n_accept), _ptr(out_tokens),
              _ptr(path_rows), _ptr(flagged), _stream(stream))


# ---------------------------------------------------------------- after step 5
def glance_commit_kv(tree_k, tree_v, path_rows, n_accept, L, kv_offsets, k_cache, v_cache,
                     stream=None):
    """Append one layer's accepted path entries to its cache (one sequence)."""
    _, Hkv, D = tree_k.shape
    _lib.call("glance_commit_kv", _ptr(tree_k), _ptr(tree_v), dtype_code(tree_k), _ptr(path_rows),
              _ptr(n_accept), n_accept.shape[0], L, Hkv, D, _ptr(kv_offsets), _ptr(k_cache),
              _ptr(v_cache), k_cache.shape[0], _stream(stream))


def glance_advance_round(n_accept, out_tokens, kv_offsets, root_token, stream=None):
    """Move the prefix end past the committed entries and set the next root."""
    _lib.call("glance_advance_round", _ptr(n_accept), _ptr(out_tokens), n_accept.shape[0],
              _ptr(kv_offsets), _ptr(root_token), _stream(stream))
