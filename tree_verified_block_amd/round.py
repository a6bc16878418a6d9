"""One verify round on the device: the synthetic workload's tensors uploaded once
into HBM, output and workspace buffers allocated once, and the four C-ABI calls
launched in stream order (steps 1-2, one tree-attention call per layer, the LM
head, the walk)."""
from __future__ import annotations

import numpy as np
import torch

from . import api
from ._lib import GLANCE_BF16, GLANCE_F32

GAP_FLAG = 1e-3


def to_device(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Stored synthetic tensor -> device tensor (bf16 bit patterns -> bfloat16)."""
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


class DeviceRound:
    """``capacity`` (one sequence only): the caches get room for that many rows and
    every layer keeps its own tree-row K/V, so that ``commit()`` can append each
    round's accepted path and chain rounds on the device.

    ``temperature``: every verify row also draws a token from softmax(z / T)
    (Philox key ``seed``, counter round ``round_id``) and the walk runs on the
    draws instead of the argmax; ``commit()`` moves to the next round id.

    ``packed_head`` (bf16): the LM-head weights, the attention weights (and the
    MLP weights of full layers) are packed once into their kernels' tile orders
    and every round reads the packed copies."""

    def __init__(self, inp: dict, device="cuda", keep_layers: bool = False,
                 want_logits: bool = False, capacity: int | None = None,
                 temperature: float | None = None, seed: int = 0, packed_head: bool = False):
        cfg = inp["cfg"]
        self.cfg = cfg
        self.inp = inp
        self.device = device
        self.dt = GLANCE_BF16 if cfg.dtype == "bf16" else GLANCE_F32
        dt = cfg.dtype
        self.nseq, self.L, self.N, self.V = cfg.nseq, cfg.L, cfg.N, cfg.V
        self.n_rows = cfg.N + 1
        self.R = self.nseq * self.n_rows
        d = cfg.d_model
        self.embed = to_device(inp["embed"], dt, device)
        self.w_head = to_device(inp["w_head"], dt, device)
        self.w_packed = None
        if packed_head:
            if dt != "bf16":
                raise ValueError("the packed head is bf16 only")
            self.w_packed = api.glance_head_pack(self.w_head)
        self.layers = [{k: to_device(v, dt, device) for k, v in lw.items()} for lw in inp["layers"]]
        if packed_head:
            for lw in self.layers:
                lw["attn_packed"] = api.glance_attn_pack(lw, cfg.Hq, cfg.Hkv)
                if getattr(cfg, "mlp", 0) > 0:
                    lw["mlp_packed"] = api.glance_mlp_pack(lw)
        self.kv_offsets = torch.from_numpy(inp["kv_offsets"].astype(np.int64)).to(device)
        self.max_prefix = int(inp["prefix_len"].max())
        self.capacity = capacity
        if capacity is not None:
            if cfg.nseq != 1:
                raise ValueError("chained rounds need one sequence")
            P = int(inp["prefix_len"][0])
            if capacity < P + cfg.L + 1:
                raise ValueError("capacity below one round")
            for lw in self.layers:
                for name in ("k_cache", "v_cache"):
                    c = lw[name]
                    big = torch.zeros((capacity,) + tuple(c.shape[1:]), dtype=c.dtype, device=device)
                    big[:c.shape[0]].copy_(c)
                    lw[name] = big
            self.max_prefix = capacity - cfg.L - 1
        self.rope_cos = torch.from_numpy(inp["rope_cos"]).to(device)
        self.rope_sin = torch.from_numpy(inp["rope_sin"]).to(device)
        self.tree = api.tree_outputs(self.nseq, self.N, device)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        self.h = [torch.empty((self.R, d), dtype=tdt, device=device) for _ in range(2)]
        self.keep_layers = keep_layers
        HD = cfg.Hq * cfg.D
        n_keep = cfg.n_layers if keep_layers else 0
        self.attn_out = [torch.empty((self.R, HD), dtype=torch.float32, device=device)
                         for _ in range(n_keep)]
        self.h_layers = [torch.empty((self.R, d), dtype=tdt, device=device) for _ in range(n_keep)]
        n_kv = cfg.n_layers if capacity is not None else 1
        self.tree_ks = [torch.empty((self.R, cfg.Hkv, cfg.D), dtype=tdt, device=device) for _ in range(n_kv)]
        self.tree_vs = [torch.empty((self.R, cfg.Hkv, cfg.D), dtype=tdt, device=device) for _ in range(n_kv)]
        self.tree_k, self.tree_v = self.tree_ks[-1], self.tree_vs[-1]
        self.argmax = torch.empty(self.R, dtype=torch.int32, device=device)
        self.top1 = torch.empty(self.R, dtype=torch.float32, device=device)
        self.gap = torch.empty(self.R, dtype=torch.float32, device=device)
        self.entropy = torch.empty(self.R, dtype=torch.float32, device=device)
        self.logits = (torch.empty((self.R, self.V), dtype=torch.float32, device=device)
                       if want_logits else None)
        self.temperature = temperature
        self.seed = int(seed)
        self.round_id = 0
        if temperature is not None:
            self.sample_tok = torch.empty(self.R, dtype=torch.int32, device=device)
            self.sample_gap = torch.empty(self.R, dtype=torch.float32, device=device)
        self.n_accept = torch.empty(self.nseq, dtype=torch.int32, device=device)
        self.out_tokens = torch.empty((self.nseq, self.L + 1), dtype=torch.int32, device=device)
        self.path_rows = torch.empty((self.nseq, self.L + 1), dtype=torch.int32, device=device)
        self.flagged = torch.empty(self.nseq, dtype=torch.int32, device=device)
        self.ws_tree = api.workspace(api.build_tree_ws_bytes(self.nseq, self.L, self.V, self.N), device)
        self.full = getattr(cfg, "mlp", 0) > 0
        if self.full:
            self.ws_attn = api.workspace(api.tree_layer_ws_bytes(self.nseq, self.n_rows, self.max_prefix,
                                                                 d, cfg.Hq, cfg.Hkv, cfg.D, cfg.mlp), device)
        else:
            self.ws_attn = api.workspace(api.tree_attn_ws_bytes(self.nseq, self.n_rows, self.max_prefix, d,
                                                                cfg.Hq, cfg.Hkv, cfg.D), device)
        self.ws_head = api.workspace(api.verify_head_ws_bytes(self.R, self.V, d, self.dt), device)
        self.draft = None
        self.root = None
        self.given_tree = cfg.draft == "topology"

    def set_round(self, r: int):
        rd = self.inp["rounds"][r]
        self.root = torch.from_numpy(rd["root"].astype(np.int32)).to(self.device)
        if self.given_tree:
            self.tree["parent"].copy_(torch.from_numpy(rd["parent"]))
            self.tree["depth"].copy_(torch.from_numpy(rd["depth"]))
            self.tree["token"].copy_(torch.from_numpy(rd["token"]))
            self.tree["anc"].copy_(torch.from_numpy(rd["anc"].view(np.int64)))
            self.tree["score"].zero_()
            self.tree["n_valid"].fill_(self.n_rows)
        else:
            self.draft = to_device(rd["draft_logits"], self.cfg.dtype, self.device)

    # -------------------------------------------------------------- the path
    def step_tree(self, stream=None):
        if not self.given_tree:
            api.glance_build_tree(self.draft, self.root, self.N, self.tree, self.ws_tree, stream)

    def step_attn(self, stream=None):
        cfg = self.cfg
        t = self.tree
        for li, lw in enumerate(self.layers):
            h_in = None if li == 0 else self.h[(li - 1) % 2]
            h_out = self.h[li % 2]
            if self.full:
                api.glance_tree_layer(lw, cfg.norm_eps, self.embed if li == 0 else None, t["token"],
                                      h_in, h_out, self.kv_offsets, self.max_prefix, t["depth"],
                                      t["anc"], self.rope_cos, self.rope_sin, self.nseq, self.n_rows,
                                      cfg.d_model, cfg.Hq, cfg.Hkv, cfg.D, self.ws_attn,
                                      attn_out=self.attn_out[li] if self.keep_layers else None,
                                      tree_k=self.tree_ks[min(li, len(self.tree_ks) - 1)],
                                      tree_v=self.tree_vs[min(li, len(self.tree_vs) - 1)],
                                      stream=stream)
                if self.keep_layers:
                    self.h_layers[li].copy_(h_out)
                continue
            api.glance_tree_attn(lw, self.dt, self.embed if li == 0 else None, t["token"], h_in,
                                 h_out, self.kv_offsets, self.max_prefix, t["depth"], t["anc"],
                                 self.rope_cos, self.rope_sin, self.nseq, self.n_rows,
                                 cfg.d_model, cfg.Hq, cfg.Hkv, cfg.D, self.ws_attn,
                                 attn_out=self.attn_out[li] if self.keep_layers else None,
                                 tree_k=self.tree_ks[min(li, len(self.tree_ks) - 1)],
                                 tree_v=self.tree_vs[min(li, len(self.tree_vs) - 1)], stream=stream)
            if self.keep_layers:
                self.h_layers[li].copy_(h_out)

    @property
    def h_final(self):
        return self.h[(self.cfg.n_layers - 1) % 2]

    def step_head(self, stream=None):
        if self.w_packed is not None:
            kw = {}
            if self.temperature is not None:
                kw = dict(temperature=self.temperature, seed=self.seed, round_id=self.round_id,
                          sample_tok=self.sample_tok, sample_gap=self.sample_gap)
            api.glance_verify_head_packed(self.h_final, self.w_packed, self.V, self.argmax,
                                          self.top1, self.gap, self.entropy, self.ws_head,
                                          logits=self.logits, stream=stream, **kw)
        elif self.temperature is None:
            api.glance_verify_head(self.h_final, self.w_head, self.argmax, self.top1, self.gap,
                                   self.entropy, self.ws_head, logits=self.logits, stream=stream)
        else:
            api.glance_verify_head_sampled(self.h_final, self.w_head, self.temperature, self.seed,
                                           self.round_id, self.argmax, self.top1, self.gap,
                                           self.entropy, self.sample_tok, self.sample_gap,
                                           self.ws_head, logits=self.logits, stream=stream)

    def step_walk(self, stream=None, gap_flag=GAP_FLAG):
        t = self.tree
        tok, gap = ((self.argmax, self.gap) if self.temperature is None
                    else (self.sample_tok, self.sample_gap))
        api.glance_accept_walk(t["parent"], t["token"], t["n_valid"], tok, gap,
                               self.nseq, self.n_rows, self.L, gap_flag, self.n_accept,
                               self.out_tokens, self.path_rows, self.flagged, stream)

    def step_verify(self, stream=None, gap_flag=GAP_FLAG):
        """Steps 4-5: with packed head weights one call (the head's last row to
        finish walks), else the head and the walk in turn."""
        if self.w_packed is None:
            self.step_head(stream)
            self.step_walk(stream, gap_flag)
            return
        kw = {}
        if self.temperature is not None:
            kw = dict(temperature=self.temperature, seed=self.seed, round_id=self.round_id,
                      sample_tok=self.sample_tok, sample_gap=self.sample_gap)
        t = self.tree
        api.glance_verify_head_walk(self.h_final, self.w_packed, self.V, self.argmax, self.top1,
                                    self.gap, self.entropy, self.ws_head, t["parent"], t["token"],
                                    t["n_valid"], self.nseq, self.n_rows, self.L, gap_flag,
                                    self.n_accept, self.out_tokens, self.path_rows, self.flagged,
                                    logits=self.logits, stream=stream, **kw)

    def run(self, stream=None):
        self.step_tree(stream)
        self.step_attn(stream)
        self.step_verify(stream)

    def set_draft(self, draft_logits: np.ndarray, root: int | None = None):
        """Next round's draft logits [1][L][V] (and, optionally, its root)."""
        self.draft = to_device(draft_logits, self.cfg.dtype, self.device)
        if root is not None:
            self.root = torch.tensor([root], dtype=torch.int32, device=self.device)

    def commit(self, stream=None):
        """Append the round's accepted path to every layer's cache, move the prefix
        end past it and make the emitted token the next root (on the device)."""
        if self.capacity is None:
            raise RuntimeError("commit needs a DeviceRound built with a capacity")
        for li, lw in enumerate(self.layers):
            api.glance_commit_kv(self.tree_ks[li], self.tree_vs[li], self.path_rows, self.n_accept,
                                 self.L, self.kv_offsets, lw["k_cache"], lw["v_cache"], stream)
        api.glance_advance_round(self.n_accept, self.out_tokens, self.kv_offsets, self.root, stream)
        self.round_id += 1

    def fetch(self) -> dict:
        torch.cuda.synchronize()
        out = {k: v.cpu().numpy() for k, v in self.tree.items()}
        out["anc"] = out["anc"].view(np.uint64)
        out.update(argmax=self.argmax.cpu().numpy(), top1=self.top1.cpu().numpy(),
                   gap=self.gap.cpu().numpy(), entropy=self.entropy.cpu().numpy(),
                   n_accept=self.n_accept.cpu().numpy(), out_tokens=self.out_tokens.cpu().numpy(),
                   path_rows=self.path_rows.cpu().numpy(), flagged=self.flagged.cpu().numpy())
        out["h_final"] = self.h_final.float().cpu().numpy()
        if self.logits is not None:
            out["logits"] = self.logits.cpu().numpy()
        if self.temperature is not None:
            out["sample_tok"] = self.sample_tok.cpu().numpy()
            out["sample_gap"] = self.sample_gap.cpu().numpy()
        if self.keep_layers:
            out["attn_out"] = [a.cpu().numpy() for a in self.attn_out]
            out["h_layers"] = [h.float().cpu().numpy() for h in self.h_layers]
        out["tree_k"] = self.tree_k.float().cpu().numpy()
        out["tree_v"] = self.tree_v.float().cpu().numpy()
        return out
