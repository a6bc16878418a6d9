"""Writes precision_bounds.json: how far two valid evaluations of the same
verify rows drift apart from rounding alone, per workload, measured with the
oracle only (no GPU value enters).

For every workload the parity tests use, every verify row of the listed rounds
is evaluated twice by the oracle: in float64 between storage points (the
reference) and in float32 between the same storage points (a second correct
implementation: same definition, same bf16 storage points, same order of
operations, only the arithmetic between storage points is float32).  Recorded
per workload, as maxima over its rounds:

  dz        max |z_f32 - z_f64| over every logit of every row (logit units)
  logits    norm-wise relative drift of the logits, max|dz| / max|z_f64|
  h, attn   norm-wise relative drift of every layer's output rows and
            attention outputs (max over layers)

The comparison rules take two things from this file.  An argmax is decided
(bit-exact required) when the reference top-2 gap exceeds max(1e-3, 2 dz):
two evaluations whose logits differ by at most dz can only disagree on a row
whose gap is at most 2 dz.  And the parity tolerances for floating point
(1e-5 fp32, 1e-2 bf16) stand as long as the recorded drift stays below them.

Run:  python -m tests.golden.make_precision_bounds   (about 15 minutes, ~20 GB)
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import model as mdl, round as orr, tree as tr  # noqa: E402
from synth import gen_round, make_config  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "precision_bounds.json")

# (config, overrides, seed, rounds): the rounds the GPU parity tests compare
CASES = [
    ("tiny", {}, 1000, [0]), ("tiny", {}, 1001, [0]), ("tiny", {}, 1002, [0]),
    ("tiny_widehead", {}, 1000, [0]), ("tiny_widehead", {}, 1003, [0]),
    ("mini_bf16", {}, 1, [0]), ("mini_bf16", {}, 2, [0]),
    ("mini_bf16_ragged", {}, 3, [0]), ("mini_bf16_ragged", {}, 4, [0]),
    ("mini_bf16_ragged", dict(draft="topology", n_layers=3, nseq=2, N=63, L=15), 9, [0]),
    ("mini_bf16_copy", {}, 3, [0, 1, 2, 3]),
    ("mini_bf16_full", {}, 1, [0]), ("mini_bf16_full", {}, 2, [0]),
    ("qwen8b_1layer", {}, 2000, [0, 1, 2, 3, 4, 5]),
    ("qwen8b_copy", {}, 3000, [0, 1, 2, 3]),
    ("qwen8b_ragged8", {}, 5000, [0]),
    ("qwen8b_full", {}, 6000, [0]),
    ("qwen8b_deep36", {}, 4000, [0]),
]


def _paths(rd, cfg, s):
    root = int(rd["root"][s])
    if "draft_logits" in rd:
        return root, orr.build_tree(rd["draft_logits"][s], cfg.dtype, root, cfg.N)["order"]
    return root, [()] + tr.paths_from_layout(rd["parent"][s], rd["token"][s], cfg.N + 1)


def _rel(a, b) -> float:
    den = float(np.abs(b).max())
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def measure(name, over, seed, rounds) -> dict:
    inp = gen_round(make_config(name, **over), seed)
    cfg = inp["cfg"]
    big = cfg.V * cfg.d_model > 1e8
    m64 = mdl.TargetModel(inp, cache_head=big)
    m32 = mdl.TargetModel(inp, cache_head=big, compute="f32")
    res = {"dz": 0.0, "logits": 0.0, "h": 0.0, "attn": 0.0, "rows": 0}
    for r in rounds:
        rd = inp["rounds"][r]
        for s in range(cfg.nseq):
            root, paths = _paths(rd, cfg, s)
            e64 = mdl.evaluate_paths(m64, s, root, paths)
            e32 = mdl.evaluate_paths(m32, s, root, paths)
            z64, z32 = m64.logits(e64["final"]), m32.logits(e32["final"])
            res["dz"] = max(res["dz"], float(np.abs(z32 - z64).max()))
            res["logits"] = max(res["logits"], _rel(z32, z64))
            for li in range(cfg.n_layers):
                res["h"] = max(res["h"], _rel(e32["h"][li], e64["h"][li]))
                res["attn"] = max(res["attn"], _rel(e32["attn"][li], e64["attn"][li]))
            res["rows"] += len(paths)
    return res


def main():
    table: dict = {}
    for name, over, seed, rounds in CASES:
        t0 = time.perf_counter()
        m = measure(name, over, seed, rounds)
        ent = table.setdefault(name, {"dz": 0.0, "logits": 0.0, "h": 0.0, "attn": 0.0,
                                      "rows": 0, "cases": []})
        for k in ("dz", "logits", "h", "attn"):
            ent[k] = max(ent[k], m[k])
        ent["rows"] += m["rows"]
        ent["cases"].append(f"seed {seed} rounds {rounds}" + (f" {over}" if over else ""))
        print(f"{name} seed {seed}: {m} ({time.perf_counter() - t0:.0f} s)", flush=True)
    with open(OUT, "w") as f:
        json.dump({"about": "float32-vs-float64 oracle drift per workload; written by "
                            "tests/golden/make_precision_bounds.py (oracle only)",
                   "workloads": table}, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
