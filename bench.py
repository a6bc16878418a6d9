"""Benchmark of the verify round on one MI355X.

A step is one whole round (steps 1-5: tree build, one packed tree-attention
layer, LM head with its epilogue, accept walk) over device-resident synthetic
inputs of the 8B-shaped single-layer workload: d_model 4096, 32 query / 8 KV
heads, head_dim 128, V 151936, L 15, N 63, a 1024-token prefix, bf16 storage,
packed head and attention weights.  Prints one JSON line: rounds/s of K rounds
launched on one stream (the headline), the per-round distribution, the same
rounds replayed from HIP graphs, per-step microseconds and HBM fractions (HIP
events on the launch stream), the roofline of the dominant kernel (the LM head),
the other workloads (tiny fp32, copy regime, ragged batch of 8, 36-layer
stack), sampled and chained rounds, the shared-budget build, full decoder
layers, a plain device copy, and the CPU oracle on a sample of the workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify rounds/s at N=63, L=15, V=151936 (8B shape); % of HBM peak per kernel"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def step_bytes(cfg, P: int) -> dict:
    """Algorithmic HBM bytes of each step of one round (each tensor moved once)."""
    es = 2 if cfg.dtype == "bf16" else 4
    R = cfg.nseq * (cfg.N + 1)
    d, HD, KD = cfg.d_model, cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    tree = cfg.nseq * cfg.L * cfg.V * es + R * 28
    attn_layer = ((HD + 2 * KD) * d + d * HD) * es + 2 * P * KD * es * cfg.nseq + 2 * R * d * es
    attn = cfg.n_layers * attn_layer
    head = cfg.V * d * es + R * d * es + R * 16
    walk = R * 16 + cfg.nseq * (cfg.L + 1) * 8
    return {"build_tree": tree, "tree_attn": attn, "verify_head": head, "accept_walk": walk}


def head_traffic(cfg):
    """HBM bytes per LM-head launch from the committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by the same counters on a copy of known
    size), or None when the head's source has changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "verify_head_traffic_qwen8b_1layer.json")
    src = os.path.join(ROOT, "tree_verified_block_amd", "csrc", "gemm.hip")
    if cfg.name != "qwen8b_1layer" or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("gemm_hip_sha256") != digest:
        return None
    return rec.get("traffic_bytes")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(inp, budget_s: float = 10.0) -> dict:
    """The CPU oracle as it stands, on whole rounds of the same workload (log-
    softmax, exact top-N tree, every verify row by unpacked evaluation, head
    statistics and the walk; the independent greedy re-decode is left out), run
    round after round until about budget_s seconds of work: once with the BLAS
    pool limited to one thread, once with all the host's cores."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import round as orr
    n_avail = len(inp["rounds"])

    def timed(limit):
        with threadpool_limits(limits=limit):
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            n = 0
            t0 = time.perf_counter()
            while True:
                orr.oracle_round(inp, n % n_avail, exact="beam", continuation_check=False)
                n += 1
                dt = time.perf_counter() - t0
                if dt >= budget_s or n >= 4 * n_avail:
                    break
        return n, dt, threads

    n1, dt1, _ = timed(1)
    na, dta, threads = timed(None)
    return {"value": round(na / dta, 4), "unit": "rounds/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{na} rounds of {inp['cfg'].name} (steps 1-5, float64 NumPy), {dta:.1f} s",
            "one_thread": {"value": round(n1 / dt1, 4), "cores": 1,
                           "sample": f"{n1} rounds, {dt1:.1f} s"},
            "host_cpu": _cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cache_residency(dev, drafts, K: int, copies: int = 4) -> dict:
    """The single-layer round with its layer's weights and prefix cache rotated
    over ``copies`` device copies (4 x 88 MB, more than the 256 MB Infinity
    Cache) against one copy: a round-time difference would mean that the one
    copy is served from that cache between rounds."""
    import torch
    base = dev.layers[0]
    sets = [base] + [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
                     for _ in range(copies - 1)]
    stream = torch.cuda.current_stream()

    def run(rotate: bool) -> float:
        for i in range(K + 3):
            if i == 3:
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            dev.layers[0] = sets[i % copies] if rotate else base
            if drafts:
                dev.draft = drafts[i % len(drafts)]
            dev.step_tree()
            dev.step_attn()
            dev.step_verify()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    try:
        one, rot = run(False), run(True)
        one2 = run(False)
    finally:
        dev.layers[0] = base
    del sets
    torch.cuda.empty_cache()
    return {"copies": copies, "one_copy_us": round(min(one, one2), 2), "rotated_us": round(rot, 2),
            "note": "rounds launched call by call, K each; the layer's packed weights and prefix "
                    "cache rotated over the copies"}


def graph_replays(dev, drafts, K: int, warm: int = 3, dist: int = 0) -> dict:
    """Rounds replayed from HIP graphs: one graph per draft (each captures the
    whole round reading that draft's tensor; a given-topology workload has one),
    replayed in turn.  Times exactly K replays between two synchronisations;
    with dist > 0 also `dist` replays bracketed one by one with events on the
    replay stream (median, p10, p90 of the per-round time)."""
    import torch
    graphs = []
    for d in (drafts or [None]):
        if d is not None:
            dev.draft = d
        dev.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dev.run()
        graphs.append(g)
    for i in range(warm):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out = {"rounds_per_s": round(K / wall, 2), "us_per_round": round(wall / K * 1e6, 2),
           "replays": K, "graphs": len(graphs)}
    if dist > 0:
        stream = torch.cuda.current_stream()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(dist)]
        for i, e in enumerate(ev):
            e[0].record(stream)
            graphs[i % len(graphs)].replay()
            e[1].record(stream)
        torch.cuda.synchronize()
        us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in ev])
        out["per_round_us"] = {"median": round(float(np.median(us)), 2),
                               "p10": round(float(np.percentile(us, 10)), 2),
                               "p90": round(float(np.percentile(us, 90)), 2), "n": dist}
    del graphs
    return out


def config_leg(name: str, K: int, seed: int, model: dict | None = None, layer_copies: int = 0,
               head_peak: bool = False, overrides: dict | None = None) -> dict:
    """Graph-replayed rounds of another workload (packed weights when bf16).
    ``model``: an 8B-shaped workload whose embedding, head and layer weights are
    reused (its prefix caches, drafts and trees are this config's own).
    layer_copies > 0: the config's layer count built from copies of its first
    layer's weights and cache (each layer still its own device copy, streamed
    from HBM every round), which keeps generation on the host short."""
    import torch
    from synth import gen_round, make_config
    from tree_verified_block_amd.round import DeviceRound, to_device
    cfg = make_config(name, **(overrides or {}))
    t0 = time.perf_counter()
    if layer_copies:
        inp = gen_round(cfg.replace(n_layers=1), seed, model=model)
        inp["layers"] = [inp["layers"][0]] * layer_copies
        inp["cfg"] = cfg
    else:
        inp = gen_round(cfg, seed, model=model)
    gen_s = time.perf_counter() - t0
    bf16 = cfg.dtype == "bf16"
    dev = DeviceRound(inp, device="cuda", packed_head=bf16)
    dev.set_round(0)
    drafts = [to_device(rd["draft_logits"], cfg.dtype, "cuda") for rd in inp["rounds"]
              if "draft_logits" in rd]
    res = {"workload": f"{cfg.name}: {cfg.n_layers} layer(s), d_model {cfg.d_model}, "
                       f"{cfg.Hq}q/{cfg.Hkv}kv x {cfg.D}, V {cfg.V}, L {cfg.L}, N {cfg.N}, "
                       f"nseq {cfg.nseq}, prefix {cfg.prefix}, {cfg.dtype}",
           "host_generation_s": round(gen_s, 1)}
    res.update(graph_replays(dev, drafts, K))
    # eager per-step split of one round (HIP events on the launch stream)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    if drafts:
        dev.draft = drafts[0]
    ev[0].record(stream)
    dev.step_tree()
    ev[1].record(stream)
    dev.step_attn()
    ev[2].record(stream)
    dev.step_head()
    ev[3].record(stream)
    dev.step_walk()
    ev[4].record(stream)
    torch.cuda.synchronize()
    names = ["build_tree", "tree_attn", "verify_head", "accept_walk"]
    res["eager_step_us"] = {n: round(ev[k].elapsed_time(ev[k + 1]) * 1e3, 2) for k, n in enumerate(names)}
    P = int(inp["prefix_len"].max())
    nbytes = step_bytes(cfg, P) if bf16 else None
    if nbytes:
        res["round_bytes"] = sum(nbytes.values())
        res["round_hbm_frac"] = round(res["round_bytes"] / (res["us_per_round"] * 1e-6) /
                                      (HBM_PEAK_GBS * 1e9), 4)
        la = res["eager_step_us"]["tree_attn"]
        res["tree_attn_hbm_frac"] = round(nbytes["tree_attn"] / (la * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)
    if head_peak:
        R = cfg.nseq * (cfg.N + 1)
        flops = 2.0 * R * cfg.d_model * cfg.V
        hu = res["eager_step_us"]["verify_head"]
        res["verify_head_tflops"] = round(flops / (hu * 1e-6) / 1e12, 1)
        res["verify_head_mfma_frac"] = round(flops / (hu * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4)
        res["verify_head_hbm_frac"] = round(nbytes["verify_head"] / (hu * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)
    del dev
    torch.cuda.empty_cache()
    return res


def chain_measure(inp, cfg, drafts, K: int, warm: int = 5, packed: bool = False) -> dict:
    """Chained rounds on the device: each round's verify path, then the commit of
    the accepted path into the cache and the advance of prefix and root (no host
    round trip).  The prefix grows by A + 1 per round; the synthetic drafts do
    not follow the target, so A is mostly 0 here.  HIP events on the launch
    stream bracket the commit of every fourth round."""
    import torch
    from synth.gen import rope_tables
    from tree_verified_block_amd.round import DeviceRound
    P0 = int(inp["prefix_len"][0])
    cap = P0 + (K + warm + 1) * (cfg.L + 1)
    inp = dict(inp)  # rotary tables covering every position the chain reaches
    inp["rope_cos"], inp["rope_sin"] = rope_tables(cap + cfg.N + 1, cfg.D, cfg.rope_theta)
    dev = DeviceRound(inp, device="cuda", capacity=cap, packed_head=packed)
    dev.set_round(0)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        dev.draft = drafts[i % len(drafts)]
        dev.run()
        if ev:
            ev[0].record(stream)
        dev.commit()
        if ev:
            ev[1].record(stream)

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    p_start = int(dev.kv_offsets[1])
    cev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in range(0, K, 4)}
    t0 = time.perf_counter()
    for i in range(K):
        step(i, cev.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_end = int(dev.kv_offsets[1])
    return {"rounds_per_s": round(K / wall, 2), "ms_per_round": round(wall / K * 1e3, 4),
            "commit_us": round(float(np.mean([e[0].elapsed_time(e[1]) for e in cev.values()])) * 1e3, 2),
            "tokens_per_round": round((p_end - p_start) / K, 3), "prefix": [p_start, p_end],
            "rounds": K}


def sampled_measure(inp, cfg, drafts, K: int, T: float = 1.0, warm: int = 5,
                    packed: bool = False) -> dict:
    """Verify rounds that also draw one token per row at temperature T and walk
    on the draws (a new Philox round id per round; steps 4-5 in one call); HIP
    events bracket the LM head of every fourth round (then called on its own)."""
    import torch
    from tree_verified_block_amd.round import DeviceRound
    dev = DeviceRound(inp, device="cuda", temperature=T, seed=1234, packed_head=packed)
    dev.set_round(0)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        dev.draft = drafts[i % len(drafts)]
        dev.round_id = i
        dev.step_tree()
        dev.step_attn()
        if ev is None:
            dev.step_verify()
            return
        ev[0].record(stream)
        dev.step_head()
        ev[1].record(stream)
        dev.step_walk()

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    hev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in range(0, K, 4)}
    t0 = time.perf_counter()
    for i in range(K):
        step(i, hev.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"temperature": T, "rounds_per_s": round(K / wall, 2),
            "ms_per_round": round(wall / K * 1e3, 4),
            "head_us": round(float(np.mean([e[0].elapsed_time(e[1]) for e in hev.values()])) * 1e3, 2),
            "rounds": K}


def shared_measure(K: int, seed: int = 4, budget_per_seq: int = 31, n_max: int = 63,
                   oracle: bool = True) -> dict:
    """Steps 1-2 of an 8-sequence batch (8B vocabulary, L 15, mixed draft
    entropies) under one shared node budget (8 x 31 nodes, at most 63 per
    sequence), each round keyed by ln V(H) of its root entropy through the
    entropy law (pooled fit b0 0.96, b1 0.63, horizon L; root entropies drawn
    uniform over the pages' 0.1-6 nat span), timed with HIP events around the
    two calls; beside it the fixed-width build of the same batch (31 nodes
    each) and the CPU oracle of the shared build."""
    import torch
    from synth import gen_round, make_config
    from tree_verified_block_amd import api
    from tree_verified_block_amd.round import to_device
    cfg = make_config("qwen8b_ragged8")
    inp = gen_round(cfg, seed, with_model=False)
    rd = inp["rounds"][0]
    nseq, L, V = rd["draft_logits"].shape
    draft = to_device(rd["draft_logits"], cfg.dtype, "cuda")
    root = torch.tensor(rd["root"].astype(np.int32), device="cuda")
    b0, b1 = 0.96, 0.63
    Hroot = np.random.default_rng(seed).uniform(0.1, 6.0, nseq).astype(np.float32)
    Hd = torch.tensor(Hroot, device="cuda")
    wd = torch.empty(nseq, dtype=torch.float32, device="cuda")
    B = nseq * budget_per_seq
    out = api.tree_outputs(nseq, n_max, "cuda")
    out_fixed = api.tree_outputs(nseq, budget_per_seq, "cuda")
    ws = api.workspace(api.build_tree_ws_bytes(nseq, L, V, n_max), "cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(5):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]) * 1e3)

    def keyed():
        api.glance_entropy_log_value(Hd, b0, b1, L, wd)
        api.glance_build_tree_shared(draft, root, wd, n_max, B, out, ws)

    us = timed(keyed)
    us_fixed = timed(lambda: api.glance_build_tree(draft, root, budget_per_seq, out_fixed, ws))
    n = (out["n_valid"].cpu().numpy() - 1).tolist()
    nbytes = nseq * L * V * 2 + nseq * (n_max + 1) * 28
    res = {"workload": f"qwen8b_ragged8 drafts: {nseq} sequences x L {L} x V {V} bf16, budget {B} "
                       f"nodes (at most {n_max} per sequence), weights ln V(H) of root entropies "
                       f"U(0.1, 6) nats (b0 {b0}, b1 {b1}, horizon {L})",
           "us_per_call": round(us, 2), "calls_per_s": round(1e6 / us, 1), "nodes": n,
           "algorithmic_bytes": nbytes, "hbm_frac": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
           "fixed_width_us": round(us_fixed, 2)}
    if oracle:
        from oracle import shared as sh
        t0 = time.perf_counter()
        w = sh.log_value(Hroot.astype(np.float64), b0, b1, L).astype(np.float32).astype(np.float64)
        sh.build_trees([rd["draft_logits"][s] for s in range(nseq)], cfg.dtype, rd["root"],
                       w, B, n_max)
        res["oracle_s"] = round(time.perf_counter() - t0, 2)
    return res


def full_layer_measure(K: int, seed: int = 2000, deep: int = 36) -> dict:
    """Rounds of the 8B-shaped workload with full decoder layers (RMSNorm,
    QK-norm, SwiGLU MLP with intermediate 12288): one layer, and a stack of
    `deep` layers whose weights and caches are copies of that layer's (every
    layer still streams its own 386 MB of weights from HBM), with the packed
    head; HIP events around each round."""
    import torch
    from synth import gen_round, make_config
    from tree_verified_block_amd.round import DeviceRound, to_device
    cfg = make_config("qwen8b_full")
    inp = gen_round(cfg, seed)
    drafts = [to_device(rd["draft_logits"], cfg.dtype, "cuda") for rd in inp["rounds"]]
    lw = inp["layers"][0]
    layer_bytes = sum(lw[k].nbytes for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"))
    res = {"workload": f"qwen8b_full: d_model {cfg.d_model}, {cfg.Hq}q/{cfg.Hkv}kv heads x {cfg.D}, "
                       f"MLP {cfg.mlp}, V {cfg.V}, L {cfg.L}, N {cfg.N}, prefix 1024",
           "layer_weight_bytes": layer_bytes}
    stream = torch.cuda.current_stream()
    for n_layers in (1, deep):
        sub = dict(inp)
        sub["cfg"] = cfg.replace(n_layers=n_layers)
        sub["layers"] = [lw] * n_layers
        dev = DeviceRound(sub, device="cuda", packed_head=True)
        dev.set_round(0)
        for i in range(3):
            dev.draft = drafts[i % len(drafts)]
            dev.run()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i, e in enumerate(ev):
            dev.draft = drafts[i % len(drafts)]
            e[0].record(stream)
            dev.run()
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        nbytes = n_layers * layer_bytes + cfg.V * cfg.d_model * 2
        res[f"layers_{n_layers}"] = {"rounds_per_s": round(1e3 / ms, 1), "ms_per_round": round(ms, 4),
                                     "weight_bytes": nbytes,
                                     "hbm_frac": round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}
        del dev
        torch.cuda.empty_cache()
    return res


def run_legs(args, model_inp) -> dict:
    """The other workloads (``--legs``), the 8B ones reusing model_inp's weights."""
    K = args.leg_rounds
    want = set(args.legs.split(","))
    legs = {}
    for key, name, seed, kw in (
            ("tiny_f32", "tiny", 1000, {}),
            ("copy_regime", "qwen8b_copy", 3000, dict(model=model_inp)),
            ("ragged8", "qwen8b_ragged8", 4, dict(model=model_inp, head_peak=True)),
            ("deep36", "qwen8b_deep36", 4000, dict(model=model_inp, layer_copies=36))):
        if key not in want:
            continue
        k = max(5, K // 5) if key == "deep36" else K
        legs[key] = config_leg(name, k, seed, **kw)
        print(f"[bench] leg {key}: {legs[key]['us_per_round']} us per round", file=sys.stderr,
              flush=True)
    if "budget_sweep" in want:
        # the single-layer 8B round at the pages' smaller node budgets (N = 63 is
        # the headline), same weights, prefix and draft temperatures
        for n in (15, 31, 47):
            key = f"budget_N{n}"
            legs[key] = config_leg("qwen8b_1layer", K, 2000, model=model_inp, overrides={"N": n})
            print(f"[bench] leg {key}: {legs[key]['us_per_round']} us per round", file=sys.stderr,
                  flush=True)
    return legs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen8b_1layer")
    ap.add_argument("--seed", type=int, default=2000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chain-rounds", type=int, default=50,
                    help="chained rounds (verify + KV commit + advance) to time; 0 skips")
    ap.add_argument("--sampled-rounds", type=int, default=50,
                    help="verify rounds that sample at T = 1 to time; 0 skips")
    ap.add_argument("--shared-calls", type=int, default=50,
                    help="shared-budget tree builds of an 8-sequence batch to time; 0 skips")
    ap.add_argument("--full-rounds", type=int, default=20,
                    help="rounds of the full-layer workload (1 and 36 layers) to time; 0 skips")
    ap.add_argument("--skip-main", action="store_true",
                    help="run only the extra legs (shared budget, full layers) and print them")
    ap.add_argument("--row-major-head", action="store_true",
                    help="LM head over the row-major weights instead of the packed copy")
    ap.add_argument("--probe-copy", action="store_true",
                    help="accepted for older command lines: the 1 GiB device copy (the counter "
                         "calibration and hbm_probe) always runs")
    ap.add_argument("--leg-rounds", type=int, default=50,
                    help="graph-replayed rounds of each other workload (tiny fp32, copy regime, "
                         "ragged batch of 8; the 36-layer stack takes a fifth); 0 skips them")
    ap.add_argument("--dist-rounds", type=int, default=200,
                    help="rounds timed one by one for the per-round distribution")
    ap.add_argument("--legs", default="tiny_f32,copy_regime,ragged8,deep36,budget_sweep",
                    help="which other workloads to run (comma-separated)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; use --gpus 1"}))
        sys.exit(2)

    import torch
    if args.skip_main:
        out = {}
        if args.shared_calls > 0:
            out["shared_budget"] = shared_measure(args.shared_calls, oracle=not args.no_cpu_baseline)
        if args.full_rounds > 0:
            out["full_layer"] = full_layer_measure(args.full_rounds)
        if args.leg_rounds > 0 and args.legs:
            from synth import gen_round, make_config
            out["configs"] = run_legs(args, gen_round(make_config(args.config), args.seed))
        print(json.dumps(out), flush=True)
        return
    from synth import gen_round, make_config
    from tree_verified_block_amd.round import DeviceRound, to_device

    cfg = make_config(args.config)
    t0 = time.perf_counter()
    inp = gen_round(cfg, args.seed)
    print(f"[bench] generated {cfg.name} in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)
    packed = cfg.dtype == "bf16" and not args.row_major_head
    dev = DeviceRound(inp, device="cuda", packed_head=packed)
    dev.set_round(0)
    drafts = [to_device(rd["draft_logits"], cfg.dtype, "cuda") for rd in inp["rounds"]
              if "draft_logits" in rd]
    stream = torch.cuda.current_stream()

    def one_step(i, ev=None, head_ev=None):
        if drafts:
            dev.draft = drafts[i % len(drafts)]
        if ev is None and head_ev is None:
            # the production round: steps 4-5 in one call (the head's last row walks)
            dev.step_tree()
            dev.step_attn()
            dev.step_verify()
            return
        if ev:
            ev[0].record(stream)
        dev.step_tree()
        if ev:
            ev[1].record(stream)
        dev.step_attn()
        if ev:
            ev[2].record(stream)
        if head_ev:
            head_ev[0].record(stream)
        dev.step_head()
        if head_ev:
            head_ev[1].record(stream)
        if ev:
            ev[3].record(stream)
        dev.step_walk()
        if ev:
            ev[4].record(stream)

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()

    # the LM-head call's live duration (HIP events on the launch stream around it,
    # in K further rounds; the dominant kernel's roofline is taken from these)
    hev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        one_step(i, head_ev=hev[i])
    torch.cuda.synchronize()
    head_us = float(np.mean([e[0].elapsed_time(e[1]) for e in hev]) * 1e3)
    # the dominant kernel alone, the LM-head GEMM: the library records a pair of
    # events on the launch stream right around it (glance_head_timing), in K
    # further production rounds; the roofline line is taken from these
    from tree_verified_block_amd import api
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in gev:  # torch creates an event at its first record
        e[0].record(stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    try:
        for i in range(args.steps):
            api.glance_head_timing(gev[i][0], gev[i][1])
            one_step(i)
    finally:
        api.glance_head_timing(None, None)
    torch.cuda.synchronize()
    gemm_us = float(np.mean([e[0].elapsed_time(e[1]) for e in gev]) * 1e3)

    # per-step breakdown (events between all steps cost a few microseconds per
    # round of their own) and the per-round distribution (events between rounds)
    nd = min(args.steps, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nd)]
    for i in range(nd):
        one_step(i, evs[i])
    torch.cuda.synchronize()
    # steps 4-5 as the timed rounds run them (one fused call)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nd)]
    for i in range(nd):
        if drafts:
            dev.draft = drafts[i % len(drafts)]
        dev.step_tree()
        dev.step_attn()
        fev[i][0].record(stream)
        dev.step_verify()
        fev[i][1].record(stream)
    torch.cuda.synchronize()
    fused_us = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]) * 1e3)
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.dist_rounds)]
    for i, e in enumerate(rev):
        e[0].record(stream)
        one_step(i)
        e[1].record(stream)
    torch.cuda.synchronize()
    rus = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in rev]) if rev else None

    # timed region: exactly K whole rounds launched call by call on one stream,
    # a synchronisation on both sides and nothing else in between (it runs after
    # the untimed measurement passes above, so the GPU has left its idle state)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same rounds replayed from HIP graphs (one graph per draft)
    gr = graph_replays(dev, drafts, args.steps, warm=args.warmup, dist=args.dist_rounds)
    residency = cache_residency(dev, drafts, 50) if packed and cfg.n_layers == 1 else None

    names = ["build_tree", "tree_attn", "verify_head", "accept_walk"]
    us = {n: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs]) * 1e3)
          for k, n in enumerate(names)}
    us["verify_head"] = head_us
    P = int(inp["prefix_len"].max())
    nbytes = step_bytes(cfg, P)
    per_kernel = {n: {"us": round(us[n], 2), "bytes": nbytes[n],
                      "hbm_frac": round(nbytes[n] / (us[n] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)}
                  for n in names}
    vb = nbytes["verify_head"] + nbytes["accept_walk"]
    per_kernel["verify_head+accept_walk (fused, as timed)"] = {
        "us": round(fused_us, 2), "bytes": vb,
        "hbm_frac": round(vb / (fused_us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)}
    total_bytes = sum(nbytes.values())
    ms = wall / args.steps * 1e3
    es = 2 if cfg.dtype == "bf16" else 4
    R = cfg.nseq * (cfg.N + 1)
    gemm_bytes = (cfg.V + R) * cfg.d_model * es  # head weights + activation rows
    head_gbs = gemm_bytes / (gemm_us * 1e-6) / 1e9
    dist = None
    if rus is not None:
        dist = {"median": round(float(np.median(rus)), 2), "p10": round(float(np.percentile(rus, 10)), 2),
                "p90": round(float(np.percentile(rus, 90)), 2), "n": len(rus)}
    out = {
        "metric": METRIC, "value": round(args.steps / wall, 2), "unit": "rounds/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_layers} tree-attention layer(s), d_model "
                   f"{cfg.d_model}, {cfg.Hq}q/{cfg.Hkv}kv heads x {cfg.D}, V {cfg.V}, L {cfg.L}, "
                   f"N {cfg.N}, prefix {P}, nseq {cfg.nseq}", "seed": args.seed,
                   "head_weights": "packed tile order" if packed else "row-major",
                   "timing": f"{args.steps} rounds launched call by call on one stream, "
                             f"drafts cycling over {len(drafts)}, timed after the warm-up and "
                             "the untimed per-step, head and per-round passes"},
        "per_round_us": dist,
        "graph": dict(gr, note="the same rounds replayed from HIP graphs, one per draft"),
        "cache_residency": residency,
        "round_hbm_frac": round(total_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "round_bytes": total_bytes,
        "per_kernel": per_kernel,
        "roofline": {"bound": "hbm", "kernel": "LM-head GEMM ("
                     + ("bf16, packed weights)" if packed else f"{cfg.dtype}, row-major weights)"),
                     "achieved": round(head_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head_gbs / HBM_PEAK_GBS, 4),
                     "traffic": head_traffic(cfg), "kernel_us": round(gemm_us, 2),
                     "algorithmic_bytes": gemm_bytes,
                     "head_call_us": round(head_us, 2)},
    }
    del dev
    torch.cuda.empty_cache()
    if args.sampled_rounds > 0 and drafts:
        out["sampled"] = sampled_measure(inp, cfg, drafts, args.sampled_rounds, packed=packed)
        torch.cuda.empty_cache()
    if args.chain_rounds > 0 and cfg.nseq == 1 and drafts:
        out["chain"] = chain_measure(inp, cfg, drafts, args.chain_rounds, packed=packed)
    if args.shared_calls > 0:
        out["shared_budget"] = shared_measure(args.shared_calls, oracle=not args.no_cpu_baseline)
    if args.full_rounds > 0:
        out["full_layer"] = full_layer_measure(args.full_rounds)
    if args.leg_rounds > 0 and args.legs and cfg.name == "qwen8b_1layer":
        out["configs"] = run_legs(args, inp)
    # plain device copy of 1 GiB (read + write bytes over the event-timed copy):
    # what this machine's HBM sustains outside the path's kernels
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    stream = torch.cuda.current_stream()
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    for _ in range(5):
        b.copy_(a)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_us = ce[0].elapsed_time(ce[1]) * 1e3 / 5
    out["hbm_probe"] = {"kind": "device copy, 1 GiB read + 1 GiB written (torch copy_)",
                        "us": round(copy_us, 1),
                        "GB/s": round(2 * (1 << 30) / (copy_us * 1e-6) / 1e9, 1),
                        "frac_of_peak": round(2 * (1 << 30) / (copy_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del a, b
    torch.cuda.empty_cache()
    # streaming read of 2 GiB with the head's own load kind (glance_read_probe,
    # 2048 work-groups, median of 10 event-timed passes): the read bandwidth the
    # box delivers, beside which the head GEMM's achieved figure is also given
    from tree_verified_block_amd import api
    rb = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    rb.zero_()
    rout = torch.empty(2048, dtype=torch.int32, device="cuda")
    for _ in range(3):
        api.glance_read_probe(rb, rout, 2048)
    re_ = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
    for e in re_:
        e[0].record(stream)
        api.glance_read_probe(rb, rout, 2048)
        e[1].record(stream)
    torch.cuda.synchronize()
    read_us = float(np.median([e[0].elapsed_time(e[1]) for e in re_])) * 1e3
    read_gbs = (1 << 31) / (read_us * 1e-6) / 1e9
    out["hbm_read_probe"] = {"kind": "streaming read, 2 GiB, 16-byte non-temporal loads (glance_read_probe)",
                             "us": round(read_us, 1), "GB/s": round(read_gbs, 1),
                             "frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4)}
    out["roofline"]["frac_of_read_probe"] = round(out["roofline"]["achieved"] / read_gbs, 4)
    del rb, rout
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
