"""Comparison rules between the HIP path's outputs and the CPU oracle.

Integer outputs (tree layout, argmax, walk) must match bit-exactly wherever the
oracle's decision is not a near-tie (top-2 logit gap, or the tree's boundary
gap, above 1e-3: the pages' uniqueness assumption of Theorem 1; for the argmax
also above twice the largest difference between the GPU's and the oracle's
logits of the round, since each of the two best logits can move by that much);
near-ties are flagged, counted and checked for validity instead.  Float tensors
are compared norm-wise, max|gpu - oracle| / max|oracle|, against 1e-5 (fp32
runs), 1e-2 (bf16 runs) or 2e-2 (bf16 runs of full layers: five more bf16
storage points per layer, where a rounding flip moves an element by one bf16
ulp, up to 2^-7 of max|x| for the largest elements, and the next products carry
it to every element; measured errors reach about 1% of max|h|)."""
from __future__ import annotations

import numpy as np

from oracle import draft, model as mdl, round as orr, tree as tr, walk as wk

GAP = 1e-3


def tol_for(dtype: str, full: bool = False) -> float:
    if dtype == "f32":
        return 1e-5
    return 2e-2 if full else 1e-2


def rel_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.abs(want).max()
    return float(np.abs(got - want).max() / (den if den > 0 else 1.0))


def gpu_paths(parent, token, n_valid):
    return [()] + tr.paths_from_layout(parent, token, int(n_valid))


def check_tree(gpu: dict, s: int, ora_tree: dict, logq: np.ndarray, N: int, L: int, report: dict):
    """Tree of sequence s: exact layout when the oracle's boundary gap > 1e-3,
    else a valid top-N set within 1e-3 of the oracle's boundary."""
    R = N + 1
    g_parent = gpu["parent"][s]
    g_token = gpu["token"][s]
    g_nv = int(gpu["n_valid"][s])
    paths = gpu_paths(g_parent, g_token, g_nv)
    S = set(paths[1:])
    # structure always holds
    assert g_parent[0] == -1 and gpu["depth"][s][0] == 0 and gpu["anc"][s][0] == 1
    for i in range(1, g_nv):
        p = paths[i]
        assert 1 <= len(p) <= L and (len(p) == 1 or p[:-1] in S)
        assert int(gpu["depth"][s][i]) == len(p)
        assert int(gpu["anc"][s][i]) == int(gpu["anc"][s][g_parent[i]]) | (1 << i)
    for i in range(g_nv, R):
        assert g_parent[i] == -1 and g_token[i] == -1 and int(gpu["anc"][s][i]) == 0
    # GPU scores against the oracle's float64 plug-in scores of the same paths
    for i in range(1, g_nv):
        p = paths[i]
        want = sum(logq[j, t] for j, t in enumerate(p))
        got = float(gpu["score"][s][i])
        assert abs(got - want) <= 1e-5 * max(1.0, abs(want)), (p, got, want)
    if ora_tree["boundary_gap"] > GAP:
        for k in ("parent", "depth", "token"):
            assert np.array_equal(gpu[k][s], ora_tree[k]), k
        assert np.array_equal(gpu["anc"][s], ora_tree["anc"])
        assert g_nv == ora_tree["n_valid"]
        report["tree_exact"] = report.get("tree_exact", 0) + 1
    else:
        report["tree_flagged"] = report.get("tree_flagged", 0) + 1
        assert g_nv == ora_tree["n_valid"]
        in_scores = [sum(logq[j, t] for j, t in enumerate(p)) for p in paths[1:]]
        best_out = -np.inf
        V = logq.shape[1]
        for p in paths:
            if len(p) >= L:
                continue
            kids = {q[-1] for q in S if len(q) == len(p) + 1 and q[:-1] == p}
            order = tr.token_ranking(logq[len(p)], V)
            for t in order:
                if int(t) not in kids:
                    base = sum(logq[j, u] for j, u in enumerate(p))
                    best_out = max(best_out, base + logq[len(p), int(t)])
                    break
        assert min(in_scores) >= best_out - GAP
    return paths


def check_rows(gpu: dict, ev: dict, z: np.ndarray, s: int, n_rows: int, dtype: str, report: dict,
               rows=None, full: bool = False):
    """Verify rows of sequence s (the oracle evaluated on the GPU's own tree).
    Leaves the round's decision threshold in report["flag"] (see module doc)."""
    tol = tol_for(dtype, full)
    sl = slice(s * n_rows, (s + 1) * n_rows)
    idx = np.arange(len(ev["final"])) if rows is None else np.asarray(rows)
    if "attn_out" in gpu:
        for li in range(len(ev["attn"])):
            e = rel_err(gpu["attn_out"][li][sl][idx], ev["attn"][li])
            report.setdefault("attn_err", []).append(e)
            assert e <= tol, ("attn", li, e)
            e = rel_err(gpu["h_layers"][li][sl][idx], ev["h"][li])
            report.setdefault("h_err", []).append(e)
            assert e <= tol, ("h", li, e)
    am, top1, gap, H = mdl.row_stats(z)
    flag = GAP
    if "logits" in gpu:
        e = rel_err(gpu["logits"][sl][idx], z)
        report.setdefault("logit_err", []).append(e)
        assert e <= tol, ("logits", e)
        e_abs = float(np.abs(gpu["logits"][sl][idx].astype(np.float64) - z).max())
        flag = max(GAP, 2.0 * e_abs)
    report["flag"] = max(report.get("flag", GAP), flag)
    e = rel_err(gpu["top1"][sl][idx], top1)
    assert e <= tol, ("top1", e)
    eH = np.max(np.abs(gpu["entropy"][sl][idx] - H) / np.maximum(1.0, H))
    report.setdefault("H_err", []).append(float(eH))
    assert eH <= tol, ("entropy", eH)
    g_am = gpu["argmax"][sl][idx]
    sure = gap > flag
    report["rows"] = report.get("rows", 0) + len(idx)
    report["rows_flagged"] = report.get("rows_flagged", 0) + int((~sure).sum())
    assert np.array_equal(g_am[sure], am[sure]), "argmax mismatch on an unflagged row"
    # the GPU gap is the top-2 gap of its own logits
    return am, gap


def check_walk(gpu: dict, s: int, paths, am, gap, L: int, report: dict, greedy=None):
    """Walk of sequence s against the oracle's walk over the same rows (and the
    independent greedy decode when given), exact unless a visited row is a
    near-tie; always a valid root path whose tokens are row argmaxes."""
    n_rows = len(gpu["parent"][s])
    a = int(gpu["n_accept"][s])
    toks = gpu["out_tokens"][s]
    rows = gpu["path_rows"][s]
    g_am = gpu["argmax"][s * n_rows:(s + 1) * n_rows]
    assert 0 <= a <= L and rows[0] == 0
    for k in range(a + 1):
        assert toks[k] == g_am[rows[k]]
        if k:
            assert gpu["parent"][s][rows[k]] == rows[k - 1]
            assert gpu["token"][s][rows[k]] == toks[k - 1]
    assert np.all(toks[a + 1:] == -1) and np.all(rows[a + 1:] == -1)
    parent = gpu["parent"][s]
    token = gpu["token"][s]
    nv = int(gpu["n_valid"][s])
    oa, otoks, orows = wk.walk(parent, token, nv, am, L)
    flagged = bool(np.any(gap[orows] <= report.get("flag", GAP)))
    if flagged:
        report["walk_flagged"] = report.get("walk_flagged", 0) + 1
        return
    report["walk_exact"] = report.get("walk_exact", 0) + 1
    assert a == oa and list(toks[:a + 1]) == otoks and list(rows[:a + 1]) == orows
    if greedy is not None and not greedy["flagged"]:
        assert greedy["A"] == a and greedy["Y"][:a + 1] == otoks
