"""One verify round, end to end, on the CPU (test infrastructure only).

Steps, in the order of the paper's Fig. 2 round and the project page's
"Draft pass" / "Verify pass":
  1. log q_j of every draft marginal                        (draft.log_softmax)
  2. the top-N prefix-closed tree and its row layout        (tree.*)
  3. every verify row evaluated on its own sequence         (model.evaluate_paths)
  4. head logits and row statistics                         (model.row_stats)
  5. the walk over those rows, and independently the greedy
     continuation Y with A(S) from its definition            (walk.*)
"""
from __future__ import annotations

import numpy as np

from . import draft, model as mdl, tree as tr, walk as wk
from .numerics import decode

GAP_FLAG = 1e-3  # logit units; top-2 gaps at or below this are near-ties


def build_tree(logits_stored, dtype: str, root: int, N: int, exact: str = "beam"):
    """Steps 1-2 for one sequence: returns a dict with log q, the node paths in
    >- order, their scores, the layout arrays and the boundary gap
    (score of the N-th node minus that of the best non-member)."""
    logq = draft.log_softmax(decode(logits_stored, dtype))
    fn = tr.brute_force_top_n if exact == "brute" else tr.level_beam_top_n
    top, scores, nxt = fn(logq, N)
    parent, depth, token, anc, n_valid, order = tr.canonical_layout(top, root, N)
    score = np.full(N + 1, -np.inf)
    score[0] = 0.0
    for i, p in enumerate(order[1:], start=1):
        score[i] = scores[p]
    bgap = (scores[top[-1]] - nxt) if (len(top) == N and N > 0) else np.inf
    return {"logq": logq, "top": top, "scores": scores, "next_score": nxt,
            "parent": parent, "depth": depth, "token": token, "anc": anc,
            "score": score, "n_valid": n_valid, "order": order,
            "boundary_gap": bgap}


def verify_rows(model: mdl.TargetModel, s: int, root: int, order: list, N: int):
    """Steps 3-4 for the rows of one sequence laid out as ``order`` (row i is the
    path order[i]).  Padding rows (past len(order)) are left at NaN."""
    ev = mdl.evaluate_paths(model, s, root, order)
    z = model.logits(ev["final"])
    am, top1, gap, H = mdl.row_stats(z)
    n = len(order)
    R = N + 1

    def pad(x, fill=np.nan):
        out = np.full((R,) + x.shape[1:], fill, dtype=np.float64)
        out[:n] = x
        return out

    return {"attn": [pad(a) for a in ev["attn"]], "h": [pad(h) for h in ev["h"]],
            "logits": pad(z), "argmax": pad(am.astype(np.float64), -1).astype(np.int64),
            "top1": pad(top1), "gap": pad(gap), "entropy": pad(H)}


def continuation(model: mdl.TargetModel, s: int, root: int, top: list, L: int):
    """Step 5 by definition: greedy Y decoded independently of the verify rows,
    then A(S), the committed tokens Y_{1:A} and the new root Y_{A+1}."""
    tree = set(top)
    Y, zrows = wk.greedy_continuation(model, s, root, tree, L)
    A = wk.accepted_length(Y, tree)
    _, _, gaps, _ = mdl.row_stats(np.stack(zrows))
    return {"Y": Y, "A": A, "committed": Y[:A], "new_root": Y[A],
            "Y_gaps": gaps, "flagged": bool(np.any(gaps[:A + 1] <= GAP_FLAG))}


def oracle_round(inp: dict, r: int = 0, exact: str = "beam", continuation_check=True):
    """Every step of round r of a synthetic workload, per sequence."""
    cfg = inp["cfg"]
    rd = inp["rounds"][r]
    model = inp.get("_oracle_model") or mdl.TargetModel(inp)
    out = []
    for s in range(cfg.nseq):
        root = int(rd["root"][s])
        if "draft_logits" in rd:
            t = build_tree(rd["draft_logits"][s], cfg.dtype, root, cfg.N, exact)
        else:
            parent, token, n_valid = rd["parent"][s], rd["token"][s], cfg.N + 1
            order = [()] + tr.paths_from_layout(parent, token, n_valid)
            t = {"order": order, "top": order[1:], "parent": parent,
                 "depth": rd["depth"][s], "token": token, "anc": rd["anc"][s],
                 "n_valid": n_valid, "boundary_gap": np.inf}
        rows = verify_rows(model, s, root, t["order"], cfg.N)
        a, toks, path = wk.walk(t["parent"], t["token"], t["n_valid"], rows["argmax"], cfg.L)
        res = {"tree": t, "rows": rows, "walk": {"a": a, "tokens": toks, "rows": path,
               "flagged": bool(np.any(rows["gap"][path] <= GAP_FLAG))}}
        if continuation_check:
            res["greedy"] = continuation(model, s, root, t["top"], cfg.L)
        out.append(res)
    return out


def multi_round(model: mdl.TargetModel, s: int, root: int, draft_fn, n_rounds: int, dtype: str,
                N: int, L: int):
    """Rounds of the method chained by committing each round's accepted path
    (paper §3.1: a round commits A(S) + 1 tokens, the last of which is the next
    round's root; App. B.1: the next round conditions on x o b o Y_{1:A(S)}).

    Round r builds its tree from draft_fn(r, stream) (stored draft logits
    [L][V]) at the current root, evaluates every
    node on its explicit sequence after the prefix and every token committed so
    far, walks, and appends the walk's tokens to the stream.  Returns the stream
    [b, t_1, t_2, ..] (the first root, then every committed token and later root
    in order) and per round (A(S), the smallest top-2 gap on the walk)."""
    stream = [int(root)]
    rounds = []
    for r in range(n_rounds):
        z = draft_fn(r, stream)
        b = stream[-1]
        t = build_tree(z, dtype, b, N, "beam")
        ctx = tuple(stream[1:])          # committed tokens after the first root, ending at b
        order = t["order"]
        paths = [ctx[:j] for j in range(len(ctx))] + [ctx + p for p in order]
        ev = mdl.evaluate_paths(model, s, stream[0], paths)
        zr = model.logits(ev["final"][len(ctx):])
        am, _, gap, _ = mdl.row_stats(zr)
        a, toks, rows = wk.walk(t["parent"], t["token"], t["n_valid"], am, L)
        rounds.append((a, float(np.min(gap[rows]))))
        stream.extend(int(x) for x in toks)
    return stream, rounds
