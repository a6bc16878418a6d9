"""Shared pieces of the chained-round tests: a workload whose rotary tables cover
many rounds, and draft logits that favour the reference greedy stream (so that
rounds accept several tokens) while staying seeded and synthetic."""
import numpy as np

from synth import bf16_bits, gen_round, make_config
from synth.gen import rope_tables


def chained_workload(name: str, seed: int, n_rounds: int, **overrides):
    cfg = make_config(name, **overrides)
    inp = gen_round(cfg, seed)
    P = int(inp["prefix_len"][0])
    n_pos = P + (n_rounds + 1) * (cfg.L + 1) + cfg.N + 1
    inp["rope_cos"], inp["rope_sin"] = rope_tables(n_pos, cfg.D, cfg.rope_theta)
    return cfg, inp


def favoured_draft(cfg, greedy: list, m: int, rng, hit: float = 0.8) -> np.ndarray:
    """Draft logits [1][L][V] for a round whose next token is greedy[m]: offset j
    puts a large logit on greedy[m + j] with probability ``hit``, else on a random
    token, over N(0, 1) noise (the spike, +12, stands out of any row of at most
    a few hundred thousand tokens)."""
    z = rng.normal(0.0, 1.0, (1, cfg.L, cfg.V))
    for j in range(cfg.L):
        t = m + j
        tok = greedy[t] if t < len(greedy) and rng.random() < hit else int(rng.integers(cfg.V))
        z[0, j, tok] += 12.0
    z = z.astype(np.float32)
    return bf16_bits(z) if cfg.dtype == "bf16" else z


def agreed_prefix(gaps: list, flag: float) -> int:
    """Tokens of the reference stream before its first near-tie (gap <= flag)."""
    for i, g in enumerate(gaps):
        if g <= flag:
            return i
    return len(gaps)
