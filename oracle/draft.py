"""Log-domain draft marginals (test infrastructure only).

The paper (§3.2, Assumption 1) has the drafter return one marginal
q_j(. | x, b) over the vocabulary at every offset j = 1..L; the project page
("Draft pass") says the same with L = B - 1 = 15.  The draft head emits logits,
so q_j = softmax(z_j) and the oracle works with log q_j, which ranks prefixes
exactly as the product of marginals does.
"""
import numpy as np


def log_softmax(z: np.ndarray) -> np.ndarray:
    """log q_j(v) = (z_jv - max_w z_jw) - ln sum_w exp(z_jw - max_w z_jw),
    row-wise over the last axis, in float64."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    s = np.exp(z - m).sum(axis=-1, keepdims=True)
    return (z - m) - np.log(s)


def entropy_nats(logq: np.ndarray) -> np.ndarray:
    """-sum_v q(v) ln q(v) of each row of log-probabilities."""
    q = np.exp(logq)
    return -(q * logq).sum(axis=-1)
