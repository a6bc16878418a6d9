"""Storage-precision helpers of the oracle (test infrastructure only).

bfloat16 here is the storage format of the bf16 workloads: 8 significant bits,
round to nearest, ties to even.  The oracle decodes stored bits exactly and
rounds float64 values to bf16 only at the storage points of the verify pass
(tree-row K/V entries and each layer's output), computing in float64 elsewhere.
"""
import numpy as np


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (float32 values, or bf16 bit patterns as uint16) -> float64."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    Written from the format's definition: with x = m * 2**e and 0.5 <= |m| < 1,
    a bf16 value keeps 8 significant bits, i.e. m rounded to a multiple of 2**-8.
    np.rint rounds halves to even.  (Values of the workloads are far from the
    bf16 subnormal and overflow ranges.)"""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage format at a storage point (identity for fp32 runs,
    which the oracle keeps in float64 throughout)."""
    return round_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)
