"""Pins of the sampling oracle: Philox4x32-10 against the known-answer vectors
published with the Random123 library (Salmon et al. 2011), and the Gumbel-max
draw against softmax(z / T) by a chi-square test."""
import numpy as np
from scipy import stats

from oracle import sample as sp


def _kat(ctr, key):
    return [int(x) for x in sp.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]]


def test_philox4x32_10_known_answers():
    assert _kat([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    m = 0xFFFFFFFF
    assert _kat([m, m, m, m], [m, m]) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert _kat([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_uniforms_are_open_and_distinct_per_stream():
    u = sp.uniforms(7, 3, 2, 1001)
    assert u.min() > 0.0 and u.max() < 1.0
    assert not np.array_equal(u, sp.uniforms(7, 3, 1, 1001))   # another row
    assert not np.array_equal(u, sp.uniforms(7, 4, 2, 1001))   # another round
    assert not np.array_equal(u, sp.uniforms(8, 3, 2, 1001))   # another seed
    assert np.array_equal(u[:500], sp.uniforms(7, 3, 2, 500))  # a prefix of the row's stream
    # every grid point is a float32 value strictly inside (0, 1): the kernel's
    # float32 noise is then that of the same U, and never infinite
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    ends = (np.array([0, 2**23 - 1], dtype=np.float64) + 0.5) / 2**23
    assert np.all(ends.astype(np.float32) == ends) and np.float32(ends[1]) < 1.0
    assert np.all(np.isfinite(-np.log(-np.log(ends.astype(np.float32)))))


def test_gumbel_max_draws_follow_softmax():
    z = np.array([[1.0, 0.2, -0.5, 2.0, 0.0, -3.0, 1.5]])
    for T in (1.0, 0.5):
        n = 6000
        draws = np.array([sp.sample_rows(z, T, 11, r)[0][0] for r in range(n)])
        p = np.exp(z[0] / T - np.max(z[0] / T))
        p /= p.sum()
        obs = np.bincount(draws, minlength=z.shape[1])
        chi2, pval = stats.chisquare(obs, p * n)
        assert pval > 1e-4, (T, obs, p * n, pval)


def test_sample_rows_ties_and_gap():
    z = np.zeros((3, 5))
    tok, gap = sp.sample_rows(z, 1.0, 1, 2)
    assert tok.shape == (3,) and np.all(gap >= 0)
    # a dominant logit is always drawn at low temperature
    z[:, 3] = 50.0
    tok, _ = sp.sample_rows(z, 0.5, 1, 2)
    assert list(tok) == [3, 3, 3]
