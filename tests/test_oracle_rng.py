"""Pins of the oracle's keyed randomness against things other than itself:
numpy's Philox implementation, the published Philox known-answer vectors, Python's
big integers, and brute-force enumeration of the integer inverse CDF."""
import json
import os

import numpy as np
import pytest

from oracle import rng

U = np.uint64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_mulhilo_matches_python_bigints():
    r = np.random.default_rng(1)
    a = r.integers(0, 2**64 - 1, size=5000, dtype=np.uint64, endpoint=True)
    b = r.integers(0, 2**64 - 1, size=5000, dtype=np.uint64, endpoint=True)
    a[:4] = [0, 1, 2**64 - 1, 2**63]
    b[:4] = [2**64 - 1, 2**64 - 1, 2**64 - 1, 2]
    hi, lo = rng.mulhilo64(a, b)
    for x, y, h, l in zip(a.tolist(), b.tolist(), hi.tolist(), lo.tolist()):
        p = x * y
        assert h == p >> 64 and l == p & (2**64 - 1)


def test_philox_known_answers():
    """Published Philox4x64-10 known-answer vectors (Random123 distribution)."""
    with open(os.path.join(GOLDEN, "philox4x64_10_kat.json")) as f:
        kat = json.load(f)
    for case in kat["cases"]:
        ctr = np.array([int(x, 16) for x in case["ctr"]], dtype=U)
        key = np.array([int(x, 16) for x in case["key"]], dtype=U)
        out = rng.philox4x64(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in case["out"]]


def test_philox_matches_numpy_philox():
    """numpy.random.Philox is Philox4x64-10; its random_raw() bumps the counter
    before encrypting, so our block at counter c equals numpy's first block after
    seeding the counter with c - 1."""
    r = np.random.default_rng(7)
    n = 10_000
    keys = r.integers(0, 2**64 - 1, size=(n, 2), dtype=np.uint64, endpoint=True)
    ctrs = r.integers(0, 2**64 - 1, size=(n, 4), dtype=np.uint64, endpoint=True)
    ctrs[:, 0] |= U(1)  # counter word 0 >= 1, so c - 1 needs no borrow
    ours = rng.philox4x64(ctrs, keys)
    for i in range(n):
        c = ctrs[i].copy()
        c[0] -= U(1)
        bg = np.random.Philox(key=keys[i], counter=c)
        assert np.array_equal(bg.random_raw(4), ours[i]), i


def test_draw_word_layout():
    """draw_word is word 0 of Philox(key=(seed, seq), ctr=(pos, stream, iter, 0))."""
    w = rng.draw_word(11, 3, 17, 2, 5)
    bg = np.random.Philox(key=np.array([11, 3], dtype=U),
                          counter=np.array([16, 2, 5, 0], dtype=U))
    assert int(w) == int(bg.random_raw(4)[0])


def test_unif24_closed_form():
    words = np.array([0, 2**40 - 1, 2**40, 2**63, 2**64 - 1], dtype=U)
    u = rng.unif24(words)
    assert u.dtype == np.float32
    assert u.tolist() == [0.0, 0.0, 2.0**-24, 0.5, 1.0 - 2.0**-24]


def test_threshold_matches_bigints():
    r = np.random.default_rng(3)
    x = r.integers(0, 2**64 - 1, size=2000, dtype=np.uint64, endpoint=True)
    t = r.integers(1, 2**57, size=2000, dtype=np.uint64)
    tau = rng.threshold(x, t)
    for xi, ti, ta in zip(x.tolist(), t.tolist(), tau.tolist()):
        assert ta == (xi * ti) >> 64
        assert 0 <= ta < ti


def test_int_weights_exact_scaling():
    w = np.array([0.0, 1.0, 0.5, 2.0**-40, 2.0**-41, 0.1], dtype=np.float32)
    W = rng.int_weights(w)
    assert W.tolist()[:5] == [0, 2**40, 2**39, 1, 0]
    # float32(0.1) * 2^40 truncated, computed with exact rationals
    from fractions import Fraction
    assert W[5] == int(Fraction(float(np.float32(0.1))) * 2**40)
    with pytest.raises(ValueError):
        rng.int_weights(np.array([0.5, np.nan], dtype=np.float32))
    with pytest.raises(ValueError):
        rng.int_weights(np.array([0.5, -0.25], dtype=np.float32))


def _word_for_tau(tau, total):
    """Smallest 64-bit word whose threshold against ``total`` is ``tau``."""
    return -((-tau << 64) // total)


def test_icdf_brute_force_counts():
    """Enumerating every threshold tau in [0, T) selects index j exactly W_j times;
    zero-weight entries are never chosen."""
    r = np.random.default_rng(5)
    for trial in range(20):
        V = int(r.integers(1, 9))
        Wint = r.integers(0, 6, size=V)
        if trial % 3 == 0:
            Wint[r.integers(0, V)] = 0
        if Wint.sum() == 0:
            Wint[0] = 1
        w = (Wint * 2.0**-40).astype(np.float32)   # exact: W_j = Wint_j
        T = int(Wint.sum())
        counts = np.zeros(V, dtype=np.int64)
        for tau in range(T):
            word = _word_for_tau(tau, T)
            assert int(rng.threshold(np.uint64(word), np.uint64(T))) == tau
            idx, tot = rng.sample_icdf(w, np.uint64(word))
            assert int(tot) == T
            counts[int(idx)] += 1
        assert counts.tolist() == Wint.tolist()


def test_icdf_zero_total_and_extremes():
    idx, tot = rng.sample_icdf(np.zeros(5, dtype=np.float32), np.uint64(123))
    assert int(idx) == -1 and int(tot) == 0
    w = np.array([0, 0, 1, 0], dtype=np.float32)
    for word in (0, 2**63, 2**64 - 1):
        idx, _ = rng.sample_icdf(w, np.uint64(word))
        assert int(idx) == 2
    # word 0 -> tau 0 -> first nonzero; word max -> last nonzero
    w = np.array([0, 0.25, 0.25, 0, 0.5, 0], dtype=np.float32)
    assert int(rng.sample_icdf(w, np.uint64(0))[0]) == 1
    assert int(rng.sample_icdf(w, np.uint64(2**64 - 1))[0]) == 4


def test_icdf_frequencies_match_weights():
    """Over many keyed draws the empirical frequencies match the weights (chi^2)."""
    from scipy import stats
    w = np.array([0.05, 0.3, 0.0, 0.15, 0.5], dtype=np.float32)
    n = 40_000
    words = rng.draw_word(9, np.arange(n), 0, 0, 0)
    idx, _ = rng.sample_icdf(np.broadcast_to(w, (n, 5)), words)
    counts = np.bincount(idx, minlength=5)
    assert counts[2] == 0
    nz = w > 0
    chi = stats.chisquare(counts[nz], n * w[nz] / w[nz].sum())
    assert chi.pvalue > 1e-3
