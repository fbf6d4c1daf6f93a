"""Pins of the top-p truncation oracle (oracle/nucleus.py) against what the
definition fixes independently of its sort-and-scan implementation: a brute
force over every candidate threshold, the limits top_p >= 1 (identity) and
top_p -> 0 (the argmax set), a worked example, and invariants of the result."""
import numpy as np
import pytest

from oracle import nucleus


def _brute_tau(row, top_p):
    """Largest distinct value t with mass{p >= t} >= target, by trying them all."""
    row = np.asarray(row, dtype=np.float32)
    w = np.floor(row.astype(np.float64) * 2.0 ** 40).astype(np.int64)
    target = max(1, int(np.ceil(np.float64(np.float32(top_p)) * np.float64(int(w.sum())))))
    best = None
    for t in np.unique(row):
        if int(w[row >= t].sum()) >= target and (best is None or t > best):
            best = t
    return best


@pytest.mark.parametrize("seed", range(40))
def test_threshold_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(3, 14))
    logits = rng.integers(-3, 4, size=V).astype(np.float64) * 0.7    # many ties
    p = np.exp(logits - logits.max())
    p = (p / p.sum()).astype(np.float32)
    for top_p in (0.05, 0.3, 0.5, 0.8, 0.95, 0.999):
        tau, _ = nucleus.threshold(p, top_p)
        assert tau == _brute_tau(p, top_p)


def test_identity_at_one_and_argmax_at_zero():
    rng = np.random.default_rng(7)
    p = rng.random(50).astype(np.float32)
    p[[3, 17]] = p.max() + 0.5                      # a tied maximum
    p = (p / p.sum()).astype(np.float32)
    assert np.array_equal(nucleus.filter_row(p, 1.0), p)
    assert np.array_equal(nucleus.filter_row(p, 1.5), p)
    tiny = nucleus.filter_row(p, 1e-9)
    assert set(np.flatnonzero(tiny)) == {3, 17}     # the argmax set, ties kept
    assert tiny[3] == tiny[17]


def test_worked_example():
    p = np.array([0.5, 0.3, 0.15, 0.05], dtype=np.float32)
    out = nucleus.filter_row(p, 0.75)               # 0.5 + 0.3 >= 0.75 > 0.5
    assert np.flatnonzero(out).tolist() == [0, 1]
    assert abs(out[0] - 0.625) < 1e-6 and abs(out[1] - 0.375) < 1e-6
    out = nucleus.filter_row(p, 0.85)               # needs the 0.15 token as well
    assert np.flatnonzero(out).tolist() == [0, 1, 2]
    # dyadic masses: the running mass meets the target exactly at the second token,
    # which must then close the nucleus ("at least the target", not "more than")
    d = np.array([0.5, 0.25, 0.125, 0.125], dtype=np.float32)
    out = nucleus.filter_row(d, 0.75)
    assert out.tolist() == [np.float32(0.5 / 0.75), np.float32(0.25 / 0.75), 0.0, 0.0]


@pytest.mark.parametrize("V,top_p", [(32, 0.9), (2080, 0.95), (151936, 0.95), (151936, 0.5)])
def test_invariants_on_softmax_rows(V, top_p):
    rng = np.random.default_rng(V)
    logits = rng.normal(0.0, 3.0, size=V)
    p = np.exp(logits - logits.max())
    p = (p / p.sum()).astype(np.float32)
    out = nucleus.filter_row(p, top_p)
    kept = out > 0
    tau, target = nucleus.threshold(p, top_p)
    # support: exactly the upper set {p >= tau}, and nothing smaller is needed
    assert np.array_equal(kept, p >= tau)
    w = nucleus.masses(p)
    assert int(w[kept].sum()) >= target
    assert int(w[p > tau].sum()) < target
    # renormalised: sums to 1 up to float32 rounding; ratios preserved
    assert abs(float(out.astype(np.float64).sum()) - 1.0) < 1e-5
    idx = np.flatnonzero(kept)
    if len(idx) >= 2:
        i, j = idx[np.argsort(-p[idx])][[0, -1]]
        assert abs(out[i] / out[j] - p[i] / p[j]) < 1e-5 * (p[i] / p[j])
