"""Oracle of the top-p (nucleus) truncation applied to the draft and verify laws.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages fix only the setting: their evaluations sample at temperature 1 with
top-p 0.95, and losslessness then holds with respect to that filtered law
([blog] "我的判断", the author's assessment).  Applying the same truncation to
both the AR law p and the draft law q keeps speculative rejection exact for the
filtered AR law.

Reading of "top-p" (standard nucleus truncation, made exact so that two
implementations agree bit for bit; listed in the design notes):
* masses are fixed point: w_i = floor(p_i * 2^40) (exact for float32 p_i <= 1),
  W = sum w_i (an exact integer sum, independent of order);
* the target mass is max(1, ceil(top_p * W)), top_p a float32 and the product
  taken in float64;
* the threshold tau is the largest probability value such that the tokens with
  p_i >= tau carry at least the target mass (ties with tau are kept);
* kept probabilities are divided by Z = float32(W_kept * 2^-40), W_kept the kept
  mass; the others become 0.  top_p >= 1 leaves a row unchanged, and so does a
  row with no fixed-point mass at all.
"""
import numpy as np

FX = 2.0 ** 40


def masses(row):
    """Fixed-point masses floor(p * 2^40) of a float32 row (exact in float64)."""
    return np.floor(np.asarray(row, dtype=np.float32).astype(np.float64) * FX).astype(np.int64)


def threshold(row, top_p):
    """The largest value tau of the row whose upper set {p >= tau} holds the target
    mass: the tokens are taken in decreasing order of p and tau is the value at
    which their running mass first reaches the target."""
    row = np.asarray(row, dtype=np.float32)
    w = masses(row)
    W = int(w.sum())
    target = max(1, int(np.ceil(np.float64(np.float32(top_p)) * np.float64(W))))
    order = np.argsort(-row, kind="stable")
    run = np.cumsum(w[order])
    j = int(np.searchsorted(run, target, side="left"))
    return row[order[j]], target


def filter_row(row, top_p):
    """Truncate one float32 probability row to its top-p nucleus and renormalise."""
    row = np.asarray(row, dtype=np.float32)
    if np.float32(top_p) >= 1.0 or masses(row).sum() == 0:
        return row.copy()
    tau, _ = threshold(row, top_p)
    keep = row >= tau
    w_kept = int(masses(row)[keep].sum())
    z = np.float32(np.float64(w_kept) / FX)
    out = np.zeros_like(row)
    out[keep] = row[keep] / z                  # float32 division
    return out


def filter_rows(rows, top_p):
    """filter_row over the last axis of an array of rows."""
    rows = np.asarray(rows, dtype=np.float32)
    flat = rows.reshape(-1, rows.shape[-1])
    return np.stack([filter_row(r, top_p) for r in flat]).reshape(rows.shape)
