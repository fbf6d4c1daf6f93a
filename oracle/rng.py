"""Keyed randomness for the oracle: Philox4x64-10 and the integer inverse-CDF sampler.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages ask for random draws but fix no generator.  The reading used here
(stated in the design notes) is:

* Philox4x64 with 10 rounds, from Salmon, Moraes, Dror and Shaw, "Parallel random
  numbers: as easy as 1, 2, 3" (SC'11).  Key = (seed, sequence id); counter =
  (absolute position the draw decides, stream, iteration, 0).  Streams: 0 for the
  draft samples, 1 for the accept uniforms, 2 for the residual / bonus sample.
* A uniform in [0, 1 - 2^-24] is the top 24 bits of word 0 times 2^-24, exactly
  representable in float32.
* A categorical draw from non-negative float32 weights w is an inverse CDF over
  integers: W_j = trunc(w_j * 2^40), T = sum W_j, tau = floor(x * T / 2^64) with
  x = word 0, and the result is the smallest j whose running sum exceeds tau.
  Integer sums do not depend on summation order, so any correct parallel scan
  gives the same index.

Every function here is vectorised over numpy arrays of counters/keys.
"""
import numpy as np

U64 = np.uint64
MASK32 = U64(0xFFFFFFFF)

# Philox4x64 round multipliers and key-schedule (Weyl) constants, as published.
PHILOX_M0 = U64(0xD2E7470EE14C6C93)
PHILOX_M1 = U64(0xCA5A826395121157)
PHILOX_W0 = U64(0x9E3779B97F4A7C15)  # golden ratio
PHILOX_W1 = U64(0xBB67AE8584CAA73B)  # sqrt(3) - 1

STREAM_DRAFT = 0
STREAM_ACCEPT = 1
STREAM_RESAMPLE = 2


def mulhilo64(a, b):
    """Full 64x64 -> 128-bit product of uint64 arrays, returned as (hi, lo)."""
    a = np.asarray(a, dtype=U64)
    b = np.asarray(b, dtype=U64)
    a0, a1 = a & MASK32, a >> U64(32)
    b0, b1 = b & MASK32, b >> U64(32)
    p00 = a0 * b0
    p01 = a0 * b1
    p10 = a1 * b0
    p11 = a1 * b1
    mid = (p00 >> U64(32)) + (p01 & MASK32) + (p10 & MASK32)
    hi = p11 + (p01 >> U64(32)) + (p10 >> U64(32)) + (mid >> U64(32))
    lo = (mid << U64(32)) | (p00 & MASK32)
    return hi, lo


def philox4x64(ctr, key, rounds=10):
    """Philox4x64-R block function.

    ctr: uint64 array [..., 4]; key: uint64 array [..., 2] (broadcastable).
    Returns uint64 array [..., 4].  Each round multiplies words 0 and 2 by the two
    round constants, and the new state is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2),
    hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key gains the Weyl constants between
    rounds.
    """
    ctr = np.asarray(ctr, dtype=U64)
    key = np.asarray(key, dtype=U64)
    shape = np.broadcast_shapes(ctr.shape[:-1], key.shape[:-1])
    c = [np.broadcast_to(ctr[..., i], shape).copy() for i in range(4)]
    k0 = np.broadcast_to(key[..., 0], shape).copy()
    k1 = np.broadcast_to(key[..., 1], shape).copy()
    with np.errstate(over="ignore"):
        for r in range(rounds):
            if r > 0:
                k0 = k0 + PHILOX_W0
                k1 = k1 + PHILOX_W1
            hi0, lo0 = mulhilo64(PHILOX_M0, c[0])
            hi1, lo1 = mulhilo64(PHILOX_M1, c[2])
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return np.stack(c, axis=-1)


def draw_word(seed, seq_id, pos, stream, it, ctr3=0):
    """Word 0 of Philox(key=(seed, seq_id), counter=(pos, stream, it, ctr3)).

    All arguments broadcast; returns uint64.  ``ctr3`` is 0 for the linear
    sampler; the tree sampler puts the chain (draft) or trial (accept) index there.
    """
    seed, seq_id, pos, stream, it, ctr3 = np.broadcast_arrays(
        np.asarray(seed, dtype=U64), np.asarray(seq_id, dtype=U64),
        np.asarray(pos, dtype=U64), np.asarray(stream, dtype=U64),
        np.asarray(it, dtype=U64), np.asarray(ctr3, dtype=U64))
    ctr = np.stack([pos, stream, it, ctr3], axis=-1)
    key = np.stack([seed, seq_id], axis=-1)
    return philox4x64(ctr, key)[..., 0]


def unif24(word):
    """Uniform in [0, 1 - 2^-24] from the top 24 bits of a 64-bit word (float32)."""
    top = (np.asarray(word, dtype=U64) >> U64(40)).astype(np.float64)
    return (top * 2.0 ** -24).astype(np.float32)


def int_weights(w):
    """W_j = trunc(w_j * 2^40) for float32 weights in [0, 1]; uint64.

    Raises ValueError on NaN, negative or > 1 entries (the library reports these
    as a numeric error).
    """
    w = np.asarray(w, dtype=np.float32)
    wd = w.astype(np.float64)
    if np.isnan(wd).any() or (wd < 0).any() or (wd > 1).any():
        raise ValueError("sampler weights must be finite probabilities in [0, 1]")
    return np.floor(np.ldexp(wd, 40)).astype(U64)


def threshold(word, total):
    """tau = floor(word * total / 2^64), i.e. the high word of the 128-bit product."""
    hi, _ = mulhilo64(word, total)
    return hi


def sample_int(W, word):
    """Categorical draw over the last axis of integer weights ``W`` (uint64) using
    ``word``: the smallest j whose inclusive prefix sum exceeds floor(word * T /
    2^64).  Returns (index, total); index is -1 where T == 0."""
    W = np.asarray(W, dtype=U64)
    cum = np.cumsum(W, axis=-1, dtype=U64)
    total = cum[..., -1]
    tau = threshold(word, total)
    idx = np.sum(cum <= tau[..., None], axis=-1).astype(np.int64)
    idx = np.where(total == 0, -1, idx)
    return idx, total


def sample_icdf(w, word):
    """Categorical draw over the last axis of float32 weights ``w`` using ``word``.

    Returns (index, total) where total is the integer mass T; index is -1 where
    T == 0 (the caller decides the fallback).
    """
    W = int_weights(w)
    cum = np.cumsum(W, axis=-1, dtype=U64)
    total = cum[..., -1]
    tau = threshold(word, total)
    # smallest j with cum[j] > tau
    idx = np.sum(cum <= tau[..., None], axis=-1).astype(np.int64)
    idx = np.where(total == 0, -1, idx)
    return idx, total
