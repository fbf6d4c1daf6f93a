"""Oracle of the tree Psi-Spec sampler (the batch-1 mode): several drafted chains
share one draft forward and one verify forward, and acceptance walks the tree of
their common prefixes with recursive rejection sampling.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix ([summary] method key points; [blog] "the Psi-Spec sampler:
draft, verify, two modes"): the sampler has a linear mode for system throughput
and a tree mode for the throughput of a single request; both draft from the noise
block in one step and verify with the AR model, and stay lossless.  The text that
described how the tree's candidate set is built did not survive on the pages.

Reading used here (listed in the design notes):
* one draft forward gives the laws q_1..q_B of the block (q_1 is the AR law of the
  first slot; q_2..q_B come from the diffusion path and do not depend on the
  tokens drawn for the other slots);
* K chains share the first token y_1 (always accepted) and draw their tokens at
  depths d = 2..B independently: chain k at depth d is a draw from q_d with the
  Philox counter (n + d, draft stream, iteration, k); chain 0 is exactly the
  linear sampler's draft;
* the verify forward scores every chain's block [y_1, y^k_2..y^k_B] at positions
  n+1..n+B with the AR weights; the law at depth d on chain k is that of the
  chain's row holding its depth d-1 token (the y_1 row for d = 2);
* acceptance walks depth d = 2, 3, ...: the live chains are those whose tokens
  match every accepted token so far, and they are tried in increasing chain
  order against a target law r that starts at p_d (the law of the lowest live
  chain).  Trial j (0-based) uses the uniform u_j of counter (n + d, accept stream,
  iteration, j).  Trial 0 accepts candidate c iff u_0 q_d(c) < p_d(c) in float32,
  the linear test.  A rejection replaces the target by the residual max(0, r - q_d)
  renormalised, kept as integer masses on the 2^-40 grid: after trial 0,
  R_1 = trunc(max(0, p_d - q_d) * 2^40) (the linear sampler's residual row, with
  its fallback to p_d when it has no mass); after trial j >= 1,
  R_{j+1} = R_j - min(R_j, floor(T_j * Q / 2^40)) with Q = trunc(q_d * 2^40) and
  T_j = sum R_j (kept unchanged if that leaves no mass).  Trial j >= 1 accepts c
  iff (u_j * q_d(c)) * T_j < R_j(c), evaluated in float64 with each product
  rounded (the first product is exact).  An accepted token extends the path and
  the live set shrinks to the chains that drew it; if every live chain fails at
  depth d, the emitted token z is drawn from the last residual with counter
  (n + d, resample stream, iteration, 0) and the step emits d tokens; if every
  depth passes, z is drawn from the bonus law p_{B+1} of the lowest live chain;
* the cache keeps the K/V of the accepted path (the lowest live chain's forward).

Why this is lossless: the candidates at a depth are independent draws from q_d,
independent of everything that decided the earlier depths (so also of which chains
are live), and recursive rejection against the running residual returns a draw
from the target law whatever the number of candidates (SpecInfer's multi-step
speculative sampling; for one candidate it is the linear rule).  With K = 1 the
procedure is the linear sampler, draw for draw.
"""
import numpy as np

from . import model
from . import psispec
from . import rng

U64 = np.uint64


def verify_row(k, depth, B):
    """Index of the verify row that holds chain k's token at `depth` (1..B): row 0
    is the shared y_1, then B-1 rows per chain for depths 2..B."""
    return 0 if depth == 1 else 1 + k * (B - 1) + (depth - 2)


def residual_first(p, q):
    """R_1: the linear sampler's residual row trunc(max(0, p - q) * 2^40) (float32
    subtraction), or trunc(p * 2^40) when that has no integer mass."""
    R = rng.int_weights(np.maximum(np.asarray(p, np.float32) - np.asarray(q, np.float32),
                                   np.float32(0.0)))
    if int(R.sum(dtype=U64)) == 0:
        R = rng.int_weights(p)
    return R


def residual_next(R, q):
    """R_{j+1} = R_j - min(R_j, floor(T_j * Q / 2^40)), Q = trunc(q * 2^40),
    T_j = sum R_j; R_j itself when that leaves no mass."""
    R = np.asarray(R, dtype=U64)
    Q = rng.int_weights(q)
    T = R.sum(dtype=U64)
    hi, lo = rng.mulhilo64(T, Q)
    sub = (hi << U64(24)) | (lo >> U64(40))
    out = R - np.minimum(R, sub)
    return out if int(out.sum(dtype=U64)) > 0 else R


def accept_trial(j, u, qc, pc, R, T):
    """Trial j's test of candidate c: u, qc (= q_d(c)), pc (= p_d(c)) float32."""
    if j == 0:
        return bool(np.float32(u) * np.float32(qc) < np.float32(pc))
    return (float(u) * float(qc)) * float(T) < float(R)


def tree_accept(p_rows, q_rows, chains, seed, seq_ids, n, it, broken=None):
    """Walk the candidate tree of each sequence.

    p_rows: float32 [S, 1 + K(B-1), V] -- verify laws (rows as in ``verify_row``)
    q_rows: float32 [S, B, V]          -- draft laws; depth d uses row d-1
    chains: int [S, K, B]              -- drafted tokens (column 0 is y_1 for all)
    n, it:  int [S]                    -- pending position and iteration
    Returns (out int32 [S, B+1] with -1 padding, n_out int32 [S], kstar int32 [S]:
    the lowest chain on the accepted path).

    ``broken`` plants a mistake for the tests' power controls: "no_residual" keeps
    testing later candidates against p_d (no residual update) and resamples from
    the first residual.
    """
    p_rows = np.asarray(p_rows, dtype=np.float32)
    q_rows = np.asarray(q_rows, dtype=np.float32)
    chains = np.asarray(chains, dtype=np.int64)
    S, K, B = chains.shape
    V = p_rows.shape[-1]
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    n = np.asarray(n, dtype=np.int64)
    it = np.asarray(it, dtype=np.int64)
    out = np.full((S, B + 1), -1, dtype=np.int32)
    n_out = np.zeros(S, dtype=np.int32)
    kstar = np.zeros(S, dtype=np.int32)
    if ((chains < 0) | (chains >= V)).any():
        raise ValueError("drafted token out of range")
    for s in range(S):
        sid, ns, its = seq_ids[s], n[s], it[s]
        live = list(range(K))
        path = [int(chains[s, 0, 0])]
        z_row = None                    # integer weights of the correction draw
        stop = B + 1
        for d in range(2, B + 1):
            p = p_rows[s, verify_row(live[0], d - 1, B)]
            q = q_rows[s, d - 1]
            R, T = None, None
            acc = None
            for j, k in enumerate(live):
                c = int(chains[s, k, d - 1])
                u = rng.unif24(rng.draw_word(seed, sid, ns + d, rng.STREAM_ACCEPT, its, j))
                if broken == "no_residual":
                    ok = accept_trial(0, u, q[c], p[c], None, None)
                else:
                    ok = accept_trial(j, u, q[c], p[c], None if R is None else R[c], T)
                if ok:
                    acc = c
                    break
                if broken == "no_residual":
                    if R is None:
                        R = residual_first(p, q)
                elif j == 0:
                    R = residual_first(p, q)
                else:
                    R = residual_next(R, q)
                T = R.sum(dtype=U64)
            if acc is None:
                stop = d
                z_row = R
                break
            path.append(acc)
            live = [k for k in live if int(chains[s, k, d - 1]) == acc]
        word = rng.draw_word(seed, sid, ns + stop, rng.STREAM_RESAMPLE, its)
        if stop == B + 1:
            z_row = rng.int_weights(p_rows[s, verify_row(live[0], B, B)])
        z, total = rng.sample_int(z_row, word)
        if int(total) == 0:
            raise ValueError("probability row with no integer mass")
        out[s, : stop - 1] = path[: stop - 1]
        out[s, stop - 1] = z
        n_out[s] = stop
        kstar[s] = live[0]
    return out, n_out, kstar


def draft_chains(P_d, K, seed, seq_ids, n, it):
    """K chains [S, K, B] from the draft laws P_d [S, B, V]: y_1 shared (counter
    word 3 = 0), chain k's depth-d token with counter word 3 = k."""
    S, B, _ = P_d.shape
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    chains = np.empty((S, K, B), dtype=np.int64)
    for d in range(1, B + 1):
        for k in range(K):
            word = rng.draw_word(seed, seq_ids, np.asarray(n) + d, rng.STREAM_DRAFT, it,
                                 0 if d == 1 else k)
            idx, total = rng.sample_icdf(P_d[:, d - 1], word)
            if (total == 0).any():
                raise ValueError("draft row with no integer mass")
            chains[:, k, d - 1] = idx
    return chains


class TreeDecoder(psispec.Decoder):
    """The decoder of ``psispec`` with the tree step."""

    def verify_tree(self, chains):
        """Verify every chain against its own copy of the cache.  Returns
        (P_v float32 [S, 1 + K(B-1), V], the K cache copies)."""
        cfg, S = self.cfg, self.S
        _, K, B = chains.shape
        P_v = np.zeros((S, 1 + K * (B - 1), cfg.vocab), dtype=np.float32)
        caches = []
        pos = self.n[:, None] + 1 + np.arange(B)[None, :]
        for k in range(K):
            ck = {"k": self.cache["k"].copy(), "v": self.cache["v"].copy()}
            logits, _ = model.forward(cfg, self.w, chains[:, k], pos, np.zeros((S, B)), ck)
            law = self._law(logits)
            if k == 0:
                P_v[:, 0] = law[:, 0]
            P_v[:, 1 + k * (B - 1): 1 + (k + 1) * (B - 1)] = law[:, 1:]
            caches.append(ck)
        return P_v, caches

    def step_tree(self, K, broken=None):
        """One tree iteration with K chains.  Returns dict with out, n_out, kstar,
        chains, P_d, P_v."""
        P_d = self.draft_laws()
        chains = draft_chains(P_d, K, self.seed, self.seq_ids, self.n, self.it)
        P_v, caches = self.verify_tree(chains)
        out, n_out, kstar = tree_accept(P_v, P_d, chains, self.seed, self.seq_ids, self.n,
                                        self.it, broken=broken)
        for s in range(self.S):
            src = caches[int(kstar[s])]
            self.cache["k"][:, s] = src["k"][:, s]
            self.cache["v"][:, s] = src["v"][:, s]
        self.n = self.n + n_out
        self.t = out[np.arange(self.S), n_out - 1].astype(np.int64)
        self.it = self.it + 1
        self.forwards += 2
        return {"out": out, "n_out": n_out, "kstar": kstar, "chains": chains, "P_d": P_d,
                "P_v": P_v}
