"""Oracle of the linear Psi-Spec sampler: prefill, draft, verify, accept/resample, commit.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix ([blog] "the Psi-Spec sampler: draft, verify, two modes";
[summary] method key points; [blog] "method core"):
* the drafting side takes one step from the noise block: the block's first token
  is sampled with the AR base weights only, so it is always accepted, and the
  other B-1 tokens come from the diffusion path (base + LoRA) in parallel;
* the verifying side is the standard speculative rejection correction: the AR
  model scores the whole block in parallel, the longest accepted prefix is kept,
  and the first rejected position is resampled from the renormalised residual;
* every iteration costs two forwards, so tokens per forward lies in [1, (B+1)/2]
  and every iteration emits at least two tokens;
* draft and verify share the KV cache; the output distribution is the AR model's.

Readings where the pages are silent (each listed in the design notes):
* draft rows are [t, MASK x (B-1)] at positions n..n+B-1 (t = pending token, not
  yet cached), gate [0, 1, ..., 1]; row r predicts the token at n+r+1, so
  y_1 ~ p (row 0, AR-exact) and y_i ~ q_i = probs(draft row i-1), i = 2..B;
* verify rows are [y_1..y_B] at positions n+1..n+B with gate 0;
  p_i = probs(verify row i-2) for i = 2..B+1 (p_{B+1} is the bonus row);
* accept y_i iff u_i * q_i(y_i) < p_i(y_i) in float32 (one multiply, strict <);
  at the first failure k, z ~ max(0, p_k - q_k) (or p_k when that residual has no
  integer mass); if none fails, k = B+1 and z ~ p_{B+1};
* emitted tokens are y_1..y_{k-1}, z (k of them); the cache keeps positions
  n..n+k-1; then n <- n+k, t <- z, iteration += 1;
* prefill runs the AR forward over prompt[0..P-2] and leaves prompt[P-1] pending;
* random draws use rng.draw_word with the (position, stream, iteration) counter;
* with top-p on, the nucleus truncation (nucleus.filter_row) is applied to every
  draft and verify row right after the softmax, so q and p above are the filtered
  laws and the output distribution is the filtered AR law.
"""
import numpy as np

from . import model
from . import nucleus
from . import rng


def accept_block(p_rows, q_rows, drafts, seed, seq_ids, n, it,
                 broken=None):
    """Accept/reject the drafted block and resample; vectorised over sequences.

    p_rows: float32 [S, B, V]  -- p_2 .. p_{B+1} (AR verify probabilities)
    q_rows: float32 [S, B-1, V] -- q_2 .. q_B (draft probabilities of slots 2..B)
    drafts: int [S, B]          -- y_1 .. y_B
    n, it:  int [S]             -- the pending position and iteration of each sequence
    Returns (out int32 [S, B+1] with -1 padding, n_out int32 [S]).

    ``broken`` plants a deliberate mistake for the tests' power controls:
    "resample_p" draws the correction from p_k instead of the residual,
    "always_accept" skips the test.
    """
    p_rows = np.asarray(p_rows, dtype=np.float32)
    q_rows = np.asarray(q_rows, dtype=np.float32)
    drafts = np.asarray(drafts, dtype=np.int64)
    S, B = drafts.shape
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    n = np.asarray(n, dtype=np.int64)
    it = np.asarray(it, dtype=np.int64)
    sidx = np.arange(S)

    k = np.full(S, B + 1, dtype=np.int64)
    undecided = np.ones(S, dtype=bool)
    for i in range(2, B + 1):
        y = drafts[:, i - 1]
        q_y = q_rows[sidx, i - 2, y]
        p_y = p_rows[sidx, i - 2, y]
        u = rng.unif24(rng.draw_word(seed, seq_ids, n + i, rng.STREAM_ACCEPT, it))
        ok = (u * q_y) < p_y          # float32 multiply, strict compare
        if broken == "always_accept":
            ok = np.ones(S, dtype=bool)
        rej = undecided & ~ok
        k[rej] = i
        undecided &= ok

    # the correction row: residual of the first rejected slot, or the bonus row
    word = rng.draw_word(seed, seq_ids, n + k, rng.STREAM_RESAMPLE, it)
    rejected = k <= B
    kk = np.minimum(k, B)                    # index helper; unused where not rejected
    pk = p_rows[sidx, kk - 2]
    qk = q_rows[sidx, np.minimum(kk - 2, B - 2)] if B >= 2 else np.zeros_like(pk)
    resid = np.maximum(pk - qk, np.float32(0.0))      # float32 subtraction
    if broken == "resample_p":
        resid = pk
    row = np.where(rejected[:, None], resid, p_rows[:, B - 1])
    z, total = rng.sample_icdf(row, word)
    # a residual with no integer mass (p ~= q) falls back to p_k itself
    empty = rejected & (total == 0)
    if empty.any():
        z2, total2 = rng.sample_icdf(pk[empty], word[empty])
        z[empty], total[empty] = z2, total2
    if (total == 0).any():
        raise ValueError("probability row with no integer mass")

    out = np.full((S, B + 1), -1, dtype=np.int32)
    for s in range(S):
        ks = int(k[s])
        out[s, : ks - 1] = drafts[s, : ks - 1]
        out[s, ks - 1] = z[s]
    return out, k.astype(np.int32)


class Decoder:
    """Psi-Spec decoding state of S sequences against one contiguous KV cache."""

    def __init__(self, cfg, weights, seq_ids, seed, max_len, top_p=1.0):
        self.cfg = cfg
        self.top_p = top_p
        self.w = weights
        self.seq_ids = np.asarray(seq_ids, dtype=np.int64)
        self.seed = int(seed)
        S = len(self.seq_ids)
        self.cache = model.new_cache(cfg, S, max_len)
        self.n = np.zeros(S, dtype=np.int64)
        self.t = np.zeros(S, dtype=np.int64)
        self.it = np.zeros(S, dtype=np.int64)
        self.forwards = 0

    def _law(self, logits):
        """Softmax of the logits, then (0 < top_p < 1) the nucleus truncation of
        each row: the same filter on the draft and the AR law."""
        P = model.probs(logits)
        if 0.0 < self.top_p < 1.0:
            P = nucleus.filter_rows(P, self.top_p)
        return P

    @property
    def S(self):
        return len(self.seq_ids)

    def _sub(self, rows):
        return {"k": self.cache["k"][:, rows], "v": self.cache["v"][:, rows]}

    def prefill(self, prompts):
        """AR forward over prompt[0..P-2]; prompt[P-1] becomes the pending token.

        ``prompts`` is a list of 1-D int arrays (lengths may differ, each >= 1).
        """
        for s, pr in enumerate(prompts):
            pr = np.asarray(pr, dtype=np.int64)
            P = len(pr)
            if P > 1:
                sub = self._sub(slice(s, s + 1))
                model.forward(self.cfg, self.w, pr[None, : P - 1],
                              np.arange(P - 1)[None, :], np.zeros((1, P - 1)), sub,
                              want_logits=False)
            self.n[s] = P - 1
            self.t[s] = pr[-1]
            self.it[s] = 0

    def draft_laws(self):
        """The draft forward: P_d float32 [S, B, V] (row j is the law of position n+j+1)."""
        cfg, B, S = self.cfg, self.cfg.block_size, self.S
        toks = np.full((S, B), cfg.mask_id, dtype=np.int64)
        toks[:, 0] = self.t
        pos = self.n[:, None] + np.arange(B)[None, :]
        gate = np.ones((S, B))
        gate[:, 0] = 0.0
        logits, _ = model.forward(cfg, self.w, toks, pos, gate, self.cache)
        return self._law(logits)

    def draft(self):
        """Draft forward and draft sampling.  Returns (y [S, B], P_d float32 [S, B, V])."""
        B, S = self.cfg.block_size, self.S
        P_d = self.draft_laws()
        y = np.empty((S, B), dtype=np.int64)
        for j in range(1, B + 1):
            word = rng.draw_word(self.seed, self.seq_ids, self.n + j, rng.STREAM_DRAFT, self.it)
            idx, total = rng.sample_icdf(P_d[:, j - 1], word)
            if (total == 0).any():
                raise ValueError("draft row with no integer mass")
            y[:, j - 1] = idx
        return y, P_d

    def verify(self, y):
        """AR-only verify forward of the drafted block.  Returns P_v float32 [S, B, V]."""
        cfg, B, S = self.cfg, self.cfg.block_size, self.S
        pos = self.n[:, None] + 1 + np.arange(B)[None, :]
        logits, _ = model.forward(cfg, self.w, y, pos, np.zeros((S, B)), self.cache)
        return self._law(logits)

    def step(self, broken=None):
        """One Psi-Spec iteration.  Returns dict with out, n_out, y, P_d, P_v."""
        y, P_d = self.draft()
        P_v = self.verify(y)
        out, n_out = accept_block(P_v, P_d[:, 1:], y, self.seed, self.seq_ids,
                                  self.n, self.it, broken=broken)
        self.n = self.n + n_out
        self.t = out[np.arange(self.S), n_out - 1].astype(np.int64)
        self.it = self.it + 1
        self.forwards += 2
        return {"out": out, "n_out": n_out, "y": y, "P_d": P_d, "P_v": P_v}

    def ar_single(self):
        """One AR-only step (used when exactly one token remains): y_1 ~ p(t at n)."""
        cfg, S = self.cfg, self.S
        logits, _ = model.forward(cfg, self.w, self.t[:, None], self.n[:, None],
                                  np.zeros((S, 1)), self.cache)
        P = self._law(logits)[:, 0]
        word = rng.draw_word(self.seed, self.seq_ids, self.n + 1, rng.STREAM_DRAFT, self.it)
        idx, total = rng.sample_icdf(P, word)
        self.forwards += 1
        return idx

    def generate(self, n_new, broken=None):
        """Generate exactly n_new tokens per sequence (all sequences in lock-step).

        Returns (tokens int [S, n_new], per-iteration n_out list, forwards int [S]).
        An iteration whose output overshoots n_new is truncated; when exactly one
        token remains an AR-only step produces it.  Sequences that finish early stop
        stepping.  Tokens per forward of sequence s is n_new / forwards[s].
        """
        S = self.S
        toks = np.full((S, n_new), -1, dtype=np.int64)
        gen = np.zeros(S, dtype=np.int64)
        fwd = np.zeros(S, dtype=np.int64)
        history = []
        while (gen < n_new).any():
            rem = n_new - gen
            active = np.nonzero(rem > 0)[0]
            single = active[rem[active] == 1]
            multi = active[rem[active] >= 2]
            if len(multi):
                sub = self._subdecoder(multi)
                r = sub.step(broken=broken)
                self._absorb(multi, sub)
                history.append(r["n_out"])
                for a, s in enumerate(multi):
                    take = min(int(r["n_out"][a]), int(rem[s]))
                    toks[s, gen[s]: gen[s] + take] = r["out"][a, :take]
                    gen[s] += take
                fwd[multi] += 2
                self.forwards += 2
            if len(single):
                sub = self._subdecoder(single)
                idx = sub.ar_single()
                for a, s in enumerate(single):
                    toks[s, gen[s]] = idx[a]
                    gen[s] += 1
                fwd[single] += 1
                self.forwards += 1
        return toks, history, fwd

    # -- helpers that run a subset of the sequences against views of the cache --
    def _subdecoder(self, rows):
        sub = Decoder.__new__(Decoder)
        sub.cfg, sub.w, sub.seed, sub.top_p = self.cfg, self.w, self.seed, self.top_p
        sub.seq_ids = self.seq_ids[rows]
        sub.cache = {"k": self.cache["k"][:, rows], "v": self.cache["v"][:, rows]}
        sub.n, sub.t, sub.it = self.n[rows].copy(), self.t[rows].copy(), self.it[rows].copy()
        sub.forwards = 0
        return sub

    def _absorb(self, rows, sub):
        self.cache["k"][:, rows] = sub.cache["k"]
        self.cache["v"][:, rows] = sub.cache["v"]
        self.n[rows], self.t[rows], self.it[rows] = sub.n, sub.t, sub.it
