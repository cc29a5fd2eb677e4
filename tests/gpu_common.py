"""Shared helpers of the GPU parity tests: sessions, the oracle twin, and the
comparison protocol.

Protocol (per verify step, teacher forced): the oracle replays the same span
on the same committed prefix and
  1. every row's logits agree within LOGIT_TOL max-abs;
  2. the per-row argmax is equal wherever the oracle's top-2 margin is
     >= MARGIN (elsewhere both tokens are correct readings of a near-tie);
  3. the accept length is equal whenever the rows that decide it (rows
     0..min(m_gpu, m_oracle, K-1)) all have margin >= MARGIN.
After a step whose accept lengths legitimately differ, the oracle is re-synced
to the GPU's committed history.
"""
import sys
import time

import numpy as np

from draft_verify_amd import specv, synth
from oracle import oracle as O

LOGIT_TOL = 2e-2
MARGIN = 0.05


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_prefill(orc, prompt, seq=0, chunk=0):
    """The oracle's prefill of `prompt` on `seq`: one call, or chunk-row
    forwards with a progress line each; returns (g0, margin)."""
    n = len(prompt)
    if chunk <= 0 or chunk >= n:
        return orc.prefill(prompt, seq)
    orc.rewind(0, seq)
    t0 = time.time()
    for off in range(0, n, chunk):
        end = min(n, off + chunk)
        am, mg, _ = orc.forward(prompt[off:end], seq, lm_from=(end - off - 1) if end == n else (end - off))
        log(f"    oracle prefill {end}/{n} rows ({time.time() - t0:.0f}s)")
    return int(am[0]), float(mg[0])


def check_batch_step(sess, orc, ids, spans, am, acc, hist, V, tag=""):
    """The comparison protocol for one batched verify step, per sequence,
    against the oracle replaying each sequence's span on its own prefix;
    commits to `hist` and re-syncs the oracle after a legitimate difference.
    Returns the worst logit difference."""
    n_seq, S = spans.shape
    K = S - 1
    lg = specv.spec_debug_logits(sess.ctx, n_seq * S, V).reshape(n_seq, S, V)
    worst = 0.0
    for b, sid in enumerate(ids):
        p = len(hist[sid]) - 1
        amo, mo, mgo, lgo = orc.verify(spans[b], sid, want_logits=True)
        err = float(np.abs(lg[b] - lgo).max())
        worst = max(worst, err)
        assert err < LOGIT_TOL, f"{tag} seq {sid}: logits differ by {err:.3e}"
        sure = mgo >= MARGIN
        assert np.array_equal(am[b][sure], amo[sure]), f"{tag} seq {sid}: argmax differs on a sure row"
        m = int(acc[b])
        decide = min(m, mo, K - 1)
        if K == 0 or bool(np.all(sure[: decide + 1])):
            assert m == mo, f"{tag} seq {sid}: accept {m} != oracle {mo}"
        assert m == O.accept_greedy(spans[b], am[b]), f"{tag} seq {sid}: device accept != accept_greedy"
        assert 0 <= m <= K
        assert specv.spec_cache_len_seq(sess.ctx, sid) == p + m + 1
        commit = [int(x) for x in am[b][: m + 1]]
        hist[sid] += commit
        if m != mo or list(amo[: mo + 1]) != commit:
            orc.prefill(hist[sid][:-1], sid)  # re-sync to the GPU's stream
    return worst


class Twin:
    """A GPU session and an oracle over the same seeded weights (sequence 0)."""

    def __init__(self, shape, weights, max_ctx, max_seqs=1, max_rows=16, flags=specv.SPEC_FLAG_KEEP_LOGITS,
                 oracle_ctx=None, host_weights=None, orc=None, fmt="bf16"):
        """`orc`: an existing oracle over the same weights to share (not closed here)."""
        self.shape = shape
        self.sess = specv.Session(shape, specv.tree_weights(weights), max_ctx=max_ctx, max_seqs=max_seqs,
                                  max_rows=max_rows, flags=flags, fmt=fmt)
        self.own_orc = orc is None
        if orc is None:
            hw = host_weights if host_weights is not None else synth.to_numpy(weights)
            orc = O.Oracle(shape, hw, max_ctx=oracle_ctx or max_ctx, n_seq=max_seqs)
        self.orc = orc
        self.ctx = self.sess.ctx
        self.history = []
        self.temp, self.seed = 0.0, 0

    def set_sampling(self, temp, seed):
        """Sampled rows on both sides (temp 0: greedy).  With sampling on, the
        per-row "margin" is the oracle's top-2 margin of the sampled scores
        logit / T + g."""
        specv.spec_set_sampling(self.ctx, temp, seed)
        self.temp, self.seed = float(temp), int(seed)

    def prefill(self, prompt, seq=0, chunk=0):
        """Prefill both sides; chunk > 0 runs the oracle's prefill in chunks of
        that many rows with a progress line each (the oracle's rows are
        independent of how they are grouped, so the cache is the same)."""
        g = specv.spec_prefill_seq(self.ctx, seq, prompt)
        if self.temp > 0:
            go, mg = self.orc.prefill(prompt, seq, temp=self.temp, seed=self.seed)
        else:
            go, mg = oracle_prefill(self.orc, prompt, seq, chunk)
        assert g == go or mg < MARGIN, f"prefill token {g} != oracle {go} (margin {mg:.3f})"
        self.history = [int(t) for t in prompt] + [g]
        return g

    def verify_checked(self, drafts):
        """One verify of [last] + drafts on both sides (sequence 0), checked by
        the protocol."""
        seq = 0
        span = [self.history[-1]] + [int(d) for d in drafts]
        K = len(span) - 1
        p = specv.spec_cache_len(self.ctx)
        am, m = specv.spec_verify(self.ctx, span)
        lg = specv.spec_debug_logits(self.ctx, K + 1, self.shape["vocab"])
        amo, mo, mgo, lgo = self.orc.verify(span, seq, want_logits=True, temp=self.temp, seed=self.seed)
        err = float(np.max(np.abs(lg - lgo)))
        assert err < LOGIT_TOL, f"logits differ by {err:.3e} (K={K})"
        sure = mgo >= MARGIN
        assert np.array_equal(am[sure], amo[sure]), \
            f"argmax differs on a sure row: gpu {am.tolist()} oracle {amo.tolist()} margins {mgo.round(3).tolist()}"
        decide = min(m, mo, K - 1) if K > 0 else -1
        if decide < 0 or bool(np.all(sure[: decide + 1])):
            assert m == mo, f"accept length {m} != oracle {mo}"
        # on every step, near-ties included: the device's accept length is
        # accept_greedy of the span against the device's own argmax rows
        assert m == O.accept_greedy(span, am), f"device accept {m} != accept_greedy(span, device argmax)"
        assert 0 <= m <= K
        assert specv.spec_cache_len_seq(self.ctx, seq) == p + m + 1
        commit = [int(x) for x in am[: m + 1]]
        self.history += commit
        if m != mo or list(amo[: mo + 1]) != commit:
            self.orc.prefill(self.history[:-1], seq)  # re-sync to the GPU's stream
        return am, m, err

    def close(self):
        self.sess.close()
        if self.own_orc:
            self.orc.close()
