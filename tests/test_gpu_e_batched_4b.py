"""GPU parity of the paged batched verify at the Qwen3-4B shape (36 layers,
hidden 2560, 32q/8kv heads of 128, FFN 9728, vocab 151936) on the reduced
set: 4 sequences with repetition-heavy prompts of 300..700 tokens, fixed
K = 7 n-gram drafts (short drafts padded with the last history token), so
every forward has 4 x 8 = 32 rows.  Each sequence is teacher-forced against
the CPU oracle by the comparison protocol, step by step."""
import time

import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import LOGIT_TOL, MARGIN, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu
SHAPE = synth.SHAPES["qwen3_4b"]
V = SHAPE["vocab"]


def test_batched_4b_reduced_set_vs_oracle():
    n_seq, K, steps = 4, 7, 3
    S = K + 1
    t0 = time.time()
    w = synth.weights(SHAPE, seed=0, device="cuda")
    hw = synth.to_numpy(w)
    sess = specv.Session(SHAPE, specv.tree_weights(w), max_ctx=1024, max_seqs=n_seq, max_rows=n_seq * S,
                         flags=specv.SPEC_FLAG_KEEP_LOGITS)
    del w
    orc = O.Oracle(SHAPE, hw, max_ctx=1024, n_seq=n_seq)
    log(f"4B batched twin ready in {time.time() - t0:.1f}s")
    try:
        rng = np.random.default_rng(4)
        lens = [int(x) for x in rng.integers(300, 701, n_seq)]
        prompts = [synth.repetition_prompt(4000 + i, V, L) for i, L in enumerate(lens)]
        ids = list(range(n_seq))
        hist = {}
        for sid, pr in zip(ids, prompts):
            t = time.time()
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(x) for x in pr] + [g]
            log(f"  prefill seq {sid} ({len(pr)} tokens) {time.time() - t:.1f}s")
        worst = 0.0
        for step in range(steps):
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, K)
                d = d + [h[-1]] * (K - len(d))
                spans[b] = [h[-1]] + d
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            lg = specv.spec_debug_logits(sess.ctx, n_seq * S, V).reshape(n_seq, S, V)
            for b, sid in enumerate(ids):
                p = len(hist[sid]) - 1
                amo, mo, mgo, lgo = orc.verify(spans[b], sid, want_logits=True)
                err = float(np.abs(lg[b] - lgo).max())
                worst = max(worst, err)
                assert err < LOGIT_TOL, f"seq {sid} step {step}: logits differ by {err:.3e}"
                sure = mgo >= MARGIN
                assert np.array_equal(am[b][sure], amo[sure])
                m = int(acc[b])
                decide = min(m, mo, K - 1)
                if bool(np.all(sure[: decide + 1])):
                    assert m == mo, f"seq {sid} step {step}: accept {m} != oracle {mo}"
                assert 0 <= m <= K
                assert specv.spec_cache_len_seq(sess.ctx, sid) == p + m + 1
                commit = [int(x) for x in am[b][: m + 1]]
                hist[sid] += commit
                if m != mo or list(amo[: mo + 1]) != commit:
                    orc.prefill(hist[sid][:-1], sid)  # re-sync to the GPU's stream
            log(f"  step {step}: accepted {acc.tolist()}, worst logit diff so far {worst:.2e}")
    finally:
        sess.close()
        orc.close()
