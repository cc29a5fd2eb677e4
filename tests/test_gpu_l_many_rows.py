"""GPU parity of the many-row GEMM (forwards above 16 rows: the 32x32x16
MFMA kernel on prepared activations, its K slices summed by the gather
kernel, or one slice with the epilogue in the kernel) at the Qwen3-4B head
geometry (hidden 512, 32q/8kv heads of 128, FFN 512, vocab 1024, 2 layers):
the QKV, gate/up and down GEMMs run two K slices, the O GEMM sixteen and
the LM head one.  Row counts 128 (16 x 8, the batched step's), 40 (5 x 8:
an odd number of 16-row chunks) and 18 (3 x 6: a ragged last chunk), at
contexts of 60..400 tokens; and the batched step's whole geometry, 16 x 8
rows over 2100..2400-token contexts (attention workgroups taking both query
tiles of a sequence, nine or ten splits merged by the merge kernel).  Every
sequence is checked against the CPU oracle by the comparison protocol, and
every accept length against the accept rule on the GPU's own argmax."""
import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import LOGIT_TOL, MARGIN, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu
SHAPE = synth.SHAPES["attn_4b"]
V = SHAPE["vocab"]


@pytest.fixture(scope="module")
def weights():
    return synth.weights(SHAPE, seed=3)


@pytest.mark.parametrize("n_seq,S,lo,hi", [(16, 8, 60, 400), (5, 8, 60, 400), (3, 6, 60, 400), (16, 8, 2100, 2400)],
                         ids=["128_rows", "40_rows", "18_rows", "128_rows_merge_kernel"])
def test_many_rows_vs_oracle(weights, n_seq, S, lo, hi):
    K = S - 1
    max_ctx = hi + 64
    sess = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=max_ctx, max_seqs=n_seq,
                         max_rows=n_seq * S, flags=specv.SPEC_FLAG_KEEP_LOGITS)
    orc = O.Oracle(SHAPE, synth.to_numpy(weights), max_ctx=max_ctx, n_seq=n_seq)
    try:
        rng = np.random.default_rng(100 + n_seq)
        lens = [int(x) for x in rng.integers(lo, hi + 1 - 3 * S, n_seq)]
        ids = list(range(n_seq))
        hist = {}
        for sid, L in zip(ids, lens):
            pr = synth.repetition_prompt(900 + sid, V, L)
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(t) for t in pr] + [g]
        log(f"  {n_seq} x {S} rows: prefilled {min(lens)}..{max(lens)} tokens")
        for step in range(3 if hi <= 400 else 2):
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, K)
                d = d + [h[-1]] * (K - len(d))
                spans[b] = [h[-1]] + d
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            lg = specv.spec_debug_logits(sess.ctx, n_seq * S, V).reshape(n_seq, S, V)
            worst = 0.0
            for b, sid in enumerate(ids):
                p = len(hist[sid]) - 1
                m = int(acc[b])
                # the accept stage against the GPU's own argmax, whatever the margins
                assert m == O.accept_greedy(spans[b], am[b]), f"seq {sid} step {step}: accept stage"
                amo, mo, mgo, lgo = orc.verify(spans[b], sid, want_logits=True)
                err = float(np.abs(lg[b] - lgo).max())
                worst = max(worst, err)
                assert err < LOGIT_TOL, f"seq {sid} step {step}: logits differ by {err:.3e}"
                sure = mgo >= MARGIN
                assert np.array_equal(am[b][sure], amo[sure])
                decide = min(m, mo, K - 1)
                if bool(np.all(sure[: decide + 1])):
                    assert m == mo, f"seq {sid} step {step}: accept {m} != oracle {mo}"
                assert specv.spec_cache_len_seq(sess.ctx, sid) == p + m + 1
                commit = [int(x) for x in am[b][: m + 1]]
                hist[sid] += commit
                if m != mo or list(amo[: mo + 1]) != commit:
                    orc.prefill(hist[sid][:-1], sid)
            log(f"  step {step}: accepted {acc.tolist()}, worst logit diff {worst:.2e}")
    finally:
        sess.close()
        orc.close()
