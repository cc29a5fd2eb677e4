"""GPU parity above 16 rows at dims other than the 4B shape's.  int4: every
GEMM runs the int4 split-K kernel (k_gemm<NK, EPI, FMT_INT4>: 128-input
groups per slice, the slices gathered by the last to arrive); bf16 at the
32B-class dims: the many-row GEMM at its other shapes (QKV 10240 x 5120 in
two slices, O 5120 x 8192 and down 5120 x 25600 in four, gate/up 51200 x
5120 and the LM head in one), and the split-K kernel for the 16-row
prefill forwards (no one-pass plan fits these dims):
  * the smallest group-aligned int4 decoder (2 layers, hidden 128, 4q/2kv
    heads of 32, FFN 256, vocab 256) verifying 5 sequences x 8 rows = 40 rows
    per forward, every sequence against the oracle by the comparison
    protocol, every accept length against the accept rule on the GPU's own
    argmax;
  * two layers of the 32B-class shape (every GEMM at its full size), int4
    and bf16, verifying 4 sequences x 8 rows = 32 rows per forward, the same
    way, with random drafts.
(A forward holds at most 16 rows per sequence, so rows above 16 come from
batches of sequences.)"""
import time

import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import LOGIT_TOL, MARGIN, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu
TINY = synth.SHAPES["tiny_int4"]
BIG = synth.SHAPES["dense_32b"]


def batched_vs_oracle(shape, w, hw, n_seq, S, lo, hi, steps, tag, seed, fmt="int4", drafts="ngram"):
    K = S - 1
    V = shape["vocab"]
    sess = specv.Session(shape, specv.tree_weights(w), max_ctx=hi + 64, max_seqs=n_seq, max_rows=n_seq * S,
                         flags=specv.SPEC_FLAG_KEEP_LOGITS, fmt=fmt)
    orc = O.Oracle(shape, hw, max_ctx=hi + 64, n_seq=n_seq)
    try:
        rng = np.random.default_rng(seed)
        lens = [int(x) for x in rng.integers(lo, hi + 1 - steps * S, n_seq)]
        ids = list(range(n_seq))
        hist = {}
        for sid, L in zip(ids, lens):
            pr = synth.repetition_prompt(seed * 100 + sid, V, L)
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(t) for t in pr] + [g]
        for step in range(steps):
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                if drafts == "ngram":
                    d = O.ngram_propose(h, 2, 4, K)
                    d = d + [h[-1]] * (K - len(d))
                else:
                    d = [int(x) for x in rng.integers(0, V, K)]
                spans[b] = [h[-1]] + d
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            lg = specv.spec_debug_logits(sess.ctx, n_seq * S, V).reshape(n_seq, S, V)
            worst = 0.0
            for b, sid in enumerate(ids):
                p = len(hist[sid]) - 1
                m = int(acc[b])
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
            log(f"  {tag} step {step}: accepted {acc.tolist()}, worst logit diff {worst:.2e}")
    finally:
        sess.close()
        orc.close()


def test_tiny_int4_40_rows_vs_oracle():
    w = synth.weights(TINY, seed=2, fmt="int4")
    batched_vs_oracle(TINY, w, synth.to_numpy(w), 5, 8, 40, 300, 3, "int4 tiny 40 rows", 7)


@pytest.mark.parametrize("fmt", ["int4", "bf16"])
def test_32b_dims_32_rows_vs_oracle(fmt):
    shape = synth.shrink(BIG, n_layers=2)
    t0 = time.time()
    w = synth.weights(shape, seed=1, fmt=fmt, device="cuda")
    hw = synth.to_numpy(w)
    log(f"32B-dims {fmt} weights ready in {time.time() - t0:.1f}s")
    batched_vs_oracle(shape, w, hw, 4, 8, 120, 260, 2, f"{fmt} 32B dims 32 rows", 9, fmt=fmt, drafts="random")
