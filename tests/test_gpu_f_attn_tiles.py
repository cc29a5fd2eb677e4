"""GPU parity of the attention paths a batched step takes when its
(sequence, kv head, split) workgroups fill the chip: each workgroup runs all
query tiles of its sequence on one K/V load, and the splits are merged
either by the last split of the tile group (contexts of at most 8 splits of
256 keys) or by the merge kernel (longer).  A decoder with four query heads
per kv head (hidden 64, 8q/2kv heads of 16) gives two 16-column query tiles
per sequence at 8-row spans; 16 sequences of ~2000 or ~2300 tokens reach
both paths.  Every sequence is checked against the CPU oracle by the
comparison protocol, over two verify steps."""
import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import LOGIT_TOL, MARGIN, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu
SHAPE = synth.SHAPES["tiny_g4"]
V = SHAPE["vocab"]
N_SEQ, K = 16, 7


@pytest.fixture(scope="module")
def weights():
    return synth.weights(SHAPE, seed=0)


@pytest.mark.parametrize("lo,hi", [(1700, 2040), (2100, 2400)], ids=["fused_merge", "merge_kernel"])
def test_tile_groups_vs_oracle(weights, lo, hi):
    S = K + 1
    max_ctx = hi + 64
    sess = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=max_ctx, max_seqs=N_SEQ,
                         max_rows=N_SEQ * S, flags=specv.SPEC_FLAG_KEEP_LOGITS)
    orc = O.Oracle(SHAPE, synth.to_numpy(weights), max_ctx=max_ctx, n_seq=N_SEQ)
    try:
        rng = np.random.default_rng(11)
        lens = [int(x) for x in rng.integers(lo, hi + 1 - 2 * S, N_SEQ)]
        ids = list(range(N_SEQ))
        hist = {}
        for sid, L in zip(ids, lens):
            pr = synth.repetition_prompt(500 + sid, V, L)
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(t) for t in pr] + [g]
        log(f"  prefilled {N_SEQ} sequences of {min(lens)}..{max(lens)} tokens")
        # the runtime's choice: all tiles per workgroup once sequences x kv heads
        # x splits reach 256; the last split merges for at most 8 splits
        splits = (max(lens) + S + 255) // 256
        assert N_SEQ * SHAPE["n_kv"] * splits >= 256
        assert (splits <= 8) == (hi <= 2048)
        for step in range(2):
            spans = np.zeros((N_SEQ, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, K)
                d = d + [h[-1]] * (K - len(d))
                spans[b] = [h[-1]] + d
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            lg = specv.spec_debug_logits(sess.ctx, N_SEQ * S, V).reshape(N_SEQ, S, V)
            worst = 0.0
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
                assert specv.spec_cache_len_seq(sess.ctx, sid) == p + m + 1
                commit = [int(x) for x in am[b][: m + 1]]
                hist[sid] += commit
                if m != mo or list(amo[: mo + 1]) != commit:
                    orc.prefill(hist[sid][:-1], sid)
            log(f"  step {step}: accepted {acc.tolist()}, worst logit diff {worst:.2e}")
    finally:
        sess.close()
        orc.close()
