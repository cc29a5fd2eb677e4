"""GPU parity of recurrent (delta-rule) layers against the CPU oracle.  The
GPU keeps one state snapshot per verify row and commits the one after the
last accepted row on the device; the oracle restores the state from before
the verify and runs the accepted rows again (TensorSharp page, recurrent-
trunk section).  The verify steps mix full accepts, partial accepts and
all-rejected spans, so a wrong commit would leave the recurrent state of
rejected rows in the trunk and every later logit would show it.  Checked by
the comparison protocol step by step; the rows gate is bit-exact; spec-on
equals spec-off, greedy and sampled."""
import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import MARGIN, Twin, check_batch_step, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu
TINY = synth.SHAPES["tiny_rec"]


@pytest.fixture(scope="module")
def tiny_weights():
    return synth.weights(TINY, seed=0)


def test_tiny_recurrent_verify_commit(tiny_weights):
    V = TINY["vocab"]
    t = Twin(TINY, tiny_weights, max_ctx=512)
    try:
        prompt = synth.motif_prompt(1, V)
        off, _ = specv.spec_generate(t.ctx, prompt, 200, spec=False)
        t.prefill(prompt)
        rng = np.random.default_rng(8)
        n = 0
        while len(t.history) - 1 < 150:
            pos = len(t.history) - len(prompt) - 1
            kind = n % 4
            K = [6, 3, 15, 5][kind]
            if kind in (0, 2):
                d = [int(x) for x in off[pos + 1:pos + 1 + K]]
                if kind == 2 and len(d) > 4:
                    d[4] = (d[4] + 1) % V
            else:
                d = [int(x) for x in rng.integers(0, V, K)]
            t.verify_checked(d)
            n += 1
        log(f"  tiny recurrent: {n} verify steps to a {len(t.history) - 1}-token context")
        # rows gate: one 12-row forward vs 12 one-row forwards from the same state
        ctx = t.ctx
        hist = list(t.history)
        span = [hist[-1]] + [int(x) for x in rng.integers(0, V, 11)]
        specv.spec_prefill(ctx, hist[:-1])
        specv.spec_verify(ctx, span)
        multi = specv.spec_debug_logits(ctx, 12, V)
        specv.spec_prefill(ctx, hist[:-1])
        rows = []
        for tok in span:
            am, _ = specv.spec_verify(ctx, [tok])
            rows.append(specv.spec_debug_logits(ctx, 1, V)[0])
        assert np.array_equal(multi, np.stack(rows)), "12-row forward differs from 12 decodes"
        # a recurrent model rewinds only to 0
        with pytest.raises(specv.SpecError) as e:
            specv.spec_rewind(ctx, 10)
        assert e.value.code == specv.SPEC_ESTATE
        fix, s_fix = specv.spec_generate(ctx, prompt, 200, spec=True, fixed_k=4)
        ada, _ = specv.spec_generate(ctx, prompt, 200, spec=True, fixed_k=0, k_cap=7)
        assert np.array_equal(off, fix) and np.array_equal(off, ada)
        assert 0 < s_fix["accepted"] < s_fix["drafted"]
        ref, _ = t.orc.generate(prompt, 200, spec=False)
        diff = [i for i in range(200) if int(off[i]) != ref[i]]
        if diff:
            i = diff[0]
            t.orc.prefill(prompt)
            _, mg, _ = t.orc.forward(np.array(ref[:i]), lm_from=i - 1) if i else (None, [0.0], None)
            assert mg[-1] < MARGIN, f"stream diverges at {i} with oracle margin {mg[-1]:.3f}"
        specv.spec_set_sampling(ctx, 0.9, 5)
        soff, _ = specv.spec_generate(ctx, prompt, 120, spec=False)
        son, _ = specv.spec_generate(ctx, prompt, 120, spec=True, fixed_k=4)
        specv.spec_set_sampling(ctx, 0.0, 0)
        assert np.array_equal(soff, son)
        log(f"  spec-on == spec-off over 200 tokens ({s_fix['accepted']}/{s_fix['drafted']} accepted at K=4); "
            f"oracle-identical prefix {diff[0] if diff else 200}/200; sampled streams equal")
    finally:
        t.close()


def test_tiny_recurrent_batched_with_own_draft_counts(tiny_weights):
    """Several sequences, each with its own state and its own number of
    drafts (padding rows run after the real rows and are never committed)."""
    V = TINY["vocab"]
    n_seq, K = 5, 7
    S = K + 1
    sess = specv.Session(TINY, specv.tree_weights(tiny_weights), max_ctx=512, max_seqs=n_seq, max_rows=n_seq * S,
                         flags=specv.SPEC_FLAG_KEEP_LOGITS)
    orc = O.Oracle(TINY, synth.to_numpy(tiny_weights), max_ctx=512, n_seq=n_seq)
    try:
        ids = list(range(n_seq))
        hist = {}
        for sid in ids:
            pr = synth.motif_prompt(80 + sid, V) if sid % 2 else synth.repetition_prompt(80 + sid, V, 40 + 13 * sid)
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(x) for x in pr] + [g]
        rng = np.random.default_rng(4)
        for step in range(10):
            kd = [int(x) for x in rng.integers(0, K + 1, n_seq)]
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, kd[b])
                kd[b] = len(d)
                spans[b] = [h[-1]] + d + [int(x) for x in rng.integers(0, V, K - len(d))]
            am, acc = specv.spec_verify_batch_k(sess.ctx, ids, spans, kd)
            lg = specv.spec_debug_logits(sess.ctx, n_seq * S, V).reshape(n_seq, S, V)
            for b, sid in enumerate(ids):
                k, m = kd[b], int(acc[b])
                real = spans[b][: k + 1]
                amo, mo, mgo, lgo = orc.verify(real, sid, want_logits=True)
                assert float(np.abs(lg[b][: k + 1] - lgo).max()) < 2e-2
                sure = mgo >= MARGIN
                assert np.array_equal(am[b][: k + 1][sure], amo[sure])
                assert m == O.accept_greedy(real, am[b][: k + 1]) and 0 <= m <= k
                hist[sid] += [int(x) for x in am[b][: m + 1]]
                if mo != m or list(amo[: mo + 1]) != list(am[b][: m + 1]):
                    orc.prefill(hist[sid][:-1], sid)
        log(f"  batched recurrent: contexts {[len(hist[s]) - 1 for s in ids]}")
    finally:
        sess.close()
        orc.close()


@pytest.mark.timeout(600)
def test_4b_heads_recurrent_layers():
    """Head dim 128 (a 64 KB state per kv head), 32q/8kv heads, recurrent
    layers 1 and 3: 4 sequences x 8 rows, then batch 1 with 1, 8 and 16 rows."""
    shape = synth.SHAPES["attn_4b_rec"]
    V = shape["vocab"]
    n_seq, K = 4, 7
    S = K + 1
    w = synth.weights(shape, seed=0)
    sess = specv.Session(shape, specv.tree_weights(w), max_ctx=1400, max_seqs=n_seq, max_rows=n_seq * S,
                         flags=specv.SPEC_FLAG_KEEP_LOGITS)
    orc = O.Oracle(shape, synth.to_numpy(w), max_ctx=1400, n_seq=n_seq)
    try:
        ids = list(range(n_seq))
        hist = {}
        rng = np.random.default_rng(14)
        for sid in ids:
            pr = synth.repetition_prompt(950 + sid, V, int(rng.integers(700, 1200)))
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(t) for t in pr] + [g]
        for step in range(4):
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, K)
                spans[b] = [h[-1]] + d + [h[-1]] * (K - len(d))
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            worst = check_batch_step(sess, orc, ids, spans, am, acc, hist, V, tag=f"step {step}")
            log(f"  step {step}: accepted {acc.tolist()}, worst logit diff {worst:.2e}")
        for K1 in (0, 7, 15):
            span = np.array([[hist[0][-1]] + [int(x) for x in rng.integers(0, V, K1)]], np.int32)
            am, acc = specv.spec_verify_batch(sess.ctx, [0], span)
            check_batch_step(sess, orc, [0], span, am, acc, hist, V, tag=f"batch 1 K={K1}")
    finally:
        sess.close()
        orc.close()
