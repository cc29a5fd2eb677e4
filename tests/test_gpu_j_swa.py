"""GPU parity of sliding-window layers against the CPU oracle.  The GPU keeps
each window layer's KV in a ring of W + 16 slots per sequence and writes
every verify row at its true position; the oracle keeps a plain linear cache
and masks keys outside [t - W + 1, t].  The contexts here wrap the rings many
times, and the verify steps mix fully accepted spans, partial rejections and
all-rejected spans past the window -- the cases where a ring that lost
positions to a rejected verify would attend stale keys (TensorSharp page,
sliding-window section).  Every step is checked by the comparison protocol;
spec-on equals spec-off token for token."""
import time

import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import MARGIN, Twin, check_batch_step, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu
TINY = synth.SHAPES["tiny_swa"]


@pytest.fixture(scope="module")
def tiny_weights():
    return synth.weights(TINY, seed=0)


def test_tiny_window_verify_across_ring_wraps(tiny_weights):
    V = TINY["vocab"]
    t = Twin(TINY, tiny_weights, max_ctx=512)
    try:
        prompt = synth.motif_prompt(1, V)
        t.prefill(prompt)
        off, _ = specv.spec_generate(t.ctx, prompt, 300, spec=False)   # the GPU's own greedy stream
        t.prefill(prompt)
        rng = np.random.default_rng(3)
        n = 0
        while len(t.history) - 1 < 260:
            pos = len(t.history) - len(prompt) - 1       # stream index of the next token
            kind = n % 4
            K = [7, 4, 15, 2][n % 4]
            if kind == 0 or kind == 2:                    # drafts from the stream, maybe corrupted
                d = [int(x) for x in off[pos + 1:pos + 1 + K]]
                if kind == 2 and len(d) > 3:
                    d[3] = (d[3] + 1) % V
            else:                                         # random drafts (rejected)
                d = [int(x) for x in rng.integers(0, V, K)]
            t.verify_checked(d)
            n += 1
        log(f"  tiny window 24 / ring 48: {n} verify steps to a {len(t.history) - 1}-token context")
        # rows gate deep past the window
        ctx = t.ctx
        p = specv.spec_cache_len(ctx)
        span = [t.history[-1]] + [int(x) for x in rng.integers(0, V, 11)]
        specv.spec_verify(ctx, span)
        multi = specv.spec_debug_logits(ctx, 12, V)
        specv.spec_rewind(ctx, p)
        rows = []
        for tok in span:
            specv.spec_verify(ctx, [tok])
            rows.append(specv.spec_debug_logits(ctx, 1, V)[0])
        assert np.array_equal(multi, np.stack(rows)), "12-row forward past the window differs from 12 decodes"
        # spec-on == spec-off over 300 tokens, and the oracle's stream up to a near-tie
        fix, s_fix = specv.spec_generate(ctx, prompt, 300, spec=True, fixed_k=4)
        ada, _ = specv.spec_generate(ctx, prompt, 300, spec=True, fixed_k=0, k_cap=7)
        assert np.array_equal(off, fix) and np.array_equal(off, ada) and s_fix["accepted"] > 0
        ref, _ = t.orc.generate(prompt, 300, spec=False)
        diff = [i for i in range(300) if int(off[i]) != ref[i]]
        if diff:
            i = diff[0]
            t.orc.rewind(0)
            _, mg, _ = t.orc.forward(np.array(list(prompt) + ref[:i]), lm_from=len(prompt) + i - 1)
            assert mg[-1] < MARGIN, f"stream diverges at {i} with oracle margin {mg[-1]:.3f}"
        log(f"  spec-on == spec-off over 300 tokens ({s_fix['accepted']} accepted at K=4); "
            f"oracle-identical prefix {diff[0] if diff else 300}/300")
    finally:
        t.close()


def test_tiny_window_batched(tiny_weights):
    """Several sequences, each with its own ring, in one batched step."""
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
            pr = synth.repetition_prompt(70 + sid, V, 30 + 41 * sid)
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(x) for x in pr] + [g]
        for step in range(12):
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, K)
                spans[b] = [h[-1]] + d + [h[-1]] * (K - len(d))
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            worst = check_batch_step(sess, orc, ids, spans, am, acc, hist, V, tag=f"step {step}")
        log(f"  batched window: contexts {[len(hist[s]) - 1 for s in ids]}, worst logit diff {worst:.2e}")
    finally:
        sess.close()
        orc.close()


@pytest.mark.timeout(600)
def test_4b_heads_window_1024_long_contexts():
    """hd = 128, 32q/8kv heads, window 1024 on layers 0 and 2: 8 sequences x 8
    rows at contexts of 2100..4096 (the window's splits start past split 0,
    tile groups, the in-kernel merge) and one sequence at batch 1."""
    shape = synth.SHAPES["attn_4b_swa"]
    V = shape["vocab"]
    n_seq, K = 8, 7
    S = K + 1
    rng = np.random.default_rng(13)
    lens = [int(x) for x in rng.integers(2100, 4097 - 4 * S, n_seq)]
    max_ctx = max(lens) + 4 * S
    w = synth.weights(shape, seed=0)
    sess = specv.Session(shape, specv.tree_weights(w), max_ctx=max_ctx, max_seqs=n_seq, max_rows=n_seq * S,
                         flags=specv.SPEC_FLAG_KEEP_LOGITS)
    orc = O.Oracle(shape, synth.to_numpy(w), max_ctx=max_ctx, n_seq=n_seq)
    try:
        ids = list(range(n_seq))
        hist = {}
        t0 = time.time()
        for sid, L in zip(ids, lens):
            pr = synth.repetition_prompt(900 + sid, V, L)
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(t) for t in pr] + [g]
            log(f"  prefilled seq {sid} ({L} tokens), {time.time() - t0:.0f}s")
        for step in range(2):
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, K)
                spans[b] = [h[-1]] + d + [h[-1]] * (K - len(d))
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            worst = check_batch_step(sess, orc, ids, spans, am, acc, hist, V, tag=f"step {step}")
            log(f"  step {step}: accepted {acc.tolist()}, worst logit diff {worst:.2e}")
        sid = 0                                          # batch 1 on the same state
        for K1 in (0, 7, 15):
            d = [int(x) for x in rng.integers(0, V, K1)]
            span = np.array([[hist[sid][-1]] + d], np.int32)
            am, acc = specv.spec_verify_batch(sess.ctx, [sid], span)
            check_batch_step(sess, orc, [sid], span, am, acc, hist, V, tag=f"batch 1 K={K1}")
    finally:
        sess.close()
        orc.close()
