"""GPU parity of attention at head dim 128 on the long-context paths the
benchmarks take, against the CPU oracle:

  * the Qwen3-4B attention geometry (32q/8kv heads of 128) with 16 sequences
    x 8 rows and contexts of 2100..4096 tokens: every workgroup takes all
    query tiles of its sequence on one K/V load (16 x 8 x splits >= 256), and
    the 9..17 splits of 256 keys are merged by the merge kernel;
  * the 32B-class attention geometry (64q/8kv heads of 128) with int4
    group-128 weights at batch 1: a 3000-token context (12 splits, one query
    tile per workgroup, merge kernel) and an 8192-token context (33 splits,
    so three rounds of split loads in the merge; tile groups), spans of 1, 4,
    8 and 16 rows.

Both models keep the real head layout on a narrow trunk (hidden 512, FFN 512,
vocab 1024, 2 layers): the attention kernels depend on the head geometry,
the context and the row count, not on the hidden width, and a narrow trunk
lets the oracle prefill thousands of tokens in seconds.  Each verify step is
checked by the comparison protocol (logits within 2e-2, argmax and accept
length on rows with margin >= 0.05, device accept == accept_greedy)."""
import time

import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import MARGIN, Twin, check_batch_step, log, oracle_prefill
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_4b_heads_16x8_rows_long_contexts():
    shape = synth.SHAPES["attn_4b"]
    V = shape["vocab"]
    n_seq, K = 16, 7
    S = K + 1
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(2100, 4097 - 2 * S, n_seq)]
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
            pr = synth.repetition_prompt(700 + sid, V, L)
            g = specv.spec_prefill_seq(sess.ctx, sid, pr)
            go, mg = orc.prefill(pr, sid)
            assert g == go or mg < MARGIN
            hist[sid] = [int(t) for t in pr] + [g]
            log(f"  prefilled seq {sid} ({L} tokens), {time.time() - t0:.0f}s")
        splits = (max(lens) + S + 255) // 256
        assert splits > 8 and n_seq * shape["n_kv"] * splits >= 256  # merge kernel, tile groups
        for step in range(2):
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, K)
                spans[b] = [h[-1]] + d + [h[-1]] * (K - len(d))
            am, acc = specv.spec_verify_batch(sess.ctx, ids, spans)
            worst = check_batch_step(sess, orc, ids, spans, am, acc, hist, V, tag=f"step {step}")
            log(f"  step {step}: accepted {acc.tolist()}, worst logit diff {worst:.2e}")
    finally:
        sess.close()
        orc.close()


@pytest.mark.timeout(600)
def test_32b_heads_int4_batch1_long_contexts():
    shape = synth.SHAPES["attn_32b"]
    V = shape["vocab"]
    ctxs = {0: 3000, 1: 8192}
    max_ctx = 8192 + 64
    w = synth.weights(shape, seed=0, fmt="int4")
    t = Twin(shape, w, max_ctx=max_ctx, max_seqs=2, fmt="int4")
    try:
        sess_ctx, orc = t.ctx, t.orc
        for sid, L in ctxs.items():
            pr = synth.uniform_prompt(50 + sid, V, L)
            t0 = time.time()
            g = specv.spec_prefill_seq(sess_ctx, sid, pr)
            go, mg = oracle_prefill(orc, pr, sid, chunk=1024)
            assert g == go or mg < MARGIN
            log(f"  prefilled seq {sid} ({L} tokens) in {time.time() - t0:.0f}s")
            hist = {sid: [int(x) for x in pr] + [g]}
            rng = np.random.default_rng(20 + sid)
            worst = 0.0
            for K in (0, 3, 7, 15):
                span = np.array([[hist[sid][-1]] + [int(x) for x in rng.integers(0, V, K)]], np.int32)
                am, acc = specv.spec_verify_batch(sess_ctx, [sid], span)
                worst = max(worst, check_batch_step(t.sess, orc, [sid], span, am, acc, hist, V,
                                                    tag=f"ctx {L} K={K}"))
            log(f"  ctx {L}: spans 1/4/8/16 rows, worst logit diff {worst:.2e}")
    finally:
        t.close()


@pytest.mark.parametrize("S", [4, 8, 16])
def test_32b_heads_rows_gate_8192_context(S):
    """Rows gate where the attention takes its query tiles in groups: near an
    8192-token context the 32 splits x 8 kv heads fill the chip, so a span of
    8 or 16 rows (4 or 8 query tiles) runs two tiles per pass in each
    workgroup (4 rows: one tile per workgroup) while one-row decodes run one
    tile per workgroup; the S-row forward still equals S one-row decodes bit
    for bit (every column's arithmetic is the same)."""
    shape = synth.SHAPES["attn_32b"]
    V = shape["vocab"]
    w = synth.weights(shape, seed=0, fmt="int4")
    sess = specv.Session(shape, specv.tree_weights(w), max_ctx=8192 + 64, flags=specv.SPEC_FLAG_KEEP_LOGITS,
                         fmt="int4")
    try:
        g = specv.spec_prefill(sess.ctx, synth.uniform_prompt(61, V, 8192 - 16))
        p = specv.spec_cache_len(sess.ctx)
        span = [g] + [int(t) for t in synth.uniform_prompt(62, V, S - 1)]
        specv.spec_verify(sess.ctx, span)
        multi = specv.spec_debug_logits(sess.ctx, S, V)
        specv.spec_rewind(sess.ctx, p)
        rows = []
        for t in span:
            specv.spec_verify(sess.ctx, [t])
            rows.append(specv.spec_debug_logits(sess.ctx, 1, V)[0])
        assert np.array_equal(multi, np.stack(rows)), f"{S}-row forward differs from {S} one-row decodes"
        log(f"  8176-token context, {S} rows: bit-equal to one-row decodes")
    finally:
        sess.close()
