"""Batched verify over the paged KV pool (16-token blocks): several sequences
with different contexts in one forward, each accepting and rewinding on its
own.  Every sequence must match (a) the CPU oracle by the comparison protocol
and (b) bit-exactly the same sequence verified alone in a one-sequence
context, whose blocks are laid out differently (paged == linear, and batch
invariance across forward row counts)."""
import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import LOGIT_TOL, MARGIN, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu
SHAPE = synth.SHAPES["tiny"]
V = SHAPE["vocab"]


@pytest.fixture(scope="module")
def weights():
    return synth.weights(SHAPE, seed=0)


def test_batched_verify_matches_single_and_oracle(weights):
    n_seq, K = 6, 7
    S = K + 1
    flags = specv.SPEC_FLAG_KEEP_LOGITS
    multi = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=512, max_seqs=8, max_rows=64, flags=flags)
    single = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=512, max_seqs=1, max_rows=16, flags=flags)
    orc = O.Oracle(SHAPE, synth.to_numpy(weights), max_ctx=512, n_seq=8)
    rng = np.random.default_rng(4)
    lens = [int(x) for x in rng.integers(17, 300, n_seq)]
    prompts = [synth.repetition_prompt(40 + i, V, n) for i, n in enumerate(lens)]
    ids = [7, 0, 3, 5, 1, 6]
    hist = {}
    # interleave prefills so every sequence owns scattered blocks
    for sid, pr in zip(ids, prompts):
        g = specv.spec_prefill_seq(multi.ctx, sid, pr)
        go, _ = orc.prefill(pr, sid)
        assert g == go
        hist[sid] = [int(t) for t in pr] + [g]
    for step in range(4):
        spans = np.zeros((n_seq, S), np.int32)
        for b, sid in enumerate(ids):
            h = hist[sid]
            d = O.ngram_propose(h, 2, 4, K)
            d = d + [h[-1]] * (K - len(d))          # pad short drafts with the last token
            spans[b] = [h[-1]] + d
        am, acc = specv.spec_verify_batch(multi.ctx, ids, spans)
        lg = specv.spec_debug_logits(multi.ctx, n_seq * S, V).reshape(n_seq, S, V)
        for b, sid in enumerate(ids):
            # (b) alone, in the single-sequence context replaying this sequence's history
            specv.spec_prefill(single.ctx, hist[sid][:-1])
            am1, m1 = specv.spec_verify(single.ctx, spans[b])
            l1 = specv.spec_debug_logits(single.ctx, S, V)
            assert np.array_equal(lg[b], l1), f"seq {sid}: batched logits differ from alone"
            assert list(am[b]) == list(am1) and acc[b] == m1
            # (a) the oracle
            amo, mo, mgo, lgo = orc.verify(spans[b], sid, want_logits=True)
            err = float(np.abs(lg[b] - lgo).max())
            assert err < LOGIT_TOL
            sure = mgo >= MARGIN
            assert np.array_equal(am[b][sure], amo[sure])
            assert specv.spec_cache_len_seq(multi.ctx, sid) == len(hist[sid]) - 1 + acc[b] + 1
            hist[sid] += [int(t) for t in am[b][: acc[b] + 1]]
            if mo != acc[b] or list(amo[: mo + 1]) != list(am[b][: acc[b] + 1]):
                orc.prefill(hist[sid][:-1], sid)
        log(f"  step {step}: accepted {acc.tolist()}")
    # rewind one sequence and release another; the rest are unaffected
    specv.spec_rewind_seq(multi.ctx, ids[0], lens[0])
    specv.spec_release_seq(multi.ctx, ids[1])
    assert specv.spec_cache_len_seq(multi.ctx, ids[1]) == 0
    with pytest.raises(specv.SpecError) as e:
        specv.spec_verify_batch(multi.ctx, [ids[1]], np.zeros((1, 2), np.int32))
    assert e.value.code == specv.SPEC_ESTATE
    with pytest.raises(specv.SpecError) as e:
        specv.spec_verify_batch(multi.ctx, [ids[2], ids[2]], np.zeros((2, 2), np.int32))
    assert e.value.code == specv.SPEC_EINVAL
    multi.close()
    single.close()


def test_pool_exhaustion_is_refused_cleanly(weights):
    # 4 blocks of 16 tokens in total: a 40-token prompt takes 3
    s = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=128, max_seqs=2, max_rows=32, n_blocks=4)
    g = specv.spec_prefill_seq(s.ctx, 0, synth.uniform_prompt(1, V, 40))
    with pytest.raises(specv.SpecError) as e:
        specv.spec_prefill_seq(s.ctx, 1, synth.uniform_prompt(2, V, 40))
    assert e.value.code == specv.SPEC_ECAPACITY
    specv.spec_release_seq(s.ctx, 1)
    am, m = specv.spec_verify(s.ctx, [g, 1, 2, 3])        # sequence 0 still works
    assert 0 <= m <= 3
    s.close()


def test_weight_beyond_fp16_range_is_refused(weights):
    """The GEMMs hold bf16 weights as exact fp16 copies: a matrix with a
    value beyond the fp16 range (65504) is refused at load with SPEC_EINVAL
    instead of turning into an infinity."""
    bad = {**weights, "layers": [dict(layer) for layer in weights["layers"]]}
    wq = bad["layers"][1]["wq"].clone()
    wq[3, 5] = 1.0e6
    bad["layers"][1]["wq"] = wq
    with pytest.raises(specv.SpecError) as e:
        specv.Session(SHAPE, specv.tree_weights(bad), max_ctx=128)
    assert e.value.code == specv.SPEC_EINVAL and "fp16" in str(e.value)


def test_heterogeneous_drafts_per_sequence(weights):
    """spec_verify_batch_k: each sequence brings its own number of drafts
    (0..7) in one padded 8-row step.  Its accept length counts only its own
    drafts, its cache advances by m+1, and its real rows are bit-identical to
    the same sequence verified alone with its own span (the padding rows lie
    after every real row, so no real row attends to them) and agree with the
    oracle replaying the real span."""
    n_seq, K = 6, 7
    S = K + 1
    flags = specv.SPEC_FLAG_KEEP_LOGITS
    multi = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=512, max_seqs=8, max_rows=64, flags=flags)
    single = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=512, max_seqs=1, max_rows=16, flags=flags)
    orc = O.Oracle(SHAPE, synth.to_numpy(weights), max_ctx=512, n_seq=8)
    try:
        ids = [2, 7, 0, 5, 1, 4]
        hist = {}
        for i, sid in enumerate(ids):
            pr = synth.motif_prompt(60 + i, V) if i % 2 else synth.repetition_prompt(60 + i, V, 90 + 17 * i)
            g = specv.spec_prefill_seq(multi.ctx, sid, pr)
            go, _ = orc.prefill(pr, sid)
            assert g == go
            hist[sid] = [int(t) for t in pr] + [g]
        rng = np.random.default_rng(9)
        seen = set()
        for step in range(4):
            kd = [int(x) for x in rng.integers(0, K + 1, n_seq)]
            kd[step % n_seq] = 0                      # always one sequence with no drafts
            spans = np.zeros((n_seq, S), np.int32)
            for b, sid in enumerate(ids):
                h = hist[sid]
                d = O.ngram_propose(h, 2, 4, kd[b])
                d = d + [int(x) for x in rng.integers(0, V, kd[b] - len(d))]
                pad = [int(x) for x in rng.integers(0, V, K - kd[b])]
                spans[b] = [h[-1]] + d + pad
            am, acc = specv.spec_verify_batch_k(multi.ctx, ids, spans, kd)
            lg = specv.spec_debug_logits(multi.ctx, n_seq * S, V).reshape(n_seq, S, V)
            for b, sid in enumerate(ids):
                k, m = kd[b], int(acc[b])
                assert 0 <= m <= k
                seen.add((k == 0, m == k))
                real = spans[b][: k + 1]
                specv.spec_prefill(single.ctx, hist[sid][:-1])
                am1, m1 = specv.spec_verify(single.ctx, real)
                l1 = specv.spec_debug_logits(single.ctx, k + 1, V)
                assert np.array_equal(lg[b][: k + 1], l1), f"seq {sid}: real rows differ from alone"
                assert list(am[b][: k + 1]) == list(am1) and m == m1
                amo, mo, mgo, lgo = orc.verify(real, sid, want_logits=True)
                assert float(np.abs(lg[b][: k + 1] - lgo).max()) < LOGIT_TOL
                sure = mgo >= MARGIN
                assert np.array_equal(am[b][: k + 1][sure], amo[sure])
                assert m == O.accept_greedy(real, am[b][: k + 1])
                assert specv.spec_cache_len_seq(multi.ctx, sid) == len(hist[sid]) - 1 + m + 1
                hist[sid] += [int(t) for t in am[b][: m + 1]]
                if mo != m or list(amo[: mo + 1]) != list(am[b][: m + 1]):
                    orc.prefill(hist[sid][:-1], sid)
            log(f"  step {step}: drafts {kd}, accepted {acc.tolist()}")
        st = specv.spec_get_stats(multi.ctx)
        assert st["forwards_by_span"][S] == 4
        with pytest.raises(specv.SpecError) as e:
            specv.spec_verify_batch_k(multi.ctx, ids[:1], np.zeros((1, S), np.int32), [K + 1])
        assert e.value.code == specv.SPEC_EINVAL
    finally:
        multi.close()
        single.close()
        orc.close()
