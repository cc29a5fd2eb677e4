"""GPU parity of sampled verification (every row draws its token from
softmax(logit / T) by the Gumbel-max rule with Philox noise keyed by seed,
sequence and position; drafts are accepted while the draw matches), through
the C ABI, against the CPU oracle's own implementation of the same draw:
drawn tokens equal wherever the oracle's top-2 score margin is >= 0.05,
logits within 2e-2, accept lengths equal when the deciding rows are sure and
always equal to the prefix rule over the device's own draws; the sampled
speculative stream equals the sampled plain stream token for token."""
import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import MARGIN, Twin, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,fmt", [("tiny", "bf16"), ("tiny_int4", "int4")])
def test_tiny_sampled_verify_vs_oracle(name, fmt):
    shape = synth.SHAPES[name]
    V = shape["vocab"]
    w = synth.weights(shape, seed=0, fmt=fmt)
    t = Twin(shape, w, max_ctx=512, fmt=fmt)
    try:
        for T, seed in ((0.8, 7), (1.5, 2 ** 40 + 3)):
            t.set_sampling(T, seed)
            prompt = synth.motif_prompt(1, V)
            t.prefill(prompt)
            rng = np.random.default_rng(int(T * 10))
            for K in (0, 3, 7, 15, 1):
                t.verify_checked(rng.integers(0, V, K))
            # planted drafts: the GPU's own sampled plain stream, corrupted at j
            off, _ = specv.spec_generate(t.ctx, prompt, 12, spec=False)
            for j in (0, 2, 5):
                t.prefill(prompt)
                drafts = [int(x) for x in off[1:6]]
                if j < 5:
                    drafts[j] = (drafts[j] + 1) % V
                _, m, _ = t.verify_checked(drafts)
                assert m == j
        # sampled streams: spec-on == spec-off on the GPU; the oracle's stream
        # agrees up to its first near-tie
        t.set_sampling(0.8, 11)
        prompt = synth.motif_prompt(1, V)
        off, _ = specv.spec_generate(t.ctx, prompt, 96, spec=False)
        fix, s_fix = specv.spec_generate(t.ctx, prompt, 96, spec=True, fixed_k=4)
        ada, _ = specv.spec_generate(t.ctx, prompt, 96, spec=True, fixed_k=0, k_cap=7)
        assert np.array_equal(off, fix) and np.array_equal(off, ada)
        ref, _ = t.orc.generate(prompt, 96, spec=False, temp=0.8, seed=11)
        diff = [i for i in range(96) if int(off[i]) != ref[i]]
        if diff:
            i = diff[0]
            t.orc.rewind(0)
            _, _, lg = t.orc.forward(np.array(list(prompt) + ref[:i]), lm_from=len(prompt) + i - 1, want_logits=True)
            _, mg = O.sample_row(lg[-1], 0.8, 11, 0, len(prompt) + i - 1)
            assert mg < MARGIN, f"sampled stream diverges at {i} with score margin {mg:.3f}"
        log(f"  {name} sampled: K=4 {s_fix['forwards']} forwards for 95 tokens ({s_fix['accepted']} accepted); "
            f"oracle-identical prefix {diff[0] if diff else 96}/96")
    finally:
        t.close()


def test_4b_sampled_verify_vs_oracle():
    shape = synth.SHAPES["qwen3_4b"]
    V = shape["vocab"]
    w = synth.weights(shape, seed=0, device="cuda")
    hw = synth.to_numpy(w)
    t = Twin(shape, w, max_ctx=1024, host_weights=hw)
    del w
    try:
        t.set_sampling(1.0, 12345)
        prompt = synth.repetition_prompt(3, V, 256)
        t.prefill(prompt)
        rng = np.random.default_rng(21)
        for K in (0, 7, 15, 3):
            _, m, err = t.verify_checked(rng.integers(0, V, K))
            log(f"  4B sampled K={K:2d}: m={m} max|dlogit|={err:.2e}")
        off, _ = specv.spec_generate(t.ctx, prompt, 40, spec=False)
        ref = np.array(off, np.int32)
        ref[4::4] = (ref[4::4] + 1) % V
        on, st = specv.spec_generate(t.ctx, prompt, 40, spec=True, fixed_k=0, k_cap=7,
                                     draft_source=specv.SPEC_DRAFT_STREAM, ref_stream=ref)
        assert np.array_equal(off, on) and st["accepted"] > 0 and st["accepted"] < st["drafted"]
        log(f"  4B sampled stream: {st['forwards']} forwards, {st['accepted']}/{st['drafted']} accepted")
    finally:
        t.close()


def test_batched_sampled_draws_depend_on_the_sequence():
    """Sampled rows in a batched step: each sequence's draws use its own id in
    the noise counter, checked against the oracle sequence by sequence, and a
    sequence verified alone (same id) draws bit-identically."""
    shape = synth.SHAPES["tiny"]
    V = shape["vocab"]
    w = synth.weights(shape, seed=0)
    flags = specv.SPEC_FLAG_KEEP_LOGITS
    multi = specv.Session(shape, specv.tree_weights(w), max_ctx=256, max_seqs=4, max_rows=32, flags=flags)
    orc = O.Oracle(shape, synth.to_numpy(w), max_ctx=256, n_seq=4)
    T, seed = 0.9, 77
    specv.spec_set_sampling(multi.ctx, T, seed)
    try:
        ids = [0, 1, 2, 3]
        prompt = synth.motif_prompt(1, V)      # the same prompt on every sequence
        last = {}
        for sid in ids:
            last[sid] = specv.spec_prefill_seq(multi.ctx, sid, prompt)
            go, mg = orc.prefill(prompt, sid, temp=T, seed=seed)
            assert last[sid] == go or mg < MARGIN
        spans = np.array([[last[s]] + [int(x) for x in prompt[:7]] for s in ids], np.int32)
        am, acc = specv.spec_verify_batch(multi.ctx, ids, spans)
        lg = specv.spec_debug_logits(multi.ctx, 4 * 8, V).reshape(4, 8, V)
        for b, sid in enumerate(ids):
            amo, mo, mgo, lgo = orc.verify(spans[b], sid, want_logits=True, temp=T, seed=seed)
            assert float(np.abs(lg[b] - lgo).max()) < 2e-2
            sure = mgo >= MARGIN
            assert np.array_equal(am[b][sure], amo[sure])
            assert int(acc[b]) == O.accept_greedy(spans[b], am[b])
        # identical prompts, different sequence ids: the draws differ
        assert len({tuple(int(x) for x in am[b]) for b in range(4)} | {(last[s],) for s in ids}) > 2
    finally:
        multi.close()
        orc.close()
