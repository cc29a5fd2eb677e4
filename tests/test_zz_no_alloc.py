"""spec_create_static: the allocation-free context, whose workspace is the
library's static scratch, against the ordinary context over a torch-allocated
workspace, through the C ABI.  Two contexts in a row on the device (the
second with a smaller description and shorter inputs, reusing the scratch the
first left behind) must each give the ordinary context's results bit for bit:
every row's logits, the argmax rows, the accept lengths and the cache
lengths.  A second live static context on the device and a description too
large for the scratch are refused."""
import numpy as np
import pytest

from draft_verify_amd import specv, synth

pytestmark = pytest.mark.gpu


def run_pair(shape, weights, max_ctx, max_seqs, max_rows, prompt_lens, spans_k, seed):
    flags = specv.SPEC_FLAG_KEEP_LOGITS
    V = shape["vocab"]
    kw = dict(max_ctx=max_ctx, max_seqs=max_seqs, max_rows=max_rows, flags=flags)
    ref = specv.Session(shape, specv.tree_weights(weights), **kw)
    sta = specv.Session(shape, specv.tree_weights(weights), static=True, **kw)
    try:
        assert sta.ws_buf is None
        # a second live static context on this device is refused
        with pytest.raises(specv.SpecError) as e:
            specv.Session(shape, specv.tree_weights(weights), static=True, **kw)
        assert e.value.code == specv.SPEC_ESTATE
        rng = np.random.default_rng(seed)
        ids = list(range(len(prompt_lens)))
        last = {}
        for sid, n in zip(ids, prompt_lens):
            pr = synth.uniform_prompt(seed + sid, V, n)
            g0 = specv.spec_prefill_seq(ref.ctx, sid, pr)
            g1 = specv.spec_prefill_seq(sta.ctx, sid, pr)
            assert g0 == g1
            last[sid] = g0
        for K in spans_k:
            sid = int(rng.integers(0, len(ids)))
            span = [last[sid]] + [int(x) for x in rng.integers(0, V, K)]
            a0, m0 = specv.spec_verify_batch(ref.ctx, [sid], [span])
            l0 = specv.spec_debug_logits(ref.ctx, K + 1, V)
            a1, m1 = specv.spec_verify_batch(sta.ctx, [sid], [span])
            l1 = specv.spec_debug_logits(sta.ctx, K + 1, V)
            assert np.array_equal(a0, a1) and np.array_equal(m0, m1)
            assert np.array_equal(l0, l1), f"K={K}: static context logits differ"
            assert specv.spec_cache_len_seq(ref.ctx, sid) == specv.spec_cache_len_seq(sta.ctx, sid)
            last[sid] = int(a0[0][m0[0]])
        if len(ids) > 1:  # one batched step over every sequence
            K = max_rows // len(ids) - 1
            spans = np.array([[last[s]] + [int(x) for x in rng.integers(0, V, K)] for s in ids], np.int32)
            a0, m0 = specv.spec_verify_batch(ref.ctx, ids, spans)
            l0 = specv.spec_debug_logits(ref.ctx, len(ids) * (K + 1), V)
            a1, m1 = specv.spec_verify_batch(sta.ctx, ids, spans)
            l1 = specv.spec_debug_logits(sta.ctx, len(ids) * (K + 1), V)
            assert np.array_equal(a0, a1) and np.array_equal(m0, m1) and np.array_equal(l0, l1)
    finally:
        sta.close()
        ref.close()


def test_static_context_twice_second_smaller():
    shape = synth.SHAPES["tiny"]
    w = synth.weights(shape, seed=0)
    run_pair(shape, w, max_ctx=256, max_seqs=4, max_rows=64, prompt_lens=[40, 90, 17, 120],
             spans_k=[0, 3, 7, 15, 1], seed=31)
    run_pair(shape, w, max_ctx=64, max_seqs=1, max_rows=8, prompt_lens=[20], spans_k=[2, 0, 7], seed=32)


def test_static_context_4b_shape():
    shape = synth.SHAPES["qwen3_4b"]
    w = synth.weights(shape, seed=0, device="cuda")
    run_pair(shape, w, max_ctx=256, max_seqs=1, max_rows=16, prompt_lens=[64], spans_k=[0, 7, 15, 4], seed=33)


def test_static_context_refuses_what_does_not_fit():
    shape = synth.SHAPES["qwen3_4b"]
    desc = specv.make_desc(shape, max_ctx=4200, max_seqs=16, max_rows=128)
    assert specv.spec_query_buffers(desc).workspace_bytes > specv.SPEC_STATIC_SCRATCH_BYTES
    bufs = specv.spec_device_buffers()
    with pytest.raises(specv.SpecError) as e:
        specv.spec_create_static(desc, bufs, 0)
    assert e.value.code == specv.SPEC_ECAPACITY
    assert "static scratch" in str(e.value)
