"""GPU parity of the int4 group-128 path (w = s * q, q in [-8, 7], one bf16
scale per 128 inputs of an output row; dequant fused into the GEMMs), through
the C ABI, against the CPU oracle's exact dequantised matvec:
  * the smallest group-aligned decoder (2 layers, hidden 128, 4q/2kv heads of
    32, FFN 256, vocab 256): every span, the rows gate, spec-on == spec-off;
  * two layers of the 32B-class dense shape (hidden 5120, 64q/8kv heads of
    128, FFN 25600, vocab 151936) -- every GEMM at its full size -- on a
    256-token context;
  * the whole 64-layer 32B-class model at an 8192-token context: properties
    that hold at any size (rows gate, 1..K+1 commits, spec-on == spec-off)."""
import time

import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import MARGIN, Twin, log

pytestmark = pytest.mark.gpu
TINY = synth.SHAPES["tiny_int4"]
BIG = synth.SHAPES["dense_32b"]


@pytest.fixture(scope="module")
def tiny_weights():
    return synth.weights(TINY, seed=0, fmt="int4")


@pytest.fixture()
def tiny(tiny_weights):
    t = Twin(TINY, tiny_weights, max_ctx=256, fmt="int4")
    yield t
    t.close()


def test_tiny_int4_every_span(tiny):
    tiny.prefill(synth.motif_prompt(1, TINY["vocab"]))
    rng = np.random.default_rng(5)
    worst = 0.0
    for K in list(range(16)) + [0, 7]:
        _, _, err = tiny.verify_checked(rng.integers(0, TINY["vocab"], K))
        worst = max(worst, err)
    log(f"tiny int4: worst logit diff {worst:.2e}")


def rows_gate(ctx, span, V):
    """One S-row forward vs S one-row forwards at the same cache: bit-identical
    logits and argmax.  The cache is left at its starting length."""
    p = specv.spec_cache_len(ctx)
    S = len(span)
    am, _ = specv.spec_verify(ctx, span)
    multi = specv.spec_debug_logits(ctx, S, V)
    specv.spec_rewind(ctx, p)
    for i in range(S):
        a1, _ = specv.spec_verify(ctx, [span[i]])
        one = specv.spec_debug_logits(ctx, 1, V)[0]
        assert a1[0] == am[i] and np.array_equal(one, multi[i]), f"row {i} of S={S} differs"
    specv.spec_rewind(ctx, p)


def test_tiny_int4_rows_gate_and_spec_equals_off(tiny):
    """S=q forward == q sequential decodes bit-exactly; greedy spec-on stream
    == spec-off stream."""
    prompt = synth.motif_prompt(2, TINY["vocab"])
    ctx = tiny.ctx
    g = specv.spec_prefill(ctx, prompt)
    span = [g] + [int(x) for x in synth.uniform_prompt(6, TINY["vocab"], 15)]
    for q in (2, 5, 16):
        rows_gate(ctx, span[:q], TINY["vocab"])
    off, _ = specv.spec_generate(ctx, prompt, 64, spec=False)
    on, _ = specv.spec_generate(ctx, prompt, 64, spec=True, fixed_k=4)
    assert np.array_equal(off, on)


def test_32b_dims_two_layers_vs_oracle():
    """Two layers of the 32B-class shape, int4: every GEMM at its full size."""
    shape = synth.shrink(BIG, n_layers=2)
    t0 = time.time()
    w = synth.weights(shape, seed=0, fmt="int4", device="cuda")
    hw = synth.to_numpy(w)
    t = Twin(shape, w, max_ctx=512, host_weights=hw, fmt="int4")
    del w
    log(f"32B-dims int4 twin ready in {time.time() - t0:.1f}s")
    try:
        t.prefill(synth.uniform_prompt(5, shape["vocab"], 256))
        rng = np.random.default_rng(9)
        worst = 0.0
        for K in (0, 3, 7, 15):
            ts = time.time()
            _, m, err = t.verify_checked(rng.integers(0, shape["vocab"], K))
            worst = max(worst, err)
            log(f"  K={K:2d} m={m} max|dlogit|={err:.2e} ({time.time() - ts:.1f}s)")
        assert worst < 2e-2
    finally:
        t.close()


def test_32b_full_model_8192_context_properties():
    """The whole 32B-class int4 model at 8192 tokens of context: one S=8
    forward equals 8 sequential S=1 forwards bit-exactly, every verify commits
    1..K+1 tokens and moves the cache by exactly that, and a greedy spec-on
    stream equals the spec-off stream."""
    t0 = time.time()
    sess = specv.Session(BIG, specv.synth_weights(BIG, seed=0, device="cuda", fmt="int4"), max_ctx=8192 + 320,
                         flags=specv.SPEC_FLAG_KEEP_LOGITS, fmt="int4")
    log(f"32B int4 session ready in {time.time() - t0:.1f}s")
    try:
        ctx, V = sess.ctx, BIG["vocab"]
        prompt = synth.uniform_prompt(5, V, 8192)
        t1 = time.time()
        g = specv.spec_prefill(ctx, prompt)
        log(f"  prefill 8192 in {time.time() - t1:.1f}s")
        span = [g] + [int(x) for x in np.random.default_rng(8).integers(0, V, 7)]
        rows_gate(ctx, span, V)
        assert specv.spec_cache_len(ctx) == 8192
        specv.spec_rewind(ctx, 8192)
        rng = np.random.default_rng(10)
        for K in (0, 3, 7, 15):
            p = specv.spec_cache_len(ctx)
            am, m = specv.spec_verify(ctx, [g] + [int(x) for x in rng.integers(0, V, K)])
            assert 0 <= m <= K and specv.spec_cache_len(ctx) == p + m + 1
            g = int(am[m])
        specv.spec_rewind(ctx, 8192)
        off, _ = specv.spec_generate(ctx, prompt, 32, spec=False)
        on, _ = specv.spec_generate(ctx, prompt, 32, spec=True, fixed_k=7,
                                    draft_source=specv.SPEC_DRAFT_STREAM, ref_stream=off)
        assert np.array_equal(off, on)
    finally:
        sess.close()
