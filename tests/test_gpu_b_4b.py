"""GPU parity at the Qwen3-4B shape (36 layers, hidden 2560, 32q/8kv heads
of 128, FFN 9728, vocab 151936; seeded N(0, 0.02) bf16 weights), through the
C ABI, against the CPU oracle: short contexts over every span, the rows gate,
and the 848-token context the verify-cost sweep runs at."""
import time

import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import Twin, log

pytestmark = pytest.mark.gpu
SHAPE = synth.SHAPES["qwen3_4b"]


@pytest.fixture(scope="module")
def twin():
    t0 = time.time()
    w = synth.weights(SHAPE, seed=0, device="cuda")
    hw = synth.to_numpy(w)
    t = Twin(SHAPE, w, max_ctx=1024, host_weights=hw)
    del w
    log(f"4B twin ready in {time.time() - t0:.1f}s")
    yield t
    t.close()


def test_short_context_every_span(twin):
    prompt = synth.uniform_prompt(3, SHAPE["vocab"], 48)
    twin.prefill(prompt)
    rng = np.random.default_rng(1)
    worst = 0.0
    for K in (0, 1, 3, 7, 15, 4, 9):
        t = time.time()
        _, m, err = twin.verify_checked(rng.integers(0, SHAPE["vocab"], K))
        worst = max(worst, err)
        log(f"  K={K:2d} m={m} max|dlogit|={err:.2e} ({time.time() - t:.1f}s)")
    assert worst < 2e-2


def test_planted_drafts_accept(twin):
    """Drafts = the GPU's own greedy continuation: all K accepted; corrupted at
    j: exactly j accepted.  Checked against the oracle by the protocol."""
    prompt = synth.uniform_prompt(4, SHAPE["vocab"], 40)
    stream, _ = specv.spec_generate(twin.ctx, prompt, 10, spec=False)
    for j in (7, 0, 3):
        twin.prefill(prompt)
        drafts = [int(x) for x in stream[1:8]]
        if j < 7:
            drafts[j] = (drafts[j] + 1) % SHAPE["vocab"]
        _, m, err = twin.verify_checked(drafts)
        assert m == j
        log(f"  planted mismatch at {j}: accepted {m}, max|dlogit|={err:.2e}")


@pytest.mark.parametrize("S", [5, 8, 9, 12, 16])
def test_rows_gate_bit_exact(twin, S):
    """One S-row forward == S one-row decodes, bit for bit, across the row
    counts where the O and down projections change kernels (one-pass below
    nine rows, split-K with the same K parts above)."""
    prompt = synth.uniform_prompt(5, SHAPE["vocab"], 33)
    g = specv.spec_prefill(twin.ctx, prompt)
    p = specv.spec_cache_len(twin.ctx)
    span = [g] + [int(t) for t in synth.uniform_prompt(6, SHAPE["vocab"], S - 1)]
    specv.spec_verify(twin.ctx, span)
    multi = specv.spec_debug_logits(twin.ctx, S, SHAPE["vocab"])
    specv.spec_rewind(twin.ctx, p)
    rows = []
    for t in span:
        specv.spec_verify(twin.ctx, [t])
        rows.append(specv.spec_debug_logits(twin.ctx, 1, SHAPE["vocab"])[0])
    assert np.array_equal(multi, np.stack(rows)), f"{S}-row forward differs from {S} one-row decodes"


def test_spec_on_equals_off_repetition_prompt(twin):
    prompt = synth.repetition_prompt(3, SHAPE["vocab"], 512)
    off, s_off = specv.spec_generate(twin.ctx, prompt, 48, spec=False)
    on, s_on = specv.spec_generate(twin.ctx, prompt, 48, spec=True, fixed_k=0, k_cap=7)
    assert np.array_equal(off, on)
    assert s_on["forwards"] <= s_off["forwards"]
    log(f"  48 tokens: spec-off {s_off['forwards']} forwards, adaptive {s_on['forwards']} "
        f"({s_on['drafted']} drafted)")


def test_spec_on_equals_off_with_accepts_and_rejections(twin):
    """Drafts that are mostly right and sometimes wrong: the spec-off stream
    with every fifth token changed, fed as drafts at adaptive K.  Full
    accepts, partial accepts and rejections all occur, and the committed
    stream still equals the spec-off stream token for token."""
    prompt = synth.repetition_prompt(3, SHAPE["vocab"], 512)
    off, _ = specv.spec_generate(twin.ctx, prompt, 64, spec=False)
    ref = np.array(off, np.int32)
    ref[5::5] = (ref[5::5] + 1) % SHAPE["vocab"]
    on, st = specv.spec_generate(twin.ctx, prompt, 64, spec=True, fixed_k=0, k_cap=7,
                                 draft_source=specv.SPEC_DRAFT_STREAM, ref_stream=ref)
    assert np.array_equal(off, on)
    assert st["drafted"] > 0 and 0 < st["accepted"] < st["drafted"]
    assert st["accept_hist"][0] > 0 and sum(st["accept_hist"][1:]) > 0
    log(f"  64 tokens, corrupted-stream drafts: {st['forwards']} forwards, {st['drafted']} drafted, "
        f"{st['accepted']} accepted, accept histogram {st['accept_hist'][:8]}")


def test_full_848_context(twin):
    """The verify-cost sweep's context: 848 uniform tokens, then spans of 1,
    8 and 16 rows, checked against the oracle."""
    t = time.time()
    twin.prefill(synth.uniform_prompt(2, SHAPE["vocab"], 848))
    log(f"  848-token prefill on both sides: {time.time() - t:.1f}s")
    rng = np.random.default_rng(6)
    for K in (0, 7, 15):
        _, m, err = twin.verify_checked(rng.integers(0, SHAPE["vocab"], K))
        log(f"  ctx 848 K={K}: m={m} max|dlogit|={err:.2e}")
