"""GPU parity on the tiny decoder (2 layers, hidden 64, 4q/2kv heads of 16,
FFN 128, vocab 256; prompt = an 8-token motif repeated 4 times; n-gram K=4;
64 greedy tokens), through the C ABI, against the CPU oracle."""
import numpy as np
import pytest

from draft_verify_amd import specv, synth
from gpu_common import MARGIN, Twin, log

pytestmark = pytest.mark.gpu
SHAPE = synth.SHAPES["tiny"]


@pytest.fixture(scope="module")
def weights():
    return synth.weights(SHAPE, seed=0)


PATHS = {"graph": specv.SPEC_FLAG_KEEP_LOGITS,
         "eager": specv.SPEC_FLAG_KEEP_LOGITS | specv.SPEC_FLAG_NO_GRAPH}


@pytest.fixture(params=list(PATHS))
def twin(weights, request):
    t = Twin(SHAPE, weights, max_ctx=256, flags=PATHS[request.param])
    yield t
    t.close()


def test_prefill_and_verify_every_span(twin):
    prompt = synth.motif_prompt(1, SHAPE["vocab"])
    twin.prefill(prompt)
    rng = np.random.default_rng(0)
    worst = 0.0
    for K in list(range(16)) + [15, 0, 7]:
        drafts = rng.integers(0, SHAPE["vocab"], K)
        _, _, err = twin.verify_checked(drafts)
        worst = max(worst, err)
    log(f"tiny: worst logit diff {worst:.2e} over spans 1..16")


def test_planted_drafts_accept_exactly(twin):
    """Drafts from the GPU's own greedy stream, corrupted at index j, accept j."""
    prompt = synth.motif_prompt(1, SHAPE["vocab"])
    stream, _ = specv.spec_generate(twin.ctx, prompt, 12, spec=False)
    K = 8
    for j in range(K + 1):
        g = specv.spec_prefill(twin.ctx, prompt)
        assert g == stream[0]
        drafts = [int(t) for t in stream[1:K + 1]]
        if j < K:
            drafts[j] = (drafts[j] + 1) % SHAPE["vocab"]
        am, m = specv.spec_verify(twin.ctx, [g] + drafts)
        assert m == j
        assert list(am[: m + 1]) == [int(t) for t in stream[1:m + 2]]
        assert specv.spec_cache_len(twin.ctx) == len(prompt) + m + 1
    st = specv.spec_get_stats(twin.ctx)
    assert st["forwards_by_span"][K + 1] >= K + 1 and st["forward_ms_by_span"][K + 1] > 0.0


def test_rows_gate_bit_exact(twin):
    """One S-row forward gives bit-identical logits to S one-row decodes."""
    prompt = synth.motif_prompt(1, SHAPE["vocab"])
    g = specv.spec_prefill(twin.ctx, prompt)
    p = specv.spec_cache_len(twin.ctx)
    span = [g] + [int(t) for t in synth.uniform_prompt(5, SHAPE["vocab"], 15)]
    for S in (2, 5, 8, 16):
        specv.spec_verify(twin.ctx, span[:S])
        multi = specv.spec_debug_logits(twin.ctx, S, SHAPE["vocab"])
        specv.spec_rewind(twin.ctx, p)
        rows = []
        for i in range(S):
            specv.spec_verify(twin.ctx, [span[i]])
            rows.append(specv.spec_debug_logits(twin.ctx, 1, SHAPE["vocab"])[0])
        specv.spec_rewind(twin.ctx, p)
        assert np.array_equal(multi, np.stack(rows)), f"rows gate failed at S={S}"


def test_spec_on_equals_spec_off_and_oracle(twin):
    prompt = synth.motif_prompt(1, SHAPE["vocab"])
    off, s_off = specv.spec_generate(twin.ctx, prompt, 64, spec=False)
    fix, s_fix = specv.spec_generate(twin.ctx, prompt, 64, spec=True, fixed_k=4)
    ada, s_ada = specv.spec_generate(twin.ctx, prompt, 64, spec=True, fixed_k=0, k_cap=7)
    assert np.array_equal(off, fix) and np.array_equal(off, ada)
    assert s_off["forwards"] == 63 and s_fix["forwards"] < 63 and s_fix["accepted"] > 0
    assert sum(s_fix["accept_hist"][5:]) == 0  # m <= K
    ref, _ = twin.orc.generate(prompt, 64, spec=False)
    # first divergence from the oracle stream (if any) must sit at a near-tie
    diff = [i for i in range(64) if int(off[i]) != ref[i]]
    if diff:
        i = diff[0]
        twin.orc.rewind(0)
        _, mg, _ = twin.orc.forward(np.array(list(prompt) + ref[:i]), lm_from=len(prompt) + i - 1)
        assert mg[-1] < MARGIN, f"stream diverges at {i} with oracle margin {mg[-1]:.3f}"
    log(f"tiny e2e: spec-off {s_off['forwards']} forwards, K=4 {s_fix['forwards']}, adaptive {s_ada['forwards']}; "
        f"oracle-identical prefix {diff[0] if diff else 64}/64")


def test_shape_changes_between_calls(weights):
    """A forward after forwards of other span lengths (short then long, long
    then short) gives bit-identical results to the same forward in a fresh
    context: nothing of one shape leaks into the next."""
    spans = [[7] + list(range(20, 20 + k)) for k in (1, 15, 7, 15, 1, 3)]
    prompt = synth.motif_prompt(1, SHAPE["vocab"])
    flags = specv.SPEC_FLAG_KEEP_LOGITS
    s = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=256, flags=flags)
    seq_res = []
    for sp in spans:
        specv.spec_prefill(s.ctx, prompt)
        am, m = specv.spec_verify(s.ctx, sp)
        seq_res.append((am.tolist(), m, specv.spec_debug_logits(s.ctx, len(sp), SHAPE["vocab"])))
    s.close()
    for sp, (am0, m0, l0) in zip(spans, seq_res):
        f = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=256, flags=flags)
        specv.spec_prefill(f.ctx, prompt)
        am1, m1 = specv.spec_verify(f.ctx, sp)
        l1 = specv.spec_debug_logits(f.ctx, len(sp), SHAPE["vocab"])
        f.close()
        assert am0 == am1.tolist() and m0 == m1 and np.array_equal(l0, l1)


def test_error_codes(weights):
    s = specv.Session(SHAPE, specv.tree_weights(weights), max_ctx=48)
    E = specv.SpecError
    with pytest.raises(E) as e:
        specv.spec_verify(s.ctx, [1, 2])
    assert e.value.code == specv.SPEC_ESTATE          # verify before prefill
    prompt = synth.motif_prompt(1, SHAPE["vocab"])    # 32 tokens
    g = specv.spec_prefill(s.ctx, prompt)
    with pytest.raises(E) as e:
        specv.spec_verify(s.ctx, [g] + [1] * 16)     # K = 16
    assert e.value.code == specv.SPEC_EINVAL
    with pytest.raises(E) as e:
        specv.spec_verify(s.ctx, [g, SHAPE["vocab"]])  # token out of range
    assert e.value.code == specv.SPEC_EINVAL
    with pytest.raises(E) as e:
        specv.spec_rewind(s.ctx, 40)
    assert e.value.code == specv.SPEC_ESTATE
    specv.spec_verify(s.ctx, [g] + [3] * 14)          # 32 + 15 = 47 <= 48
    n = specv.spec_cache_len(s.ctx)
    with pytest.raises(E) as e:
        specv.spec_verify(s.ctx, [g] * (48 - n + 1))  # would pass max_ctx
    assert e.value.code == specv.SPEC_ECAPACITY
    assert specv.spec_cache_len(s.ctx) == n           # refused, nothing changed
    specv.spec_verify(s.ctx, [g])                     # still usable
    s.close()


def test_nan_row_leaves_the_cache_unchanged(weights):
    """A NaN logit row fails the verify with SPEC_ENAN and moves no cache
    length, on the device or the host: with the final norm gain set to NaN,
    the verify is refused, the cache length stays p, and after the gain is
    restored the next verify matches the oracle at that same p.  The same
    holds for a prefill, which leaves the sequence empty."""
    import torch
    t = Twin(SHAPE, weights, max_ctx=256)
    try:
        prompt = synth.motif_prompt(1, SHAPE["vocab"])
        t.prefill(prompt)
        ctx = t.ctx
        p = specv.spec_cache_len(ctx)
        nan = torch.full((SHAPE["hidden"],), float("nan"), dtype=torch.float32, device="cuda")
        one = torch.ones(SHAPE["hidden"], dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        specv.spec_load_norm(ctx, 0, specv.SPEC_NORM_FINAL, nan.data_ptr())
        for K in (0, 3, 7):
            with pytest.raises(specv.SpecError) as e:
                specv.spec_verify(ctx, [t.history[-1]] + [5] * K)
            assert e.value.code == specv.SPEC_ENAN
            assert specv.spec_cache_len(ctx) == p
        specv.spec_load_norm(ctx, 0, specv.SPEC_NORM_FINAL, one.data_ptr())
        rng = np.random.default_rng(3)
        for K in (3, 0, 7):
            t.verify_checked(rng.integers(0, SHAPE["vocab"], K))
        # a prefill that hits NaN leaves the sequence empty and unusable
        specv.spec_load_norm(ctx, 0, specv.SPEC_NORM_FINAL, nan.data_ptr())
        with pytest.raises(specv.SpecError) as e:
            specv.spec_prefill(ctx, prompt)
        assert e.value.code == specv.SPEC_ENAN
        assert specv.spec_cache_len(ctx) == 0
        specv.spec_load_norm(ctx, 0, specv.SPEC_NORM_FINAL, one.data_ptr())
        with pytest.raises(specv.SpecError) as e:
            specv.spec_verify(ctx, [1, 2])
        assert e.value.code == specv.SPEC_ESTATE
        t.prefill(prompt)
        t.verify_checked([3, 4])
    finally:
        t.close()


def test_governed_generation_parks_a_losing_drafter(weights):
    """A governed loop over all-wrong drafts (every draft rejected): whatever
    the timings, the first full probe ends at its fourth zero-accept step and
    parks drafting for 32 steps (later verdicts depend on measured times,
    which at this launch-bound shape are nearly equal for both kinds of
    step).  With the motif prompt's own n-gram drafts the loop drafts and
    accepts.  Either way the committed stream equals the spec-off stream
    token for token."""
    t = Twin(SHAPE, weights, max_ctx=512)
    try:
        prompt = synth.motif_prompt(1, SHAPE["vocab"])
        off, _ = specv.spec_generate(t.ctx, prompt, 200, spec=False)
        g = specv.spec_gen_handle(t.ctx, prompt, 200, spec=True, fixed_k=4, draft_source=specv.SPEC_DRAFT_WRONG,
                                  ref_stream=off, governed=True)
        g.step(1000)
        wrong = g.tokens()
        gs, st = g.governor_stats(), g.stats()
        g.close()
        assert np.array_equal(off, wrong)
        assert gs["losses"] >= 1 and st["plain_steps"] >= 3 + 32 and gs["parked_steps"] >= 32
        assert st["accepted"] == 0
        on, st_on = specv.spec_generate(t.ctx, prompt, 200, spec=True, fixed_k=4, governed=True)
        assert np.array_equal(off, on) and st_on["accepted"] > 0
        log(f"  governed: wrong drafts {st['forwards']} forwards ({st['plain_steps']} plain, governor {gs}); "
            f"n-gram drafts {st_on['forwards']} forwards ({st_on['plain_steps']} plain)")
    finally:
        t.close()
