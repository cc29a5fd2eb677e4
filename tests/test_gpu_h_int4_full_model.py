"""GPU parity of the whole 32B-class int4 model (64 layers, hidden 5120,
64q/8kv heads of 128, FFN 25600, vocab 151936; group-128 int4 weights with
bf16 scales, seeded) against the CPU oracle's exact dequantised matvec: a
256-token context, then verify spans of 1, 4, 5, 8 and 16 rows, each checked
by the comparison protocol.  This is the precision check of the deepest
model: the error the GPU path (fp16 hi + lo activations into the MFMA on
exact integer weights, fp32 group scaling, fp16 KV) accumulates over 64
layers must stay within the 2e-2 logit bound."""
import time

import numpy as np
import pytest

from draft_verify_amd import synth
from gpu_common import LOGIT_TOL, Twin, log

pytestmark = pytest.mark.gpu
BIG = synth.SHAPES["dense_32b"]


@pytest.mark.timeout(900)
def test_32b_int4_whole_model_vs_oracle():
    t0 = time.time()
    w = synth.weights(BIG, seed=0, fmt="int4", device="cuda")
    hw = synth.to_numpy(w)
    t = Twin(BIG, w, max_ctx=320, host_weights=hw, fmt="int4")
    del w
    log(f"32B int4 twin ready in {time.time() - t0:.0f}s")
    try:
        t.prefill(synth.uniform_prompt(5, BIG["vocab"], 256), chunk=32)
        log(f"  256-token prefill on both sides: {time.time() - t0:.0f}s")
        rng = np.random.default_rng(13)
        worst = 0.0
        for K in (0, 3, 4, 7, 15):
            ts = time.time()
            _, m, err = t.verify_checked(rng.integers(0, BIG["vocab"], K))
            worst = max(worst, err)
            log(f"  S={K + 1:2d}: m={m} max|dlogit|={err:.2e} ({time.time() - ts:.0f}s)")
        assert worst < LOGIT_TOL
    finally:
        t.close()
