"""The library's indexed n-gram proposer and adaptive-K rule (host C++)
against the oracle's brute-force search and the hand-worked golden cases."""
import json
import os

import numpy as np
import pytest

from draft_verify_amd import specv
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_golden_cases():
    g = json.load(open(os.path.join(GOLDEN, "ngram_cases.json")))
    for c in g["cases"]:
        ng = specv.spec_ngram_create(g["n_min"], g["n_max"], 1024)
        specv.spec_ngram_append(ng, c["history"])
        assert specv.spec_ngram_propose(ng, c["k"]) == c["drafts"], c["why"]
        specv.spec_ngram_destroy(ng)


@pytest.mark.parametrize("vocab", [2, 4, 8])
@pytest.mark.parametrize("orders", [(2, 4), (1, 3), (2, 2), (3, 6)])
def test_indexed_equals_brute_force(vocab, orders):
    n_min, n_max = orders
    rng = np.random.default_rng(vocab * 100 + n_min * 10 + n_max)
    for trial in range(20):
        L = int(rng.integers(0, 80))
        hist = rng.integers(0, vocab, L).astype(np.int32)
        ng = specv.spec_ngram_create(n_min, n_max, 4096)
        # incremental appends of random sizes, querying after each
        i = 0
        while i < L:
            step = int(rng.integers(1, 5))
            specv.spec_ngram_append(ng, hist[i:i + step])
            i = min(L, i + step)
            for K in (0, 1, 3, 7):
                want = O.ngram_propose(hist[:i], n_min, n_max, K)
                assert specv.spec_ngram_propose(ng, K) == want
        # truncation rebuilds the index
        cut = int(rng.integers(0, L + 1))
        specv.spec_ngram_truncate(ng, cut)
        assert specv.spec_ngram_len(ng) == cut
        for K in (1, 5):
            assert specv.spec_ngram_propose(ng, K) == O.ngram_propose(hist[:cut], n_min, n_max, K)
        specv.spec_ngram_destroy(ng)


def test_capacity_and_arguments():
    ng = specv.spec_ngram_create(2, 4, 4)
    specv.spec_ngram_append(ng, [1, 2, 3, 4])
    with pytest.raises(specv.SpecError) as e:
        specv.spec_ngram_append(ng, [5])
    assert e.value.code == specv.SPEC_ECAPACITY
    with pytest.raises(specv.SpecError):
        specv.spec_ngram_truncate(ng, 9)
    specv.spec_ngram_destroy(ng)
    with pytest.raises(specv.SpecError):
        specv.spec_ngram_create(3, 2, 10)


def test_adapt_k_golden_and_oracle():
    g = json.load(open(os.path.join(GOLDEN, "adapt_k_trajectory.json")))
    k, got = g["k0"], []
    for d, a in g["rounds"]:
        k = specv.spec_adapt_k(k, d, a, g["cap"])
        got.append(k)
    assert got == g["k_after"]
    for k in range(1, 9):
        for d in range(0, 9):
            for a in range(0, d + 1):
                assert specv.spec_adapt_k(k, d, a, 7) == O.adapt_k(k, d, a, 7)
