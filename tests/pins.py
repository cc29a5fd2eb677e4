"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each pin takes the path of an oracle library, so the same checks run against
the real oracle (tests/test_oracle_pins.py) and against copies built with a
deliberately planted mistake (tests/test_oracle_mutations.py), which shows that
a plausible mistake anywhere in the oracle fails at least one pin.

Kinds of pin used (no page prints a worked numeric example of a forward):
  * library special case: torch fp64 library routines (tests/torch_ref.py);
  * closed forms: RoPE at position 0, relative-position property, a single
    visible key, constant-vector RMSNorm, SiLU limits;
  * invariants the pages fix: one S-row forward equals S sequential one-row
    decodes (coreai-model-zoo dense n-gram note, rows gate); every verify
    commits 1..K+1 tokens and the cache grows by m+1 (pegainfer DFlash page,
    transaction section and draft-seed alignment paragraph); spec-on equals
    spec-off token for token (same page, greedy oracle section); rejected rows
    are never read (coreai note, KV-only rollback paragraph);
  * hand-worked golden cases under tests/golden/.
"""
import json
import os

import numpy as np
import torch

from draft_verify_amd import synth
from oracle import oracle as O
import torch_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _with_gains(w, shape, seed=7):
    """Replace the unit norm gains with seeded non-unit ones so a dropped
    gain is visible."""
    g = torch.Generator().manual_seed(seed)
    H = shape["hidden"]
    for L in w["layers"]:
        L["g_attn"] = 1.0 + 0.1 * torch.randn(H, generator=g)
        L["g_ffn"] = 1.0 + 0.1 * torch.randn(H, generator=g)
    w["g_final"] = 1.0 + 0.1 * torch.randn(H, generator=g)
    return w


WIDE = dict(n_layers=1, hidden=256, n_q=8, n_kv=2, head_dim=128, ffn=512, vocab=512,
            eps=1e-6, rope_theta=1e6)
INT4 = dict(n_layers=2, hidden=256, n_q=8, n_kv=4, head_dim=32, ffn=256, vocab=384,
            eps=1e-6, rope_theta=1e6)


def _model(shape, fmt="bf16", gains=True, seed=0, max_ctx=128, n_seq=1, lib=None):
    w = synth.weights(shape, seed=seed, fmt=fmt)
    if gains:
        w = _with_gains(w, shape)
    return w, O.Oracle(shape, synth.to_numpy(w), max_ctx=max_ctx, n_seq=n_seq, lib_path=lib)


def _torch_vs_oracle(shape, fmt, n_tok, tol, lib):
    w, orc = _model(shape, fmt, lib=lib)
    toks = synth.uniform_prompt(11, shape["vocab"], n_tok)
    _, _, lg = orc.forward(toks, want_logits=True)
    ref = torch_ref.logits(shape, w, toks)
    err = float(np.max(np.abs(lg.astype(np.float64) - ref)))
    assert err < tol, f"oracle vs torch fp64 logits: max |d| = {err:.3e} >= {tol}"
    return err


def pin_torch_tiny(lib=None):
    return _torch_vs_oracle(synth.SHAPES["tiny"], "bf16", 24, 1e-4, lib)


def pin_torch_wide(lib=None):
    return _torch_vs_oracle(WIDE, "bf16", 12, 1e-4, lib)


def pin_torch_int4(lib=None):
    return _torch_vs_oracle(INT4, "int4", 10, 1e-4, lib)


def pin_closed_forms(lib=None):
    L = O.load_lib(lib or O.DEFAULT_LIB)
    rng = np.random.default_rng(3)
    hd, theta = 128, 1e6
    q = rng.standard_normal(hd).astype(np.float32)
    k = rng.standard_normal(hd).astype(np.float32)
    # RoPE at position 0 is the identity
    assert np.array_equal(O.rope(q, 0, theta, L), q), "RoPE(pos=0) is not the identity"
    # a rotation keeps every rotated pair's length
    r = O.rope(q, 37, theta, L)
    half = hd // 2
    n0 = q[:half] ** 2 + q[half:] ** 2
    n1 = r[:half] ** 2 + r[half:] ** 2
    assert np.allclose(n0, n1, rtol=1e-5, atol=1e-6), "RoPE changed a pair's norm"
    # <RoPE(q, m), RoPE(k, n)> depends on m - n only; sign fixed by a known rotation
    d1 = float(np.dot(O.rope(q, 10, theta, L), O.rope(k, 3, theta, L)))
    d2 = float(np.dot(O.rope(q, 107, theta, L), O.rope(k, 100, theta, L)))
    assert abs(d1 - d2) < 2e-3, "RoPE inner product depends on absolute position"
    e = np.zeros(hd, np.float32)
    e[0] = 1.0
    rot = O.rope(e, 1, theta, L)  # frequency 0 pair rotates by exactly 1 rad
    assert abs(rot[0] - np.cos(1.0)) < 1e-6 and abs(rot[half] - np.sin(1.0)) < 1e-6, \
        "RoPE rotates the wrong way or pairs the wrong elements"
    # a single visible key returns its value exactly
    K = rng.standard_normal((4, hd)).astype(np.float32)
    V = rng.standard_normal((4, hd)).astype(np.float32)
    assert np.array_equal(O.attend(q, K, V, 0, L), V[0]), "one visible key must return V[0]"
    # identical value rows: the output is that row whatever the weights
    Vc = np.tile(V[1], (4, 1))
    assert np.allclose(O.attend(q, K, Vc, 3, L), V[1], rtol=1e-6, atol=1e-6)
    # a dominant key takes all the weight; scale 1/sqrt(d) is visible in the weights
    K2 = np.zeros((3, hd), np.float32)
    c = 0.5 * np.sqrt(hd) / float(np.dot(q, q))
    K2[2] = q * np.float32(c)
    o = O.attend(q, K2, V, 2, L)
    s = float(np.dot(q, K2[2].astype(np.float64))) / np.sqrt(hd)   # ~0.5
    w2 = np.exp(s) / (2.0 + np.exp(s))
    expect = (V[0] + V[1]) * (1 - w2) / 2 + V[2] * w2
    assert np.allclose(o, expect, rtol=1e-4, atol=1e-5), "softmax weights or scale wrong"
    # RMSNorm of a constant vector
    x = np.full(64, 3.0, np.float32)
    g = np.linspace(0.5, 1.5, 64).astype(np.float32)
    y = O.rmsnorm(x, g, 1e-6, L)
    assert np.allclose(y, g * 3.0 / np.sqrt(9.0 + 1e-6), rtol=1e-6), "RMSNorm closed form"
    assert O.silu(0.0, L) == 0.0 and abs(O.silu(30.0, L) - 30.0) < 1e-5
    assert abs(O.silu(-1.0, L) - (-1.0 / (1.0 + np.e))) < 1e-7


def pin_argmax(lib=None):
    L = O.load_lib(lib or O.DEFAULT_LIB)
    v = np.array([0.1, 0.7, 0.3, 0.7, -2.0], np.float32)
    a, m = O.argmax(v, L)
    assert a == 1, "ties must go to the lowest index"
    assert m == 0.0
    a, m = O.argmax(np.array([1.0, 3.0, 2.5], np.float32), L)
    assert a == 1 and abs(m - 0.5) < 1e-7
    try:
        O.argmax(np.array([1.0, np.nan], np.float32), L)
    except O.OracleError:
        pass
    else:
        raise AssertionError("NaN row must be an error")


def pin_rows_gate(lib=None):
    """One S-row forward at p > 0 is bit-identical to S one-row decodes."""
    shape = synth.SHAPES["tiny"]
    _, orc = _model(shape, lib=lib)
    prompt = synth.motif_prompt(1, shape["vocab"])
    orc.prefill(prompt)
    p = orc.cache_len()
    span = synth.uniform_prompt(5, shape["vocab"], 7)
    _, _, multi = orc.forward(span, want_logits=True)
    assert orc.cache_len() == p + 7
    orc.rewind(p)
    rows = [orc.forward(span[i:i + 1], want_logits=True)[2][0] for i in range(7)]
    assert np.array_equal(multi, np.stack(rows)), "S-row forward differs from sequential decodes"


def pin_accept_golden(lib=None):
    L = O.load_lib(lib or O.DEFAULT_LIB)
    for c in _golden("accept_cases.json")["cases"]:
        m = O.accept_greedy(c["span"], c["argmax"], L)
        assert m == c["accepted"], f"accept_greedy{c}: got {m}"


def pin_verify_planted(lib=None):
    """Drafts built from the trunk's own greedy continuation, corrupted at
    position j, accept exactly j drafts; the cache grows by m+1."""
    shape = synth.SHAPES["tiny"]
    _, orc = _model(shape, lib=lib)
    prompt = synth.motif_prompt(1, shape["vocab"])
    K = 6
    stream, _ = orc.generate(prompt, K + 2)          # g0, c1, c2, ...
    V = shape["vocab"]
    for j in range(K + 1):
        g0, _ = orc.prefill(prompt)
        assert g0 == stream[0]
        drafts = list(stream[1:K + 1])
        if j < K:
            drafts[j] = (drafts[j] + 1) % V
        p = orc.cache_len()
        am, m, _, _ = orc.verify([g0] + drafts)
        assert m == j, f"planted mismatch at {j}: accepted {m}"
        assert 1 <= m + 1 <= K + 1
        assert list(am[: m + 1]) == list(stream[1: m + 2]), "committed tokens differ from greedy"
        assert orc.cache_len() == p + m + 1, "cache must grow by m+1"


def pin_rewind_stale(lib=None):
    """Garbage verify rows left past the cache length are never read."""
    shape = synth.SHAPES["tiny"]
    _, orc = _model(shape, lib=lib)
    prompt = synth.motif_prompt(1, shape["vocab"])
    g0, _ = orc.prefill(prompt)
    _, _, clean = orc.forward([g0, 3, 4], want_logits=True)
    g0b, _ = orc.prefill(prompt)
    junk = synth.uniform_prompt(9, shape["vocab"], 6)
    orc.verify([g0b] + [int(t) for t in junk])      # rejects most of them
    orc.rewind(len(prompt))
    _, _, after = orc.forward([g0, 3, 4], want_logits=True)
    assert np.array_equal(clean, after), "stale rows leaked into a later forward"


def pin_spec_equals_off(lib=None):
    shape = synth.SHAPES["tiny"]
    _, orc = _model(shape, gains=False, lib=lib)
    prompt = synth.motif_prompt(1, shape["vocab"])
    off, s0 = orc.generate(prompt, 64, spec=False)
    fix, s1 = orc.generate(prompt, 64, spec=True, fixed_k=4)
    ada, s2 = orc.generate(prompt, 64, spec=True)
    assert len(off) == 64 and off == fix == ada, "spec-on stream differs from spec-off"
    assert s0["forwards"] == 63
    assert max(s1["accept_hist"]) <= 4 and s1["forwards"] < 63
    assert s1["accepted"] > 0 and s2["accepted"] > 0


def pin_ngram_golden(lib=None):
    L = O.load_lib(lib or O.DEFAULT_LIB)
    g = _golden("ngram_cases.json")
    for c in g["cases"]:
        d = O.ngram_propose(c["history"], g["n_min"], g["n_max"], c["k"], L)
        assert d == c["drafts"], f"ngram {c['why']}: got {d}, want {c['drafts']}"


def pin_adapt_k_golden(lib=None):
    L = O.load_lib(lib or O.DEFAULT_LIB)
    g = _golden("adapt_k_trajectory.json")
    k, got = g["k0"], []
    for drafted, accepted in g["rounds"]:
        k = O.adapt_k(k, drafted, accepted, g["cap"], L)
        got.append(k)
    assert got == g["k_after"], f"adaptive K trajectory {got}"


def pin_int4_nibbles(lib=None):
    L = O.load_lib(lib or O.DEFAULT_LIB)
    g = _golden("int4_nibbles.json")
    q4 = np.zeros((1, 64), np.uint8)
    for i, b in g["bytes"].items():
        q4[0, int(i)] = b
    sc = np.full((1, 1), g["scale_bits"], np.uint16)
    X = np.eye(128, dtype=np.float32)
    Y = O.matvec({"q4": q4, "scales": sc}, X, L)[:, 0]
    for col, val in g["columns"].items():
        assert Y[int(col)] == val, f"int4 column {col}: {Y[int(col)]} != {val}"


def pin_multiseq(lib=None):
    """Sequences keep separate caches: interleaved work equals separate work."""
    shape = synth.SHAPES["tiny"]
    _, orc = _model(shape, n_seq=2, lib=lib)
    pa = synth.motif_prompt(1, shape["vocab"])
    pb = synth.uniform_prompt(2, shape["vocab"], 20)
    ga, _ = orc.prefill(pa, seq=0)
    aa, _, _, la = orc.verify([ga, 1, 2, 3], seq=0, want_logits=True)
    gb, _ = orc.prefill(pb, seq=1)
    ga2, _ = orc.prefill(pa, seq=0)
    gb2, _ = orc.prefill(pb, seq=1)
    ab, _, _, lb = orc.verify([ga2, 1, 2, 3], seq=0, want_logits=True)
    assert ga == ga2 and gb == gb2 and np.array_equal(la, lb)


def pin_philox_kat(lib=None):
    """The counter-based generator against its published known-answer vectors."""
    L = O.load_lib(lib or O.DEFAULT_LIB)
    for c in _golden("philox_kat.json")["cases"]:
        got = O.philox4x32_10([int(x, 16) for x in c["ctr"]], [int(x, 16) for x in c["key"]], L)
        want = [int(x, 16) for x in c["out"]]
        assert got == want, f"Philox4x32-10 {c['ctr']} / {c['key']}: {[hex(x) for x in got]}"


def pin_uniform_gumbel_closed_forms(lib=None):
    L = O.load_lib(lib or O.DEFAULT_LIB)
    assert O.uniform01(0, L) == 2.0 ** -24 and O.uniform01(0xFFFFFFFF, L) == 1.0 - 2.0 ** -24
    assert O.uniform01(1 << 31, L) == 0.5 + 2.0 ** -24
    assert abs(O.gumbel(float(np.float32(np.exp(-1.0))), L)) < 1e-6  # -log(-log(1/e)) = 0
    u = np.float32(0.9)
    assert abs(O.gumbel(float(u), L) - (-np.log(-np.log(np.float64(u))))) < 1e-6
    assert O.gumbel(0.1, L) < O.gumbel(0.5, L) < O.gumbel(0.9, L)


def pin_gumbel_max_is_softmax(lib=None):
    """Drawing argmax(logit / T + g) over many positions reproduces the
    softmax(logit / T) distribution (the Gumbel-max rule), for two
    temperatures: chi-square over 5 tokens and 30000 draws each."""
    L = O.load_lib(lib or O.DEFAULT_LIB)
    logits = np.array([1.0, 0.5, -0.3, 2.0, 0.0], np.float32)
    n = 30000
    for T, seed in ((0.7, 12345), (1.6, 999)):
        counts = np.zeros(5)
        for t in range(n):
            counts[O.sample_row(logits, T, seed, 0, t, L)[0]] += 1
        p = np.exp(logits.astype(np.float64) / T)
        p /= p.sum()
        chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
        assert chi2 < 25.0, f"T={T}: draws do not follow softmax(logit/T) (chi2 {chi2:.1f}, counts {counts})"


def pin_sampled_low_temperature_is_greedy(lib=None):
    """At a tiny temperature the draw is the argmax wherever the row's top-2
    margin is not itself tiny."""
    shape = synth.SHAPES["tiny"]
    _, orc = _model(shape, lib=lib)
    prompt = synth.motif_prompt(1, shape["vocab"])
    orc.prefill(prompt)
    span = [int(x) for x in synth.uniform_prompt(8, shape["vocab"], 8)]
    p = orc.cache_len()
    am, _, mg, lg = orc.verify(span, want_logits=True)
    orc.rewind(p)
    sm, _, _, lg2 = orc.verify(span, want_logits=True, temp=1e-5, seed=3)
    assert np.array_equal(lg, lg2)
    sure = mg > 1e-3
    assert sure.sum() >= 4 and np.array_equal(am[sure], sm[sure]), "T -> 0 draws must be the argmax"


def pin_sampled_planted_and_spec_equals_off(lib=None):
    """Sampled verification: drafts taken from the sampled plain stream and
    corrupted at j accept exactly j (the cache grows by m + 1), and a sampled
    speculative stream (n-gram drafts, fixed and adaptive K) equals the
    sampled plain stream token for token, because every position's draw
    depends only on (seed, sequence, position)."""
    shape = synth.SHAPES["tiny"]
    V = shape["vocab"]
    _, orc = _model(shape, gains=False, lib=lib)
    prompt = synth.motif_prompt(1, V)
    T, seed = 0.8, 7
    off, _ = orc.generate(prompt, 48, spec=False, temp=T, seed=seed)
    greedy, _ = orc.generate(prompt, 48, spec=False)
    assert off != greedy, "sampling at T = 0.8 should leave the greedy stream"
    fix, s1 = orc.generate(prompt, 48, spec=True, fixed_k=4, temp=T, seed=seed)
    ada, _ = orc.generate(prompt, 48, spec=True, temp=T, seed=seed)
    assert off == fix == ada, "sampled spec-on stream differs from the sampled plain stream"
    other, _ = orc.generate(prompt, 48, spec=False, temp=T, seed=seed + 1)
    assert other != off, "the seed must change the draws"
    K = 5
    for j in range(K + 1):
        g0, _ = orc.prefill(prompt, temp=T, seed=seed)
        assert g0 == off[0]
        drafts = list(off[1:K + 1])
        if j < K:
            drafts[j] = (drafts[j] + 1) % V
        p = orc.cache_len()
        tk, m, _, _ = orc.verify([g0] + drafts, temp=T, seed=seed)
        assert m == j, f"sampled planted mismatch at {j}: accepted {m}"
        assert list(tk[: m + 1]) == list(off[1:m + 2])
        assert orc.cache_len() == p + m + 1


SWA = dict(n_layers=3, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=128, vocab=256,
           eps=1e-6, rope_theta=1e6, swa_window=5, swa_layers=0b101)


def pin_torch_swa(lib=None):
    """Sliding-window layers (0 and 2 of 3, window 5) against torch SDPA with
    a band mask, over 20 positions (the window slides 15 times)."""
    return _torch_vs_oracle(SWA, "bf16", 20, 1e-4, lib)


def pin_swa_window_limits(lib=None):
    """A window covering the whole context is plain causal attention (bit for
    bit); the rows gate and spec-on == spec-off hold past the window."""
    full = dict(SWA, swa_window=64)
    w, orc_w = _model(full, lib=lib)
    plain = {k: v for k, v in full.items() if k not in ("swa_window", "swa_layers")}
    orc_p = O.Oracle(plain, synth.to_numpy(w), max_ctx=128, lib_path=lib)
    toks = synth.uniform_prompt(12, SWA["vocab"], 40)
    _, _, a = orc_w.forward(toks, want_logits=True)
    _, _, b = orc_p.forward(toks, want_logits=True)
    assert np.array_equal(a, b), "a window wider than the context must change nothing"
    shape = synth.SHAPES["tiny_swa"]
    _, orc = _model(shape, lib=lib)
    prompt = synth.motif_prompt(1, shape["vocab"])
    orc.prefill(prompt)
    p = orc.cache_len()
    span = synth.uniform_prompt(5, shape["vocab"], 9)
    _, _, multi = orc.forward(span, want_logits=True)
    orc.rewind(p)
    rows = [orc.forward(span[i:i + 1], want_logits=True)[2][0] for i in range(9)]
    assert np.array_equal(multi, np.stack(rows)), "sliding-window rows gate"
    off, _ = orc.generate(prompt, 48, spec=False)
    on, st = orc.generate(prompt, 48, spec=True, fixed_k=4)
    assert off == on and st["accepted"] > 0, "sliding-window spec-on differs from spec-off"


def pin_delta_rule_closed_forms(lib=None):
    """One write with strength 1 makes the key read back its value exactly
    (the delta rule replaces the key's old association); strength 1/2 reads
    back the mean of the old read and the value; writing the current read is
    a fixed point; reads ignore the query's length."""
    L = O.load_lib(lib or O.DEFAULT_LIB)
    rng = np.random.default_rng(17)
    hd = 16
    S = (0.3 * rng.standard_normal((hd, hd))).astype(np.float32)
    k = rng.standard_normal(hd).astype(np.float32)
    v = rng.standard_normal(hd).astype(np.float32)
    old = O.delta_read(S, k, L)
    S1 = O.delta_write(S, k, v, 1.0, L)
    assert np.allclose(O.delta_read(S1, k, L), v, atol=2e-5), "a full-strength write must store v under k"
    Sh = O.delta_write(S, k, v, 0.5, L)
    assert np.allclose(O.delta_read(Sh, k, L), 0.5 * (old + v), atol=2e-5)
    assert np.allclose(O.delta_write(S, k, old, 0.7, L), S, atol=2e-6), "writing the current read changes S"
    q = rng.standard_normal(hd).astype(np.float32)
    assert np.allclose(O.delta_read(S, q, L), O.delta_read(S, 3.0 * q, L), atol=1e-6)
    # a key orthogonal to k is not disturbed
    k2 = rng.standard_normal(hd).astype(np.float32)
    k2 -= k * (np.dot(k2, k) / np.dot(k, k))
    assert np.allclose(O.delta_read(S1, k2, L), O.delta_read(S, k2, L), atol=2e-5)


def pin_delta_rule_unrolled(lib=None):
    """Twelve writes against the unrolled solution of the recurrence,
    S_T = S_0 A_1..A_T + sum_t beta v_t k_t^T A_(t+1)..A_T with
    A_t = I - beta k_t k_t^T (unit keys), evaluated by torch in fp64."""
    L = O.load_lib(lib or O.DEFAULT_LIB)
    rng = np.random.default_rng(18)
    hd, T, beta = 16, 12, 0.5
    S0 = (0.2 * rng.standard_normal((hd, hd))).astype(np.float32)
    ks = rng.standard_normal((T, hd)).astype(np.float32)
    vs = rng.standard_normal((T, hd)).astype(np.float32)
    S = S0
    for t in range(T):
        S = O.delta_write(S, ks[t], vs[t], beta, L)
    kh = torch.nn.functional.normalize(torch.tensor(ks, dtype=torch.float64), dim=-1)
    I = torch.eye(hd, dtype=torch.float64)
    A = [I - beta * torch.outer(kh[t], kh[t]) for t in range(T)]
    ref = torch.tensor(S0, dtype=torch.float64) @ torch.linalg.multi_dot(A)
    for t in range(T):
        tail = torch.linalg.multi_dot(A[t + 1:]) if t + 2 < T else (A[T - 1] if t + 1 < T else I)
        ref = ref + beta * torch.outer(torch.tensor(vs[t], dtype=torch.float64), kh[t]) @ tail
    assert float(np.abs(S - ref.numpy()).max()) < 2e-5, "delta rule differs from its unrolled solution"


def pin_recurrent_model(lib=None):
    """A decoder with a recurrent middle layer: logits against the torch
    reference; one S-row forward equals S one-row decodes; drafts from the
    greedy stream corrupted at j accept exactly j and the stream continues
    as plain decoding does (the state after row m, not after the rejected
    rows); spec-on equals spec-off, greedy and sampled."""
    shape = synth.SHAPES["tiny_rec"]
    V = shape["vocab"]
    w, orc = _model(shape, lib=lib)
    toks = synth.uniform_prompt(11, V, 20)
    _, _, lg = orc.forward(toks, want_logits=True)
    ref = torch_ref.logits(shape, w, toks)
    assert float(np.max(np.abs(lg.astype(np.float64) - ref))) < 1e-4, "recurrent model vs torch fp64"
    prompt = synth.motif_prompt(1, V)
    orc.prefill(prompt)
    span = synth.uniform_prompt(5, V, 7)
    _, _, multi = orc.forward(span, want_logits=True)
    orc.prefill(prompt)
    rows = [orc.forward(span[i:i + 1], want_logits=True)[2][0] for i in range(7)]
    assert np.array_equal(multi, np.stack(rows)), "recurrent rows gate"
    stream, _ = orc.generate(prompt, 24)
    K = 6
    for j in range(K + 1):
        g0, _ = orc.prefill(prompt)
        drafts = list(stream[1:K + 1])
        if j < K:
            drafts[j] = (drafts[j] + 1) % V
        am, m, _, _ = orc.verify([g0] + drafts)
        assert m == j
        am2, m2, _, _ = orc.verify([int(am[m])] + list(stream[m + 2:m + 2 + K]))
        assert list(am2[: m2 + 1]) == list(stream[m + 2:m + 3 + m2]), "stream after a partial accept"
    off, _ = orc.generate(prompt, 40)
    on, st = orc.generate(prompt, 40, spec=True, fixed_k=4)
    assert off == on and st["accepted"] > 0 and st["accepted"] < st["drafted"]
    soff, _ = orc.generate(prompt, 40, temp=0.9, seed=5)
    son, _ = orc.generate(prompt, 40, spec=True, fixed_k=4, temp=0.9, seed=5)
    assert soff == son


ALL_PINS = [pin_torch_tiny, pin_torch_wide, pin_torch_int4, pin_closed_forms, pin_argmax,
            pin_rows_gate, pin_accept_golden, pin_verify_planted, pin_rewind_stale,
            pin_spec_equals_off, pin_ngram_golden, pin_adapt_k_golden, pin_int4_nibbles,
            pin_multiseq, pin_philox_kat, pin_uniform_gumbel_closed_forms, pin_gumbel_max_is_softmax,
            pin_sampled_low_temperature_is_greedy, pin_sampled_planted_and_spec_equals_off, pin_torch_swa,
            pin_swa_window_limits, pin_delta_rule_closed_forms, pin_delta_rule_unrolled, pin_recurrent_model]
