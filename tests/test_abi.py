"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its host-only calls (buffer sizing, byte accounting) behave.
No GPU compute is issued here."""
import re

import numpy as np
import pytest

from draft_verify_amd import specv, synth


def _declared():
    src = open(specv.HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 25
    lib = specv.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_buffer_sizes_qwen3_4b():
    sh = synth.SHAPES["qwen3_4b"]
    d = specv.make_desc(sh, max_ctx=1024, max_rows=16)
    s = specv.spec_query_buffers(d)
    H, F, V, L = sh["hidden"], sh["ffn"], sh["vocab"], sh["n_layers"]
    per_layer = (6144 * H + H * 4096 + 2 * F * H + H * F) * 2
    assert per_layer == 201_850_880
    mats = L * per_layer + 2 * V * H * 2
    assert mats <= s.weights_bytes <= mats + 64 * 1024 * 1024
    # fp16 K and V, 16-token blocks covering 1024 tokens
    assert s.kv_bytes >= L * 2 * 64 * 8 * 16 * 128 * 2


@pytest.mark.parametrize("bad", [dict(head_dim=48), dict(hidden=100), dict(n_kv=3)])
def test_unsupported_shapes_are_rejected(bad):
    sh = dict(synth.SHAPES["tiny"], **bad)
    d = specv.make_desc(sh, max_ctx=64)
    with pytest.raises(specv.SpecError) as e:
        specv.spec_query_buffers(d)
    assert e.value.code == specv.SPEC_EINVAL


def test_int4_format_is_refused_by_this_build():
    d = specv.make_desc(synth.SHAPES["tiny"], max_ctx=64, weight_format=specv.SPEC_WFMT_INT4G128)
    with pytest.raises(specv.SpecError):
        specv.spec_query_buffers(d)


def test_op_bytes_match_the_4b_stream():
    sh = synth.SHAPES["qwen3_4b"]
    d = specv.make_desc(sh, max_ctx=1024)
    per_fwd = sum(specv.spec_op_bytes(d, op, 1, 848) for op in ("qkv", "o", "gateup", "down")) * 36
    per_fwd += specv.spec_op_bytes(d, "lm", 1, 848)
    kv = specv.spec_op_bytes(d, "attn", 1, 848) * 36
    weights = per_fwd - 36 * 1 * 8 * 128 * 2 * 2
    assert abs(weights - 8_044_544_000) < 1
    assert abs(kv - (848 + 1) * 147_456) < 1


def test_create_without_buffers_fails_cleanly():
    d = specv.make_desc(synth.SHAPES["tiny"], max_ctx=64)
    bufs = specv.spec_device_buffers()
    with pytest.raises(specv.SpecError) as e:
        specv.spec_create(d, bufs, 0)
    assert e.value.code in (specv.SPEC_ECAPACITY, specv.SPEC_EINVAL)
