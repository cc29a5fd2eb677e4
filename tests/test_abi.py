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


def test_int4_needs_whole_groups():
    """int4 group-128 weights need every GEMM depth to hold whole groups: the
    tiny decoder (hidden 64) is refused, its group-aligned sibling and the
    32B-class shape are accepted."""
    i4 = specv.SPEC_WFMT_INT4G128
    with pytest.raises(specv.SpecError):
        specv.spec_query_buffers(specv.make_desc(synth.SHAPES["tiny"], max_ctx=64, weight_format=i4))
    for name in ("tiny_int4", "dense_32b"):
        specv.spec_query_buffers(specv.make_desc(synth.SHAPES[name], max_ctx=64, weight_format=i4))


def test_int4_op_bytes_match_the_32b_stream():
    """Per forward of the 32B-class int4 model: 0.5 byte per weight plus one
    bf16 scale per 128 weights (16.49 GB), and (ctx + S) x 262,144 B of KV."""
    sh = synth.SHAPES["dense_32b"]
    d = specv.make_desc(sh, max_ctx=8192 + 16, weight_format=specv.SPEC_WFMT_INT4G128)
    L = sh["n_layers"]
    per_fwd = sum(specv.spec_op_bytes(d, op, 1, 8192) for op in ("qkv", "o", "gateup", "down")) * L
    per_fwd += specv.spec_op_bytes(d, "lm", 1, 8192)
    params = L * (10240 * 5120 + 5120 * 8192 + 2 * 25600 * 5120 + 5120 * 25600) + 151936 * 5120
    weights = per_fwd - L * 1 * 8 * 128 * 2 * 2
    assert abs(weights - params * (0.5 + 2 / 128)) < 1
    assert abs(weights - 16.49e9) < 0.01e9
    assert abs(specv.spec_op_bytes(d, "attn", 1, 8192) * L - (8192 + 1) * 262_144) < 1


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


def test_static_create_checks_before_touching_the_device():
    """spec_create_static refuses a workspace (the static scratch is the
    workspace) and a description that needs more workspace than the scratch
    holds, before any device call; the 4B shape at up to 16 rows fits."""
    sh = synth.SHAPES["qwen3_4b"]
    big = specv.make_desc(sh, max_ctx=4200, max_seqs=16, max_rows=128)
    assert specv.spec_query_buffers(big).workspace_bytes > specv.SPEC_STATIC_SCRATCH_BYTES
    with pytest.raises(specv.SpecError) as e:
        specv.spec_create_static(big, specv.spec_device_buffers(), 0)
    assert e.value.code == specv.SPEC_ECAPACITY
    small = specv.make_desc(sh, max_ctx=1024, max_rows=16, flags=specv.SPEC_FLAG_KEEP_LOGITS)
    assert specv.spec_query_buffers(small).workspace_bytes <= specv.SPEC_STATIC_SCRATCH_BYTES
    bufs = specv.spec_device_buffers(None, 0, None, 0, 4096, 4096, None, 0)
    with pytest.raises(specv.SpecError) as e:
        specv.spec_create_static(small, bufs, 0)
    assert e.value.code == specv.SPEC_EINVAL


def test_split_partials_cover_both_row_regimes():
    """A bf16 description with no one-pass plan at its dims (the 32B-class
    shape: hidden 5120, FFN 25600) runs the split-K kernel for forwards of up
    to 16 rows even when max_rows > 16 lets batches use the many-row GEMM: the
    workspace must hold the split-K partials of those forwards (the down
    projection: 25600 / 512 = 50 slices x 5120 columns x 4 bytes per row)
    beside the many-row GEMM's.  Sized for the many-row GEMM alone it held
    2.6 MB at 32 rows and the 16-row forwards wrote past it."""
    sh = synth.shrink(synth.SHAPES["dense_32b"], n_layers=2)
    s16 = specv.spec_query_buffers(specv.make_desc(sh, max_ctx=512, max_rows=16))
    s32 = specv.spec_query_buffers(specv.make_desc(sh, max_ctx=512, max_rows=32))
    down_split_per_row = 50 * 5120 * 4
    assert s16.workspace_bytes >= 16 * down_split_per_row
    assert s32.workspace_bytes >= 32 * down_split_per_row
    assert s32.workspace_bytes >= s16.workspace_bytes
