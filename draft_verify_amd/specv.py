"""ctypes binding of libspecv (include/specv.h), same names as the C ABI.

Argument marshalling only: every step of the verify transaction runs in the
library's HIP kernels and host C++.  PyTorch provides the device memory (the
weight arena, the KV pool, the workspace), pinned host staging and the HIP
stream; `Session` bundles those allocations.  There is no CPU fallback: if the
library is not built, or no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "specv.h")

SPEC_OK, SPEC_EINVAL, SPEC_ECAPACITY, SPEC_ESTATE, SPEC_EHIP, SPEC_ENAN = 0, -1, -2, -3, -4, -5
SPEC_WFMT_BF16, SPEC_WFMT_INT4G128 = 0, 1
SPEC_FLAG_KEEP_LOGITS, SPEC_FLAG_NO_GRAPH = 1, 2
SPEC_MAX_SPAN, SPEC_MAX_ROWS, SPEC_BLOCK_TOKENS = 16, 128, 16
SPEC_STATIC_SCRATCH_BYTES = 32 << 20
(SPEC_MAT_Q, SPEC_MAT_K, SPEC_MAT_V, SPEC_MAT_O, SPEC_MAT_GATE, SPEC_MAT_UP, SPEC_MAT_DOWN,
 SPEC_MAT_EMB, SPEC_MAT_LM) = range(9)
SPEC_NORM_ATTN, SPEC_NORM_FFN, SPEC_NORM_FINAL = 0, 1, 2
OPS = ("embed", "qkv", "attn", "o", "gateup", "down", "lm")
SPEC_OP_COUNT = len(OPS)
SPEC_DRAFT_NGRAM, SPEC_DRAFT_STREAM, SPEC_DRAFT_WRONG = 0, 1, 2
MAT_IDS = {"wq": SPEC_MAT_Q, "wk": SPEC_MAT_K, "wv": SPEC_MAT_V, "wo": SPEC_MAT_O,
           "wg": SPEC_MAT_GATE, "wu": SPEC_MAT_UP, "wd": SPEC_MAT_DOWN}


class SpecError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class spec_model_desc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("weight_format", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_double), ("max_ctx", C.c_int32), ("max_seqs", C.c_int32),
                ("max_rows", C.c_int32), ("n_blocks", C.c_int32), ("flags", C.c_uint32),
                ("swa_window", C.c_int32), ("reserved", C.c_int32), ("swa_layers", C.c_uint64),
                ("rec_layers", C.c_uint64), ("rec_beta", C.c_float), ("reserved2", C.c_int32)]


class spec_buffer_sizes(C.Structure):
    _fields_ = [("weights_bytes", C.c_size_t), ("kv_bytes", C.c_size_t),
                ("workspace_bytes", C.c_size_t), ("host_bytes", C.c_size_t)]


class spec_device_buffers(C.Structure):
    _fields_ = [("weights", C.c_void_p), ("weights_bytes", C.c_size_t),
                ("kv", C.c_void_p), ("kv_bytes", C.c_size_t),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("host", C.c_void_p), ("host_bytes", C.c_size_t)]


class spec_stats(C.Structure):
    _fields_ = [("forwards", C.c_int64), ("verify_calls", C.c_int64), ("drafted", C.c_int64),
                ("accepted", C.c_int64), ("forwards_by_span", C.c_int64 * (SPEC_MAX_SPAN + 1)),
                ("graphs", C.c_int64), ("forward_ms_by_span", C.c_double * (SPEC_MAX_SPAN + 1))]


class spec_gen_params(C.Structure):
    _fields_ = [("spec", C.c_int32), ("fixed_k", C.c_int32), ("k_cap", C.c_int32),
                ("n_min", C.c_int32), ("n_max", C.c_int32), ("draft_source", C.c_int32),
                ("ref_stream", C.POINTER(C.c_int32)), ("governed", C.c_int32)]


class spec_gen_stats(C.Structure):
    _fields_ = [("forwards", C.c_int64), ("drafted", C.c_int64), ("accepted", C.c_int64),
                ("accept_hist", C.c_int64 * SPEC_MAX_SPAN),
                ("forwards_by_span", C.c_int64 * (SPEC_MAX_SPAN + 1)),
                ("decode_s", C.c_double), ("host_s", C.c_double), ("prefill_s", C.c_double),
                ("plain_steps", C.c_int64)]


class spec_governor_params(C.Structure):
    _fields_ = [("probe_spec", C.c_int32), ("probe_spec_short", C.c_int32), ("probe_plain", C.c_int32),
                ("park_first", C.c_int32), ("park_max", C.c_int32), ("zero_accept_exit", C.c_int32),
                ("hold_window", C.c_int32), ("hold_refresh", C.c_int32)]


class spec_governor_stats(C.Structure):
    _fields_ = [("wins", C.c_int64), ("losses", C.c_int64), ("probes", C.c_int64),
                ("spec_steps", C.c_int64), ("plain_samples", C.c_int64), ("parked_steps", C.c_int64),
                ("state", C.c_int32), ("plain_ms_per_token", C.c_double), ("spec_ms_per_token", C.c_double)]


_lib = None


def lib():
    """Load libspecv.so (after torch, so one HIP runtime serves both)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads torch's HIP runtime first)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(python -m draft_verify_amd.build)")
    L = C.CDLL(LIB_PATH)
    P, I = C.c_void_p, C.c_int
    i32p, f32p, dp = C.POINTER(C.c_int32), C.POINTER(C.c_float), C.POINTER(C.c_double)
    sig = {
        "spec_query_buffers": [C.POINTER(spec_model_desc), C.POINTER(spec_buffer_sizes)],
        "spec_create": [C.POINTER(spec_model_desc), C.POINTER(spec_device_buffers), P, C.POINTER(P)],
        "spec_create_static": [C.POINTER(spec_model_desc), C.POINTER(spec_device_buffers), P, C.POINTER(P)],
        "spec_destroy": [P],
        "spec_load_matrix": [P, I, I, P, P],
        "spec_load_norm": [P, I, I, P],
        "spec_prefill": [P, i32p, I, i32p],
        "spec_verify": [P, i32p, I, i32p, i32p],
        "spec_rewind": [P, I],
        "spec_cache_len": [P, i32p],
        "spec_prefill_seq": [P, I, i32p, I, i32p],
        "spec_verify_batch": [P, I, i32p, i32p, I, i32p, i32p],
        "spec_verify_batch_k": [P, I, i32p, i32p, I, i32p, i32p, i32p],
        "spec_rewind_seq": [P, I, I],
        "spec_cache_len_seq": [P, I, i32p],
        "spec_release_seq": [P, I],
        "spec_debug_logits": [P, f32p, I],
        "spec_set_sampling": [P, C.c_float, C.c_uint64],
        "spec_get_stats": [P, C.POINTER(spec_stats)],
        "spec_time_verify": [P, I, I, i32p, f32p],
        "spec_profile_ops": [P, I, I, i32p, f32p, i32p],
        "spec_op_bytes": [C.POINTER(spec_model_desc), I, I, I, dp],
        "spec_measure_read_bw": [P, C.c_size_t, P, I, P, dp],
        "spec_measure_read_chain": [P, C.c_size_t, I, I, P, P, dp],
        "spec_time_op": [P, I, I, I, f32p],
        "spec_ngram_create": [I, I, I, C.POINTER(P)],
        "spec_ngram_destroy": [P],
        "spec_ngram_append": [P, i32p, I],
        "spec_ngram_truncate": [P, I],
        "spec_ngram_len": [P],
        "spec_ngram_propose": [P, I, i32p],
        "spec_adapt_k": [I, I, I, I],
        "spec_generate": [P, i32p, I, I, C.POINTER(spec_gen_params), i32p, C.POINTER(spec_gen_stats)],
        "spec_gen_begin": [P, i32p, I, I, C.POINTER(spec_gen_params), C.POINTER(P)],
        "spec_gen_step": [P, I, C.POINTER(spec_gen_stats)],
        "spec_gen_tokens": [P, i32p, I],
        "spec_gen_end": [P],
        "spec_gen_governor_stats": [P, C.POINTER(spec_governor_stats)],
        "spec_governor_create": [C.POINTER(spec_governor_params), C.POINTER(P)],
        "spec_governor_destroy": [P],
        "spec_governor_should_draft": [P],
        "spec_governor_record": [P, I, I, I, C.c_double],
        "spec_governor_new_request": [P],
        "spec_governor_get_stats": [P, C.POINTER(spec_governor_stats)],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = C.c_int
    L.spec_last_error.argtypes = [P]
    L.spec_last_error.restype = C.c_char_p
    _lib = L
    return L


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _check(rc, ctx=None):
    if rc < 0:
        msg = lib().spec_last_error(ctx).decode(errors="replace")
        raise SpecError(rc, msg or "libspecv error")
    return rc


def make_desc(shape: dict, max_ctx: int, max_seqs: int = 1, max_rows: int = 16, n_blocks: int = 0,
              flags: int = 0, weight_format: int = SPEC_WFMT_BF16) -> spec_model_desc:
    return spec_model_desc(shape["n_layers"], shape["hidden"], shape["n_q"], shape["n_kv"],
                           shape["head_dim"], shape["ffn"], shape["vocab"], weight_format,
                           shape["eps"], shape["rope_theta"], max_ctx, max_seqs, max_rows,
                           n_blocks, flags, shape.get("swa_window", 0), 0, shape.get("swa_layers", 0),
                           shape.get("rec_layers", 0), shape.get("rec_beta", 0.0), 0)


# --------------------------------------------------------------- ABI calls

def spec_query_buffers(desc):
    s = spec_buffer_sizes()
    _check(lib().spec_query_buffers(C.byref(desc), C.byref(s)))
    return s


def spec_create(desc, bufs, stream_ptr):
    h = C.c_void_p()
    _check(lib().spec_create(C.byref(desc), C.byref(bufs), C.c_void_p(stream_ptr), C.byref(h)))
    return h.value


def spec_create_static(desc, bufs, stream_ptr):
    h = C.c_void_p()
    _check(lib().spec_create_static(C.byref(desc), C.byref(bufs), C.c_void_p(stream_ptr), C.byref(h)))
    return h.value


def spec_destroy(ctx):
    return _check(lib().spec_destroy(ctx))


def spec_load_matrix(ctx, layer, which, src_ptr, scales_ptr=None):
    return _check(lib().spec_load_matrix(ctx, layer, which, C.c_void_p(src_ptr),
                                         C.c_void_p(scales_ptr) if scales_ptr else None), ctx)


def spec_load_norm(ctx, layer, which, src_ptr):
    return _check(lib().spec_load_norm(ctx, layer, which, C.c_void_p(src_ptr)), ctx)


def spec_prefill(ctx, tokens):
    t, tp = _i32(tokens)
    g = C.c_int32()
    _check(lib().spec_prefill(ctx, tp, len(t), C.byref(g)), ctx)
    return g.value


def spec_prefill_seq(ctx, seq, tokens):
    t, tp = _i32(tokens)
    g = C.c_int32()
    _check(lib().spec_prefill_seq(ctx, seq, tp, len(t), C.byref(g)), ctx)
    return g.value


def spec_verify(ctx, span):
    s, sp = _i32(span)
    am, ap = _i32(np.zeros(len(s), np.int32))
    m = C.c_int32()
    _check(lib().spec_verify(ctx, sp, len(s) - 1, ap, C.byref(m)), ctx)
    return am.copy(), m.value


def spec_verify_batch(ctx, seq_ids, spans):
    ids, idp = _i32(seq_ids)
    sp2 = np.ascontiguousarray(np.asarray(spans, np.int32))
    n, S = sp2.shape
    s, sp = _i32(sp2.reshape(-1))
    am, ap = _i32(np.zeros(n * S, np.int32))
    acc, accp = _i32(np.zeros(n, np.int32))
    _check(lib().spec_verify_batch(ctx, n, idp, sp, S - 1, ap, accp), ctx)
    return am.reshape(n, S).copy(), acc.copy()


def spec_verify_batch_k(ctx, seq_ids, spans, drafts):
    """spans [n_seq, K+1] (rows past 1 + drafts[b] are padding), drafts [n_seq]."""
    ids, idp = _i32(seq_ids)
    sp2 = np.ascontiguousarray(np.asarray(spans, np.int32))
    n, S = sp2.shape
    s, sp = _i32(sp2.reshape(-1))
    kd, kdp = _i32(drafts)
    am, ap = _i32(np.zeros(n * S, np.int32))
    acc, accp = _i32(np.zeros(n, np.int32))
    _check(lib().spec_verify_batch_k(ctx, n, idp, sp, S - 1, kdp, ap, accp), ctx)
    return am.reshape(n, S).copy(), acc.copy()


def spec_rewind(ctx, length):
    return _check(lib().spec_rewind(ctx, length), ctx)


def spec_rewind_seq(ctx, seq, length):
    return _check(lib().spec_rewind_seq(ctx, seq, length), ctx)


def spec_cache_len(ctx):
    v = C.c_int32()
    _check(lib().spec_cache_len(ctx, C.byref(v)), ctx)
    return v.value


def spec_cache_len_seq(ctx, seq):
    v = C.c_int32()
    _check(lib().spec_cache_len_seq(ctx, seq, C.byref(v)), ctx)
    return v.value


def spec_release_seq(ctx, seq):
    return _check(lib().spec_release_seq(ctx, seq), ctx)


def spec_set_sampling(ctx, temperature, seed=0):
    return _check(lib().spec_set_sampling(ctx, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF), ctx)


def spec_debug_logits(ctx, rows, vocab):
    out = np.zeros((rows, vocab), np.float32)
    _check(lib().spec_debug_logits(ctx, out.ctypes.data_as(C.POINTER(C.c_float)), rows), ctx)
    return out


def spec_get_stats(ctx):
    s = spec_stats()
    _check(lib().spec_get_stats(ctx, C.byref(s)), ctx)
    return {"forwards": s.forwards, "verify_calls": s.verify_calls, "drafted": s.drafted,
            "accepted": s.accepted, "forwards_by_span": list(s.forwards_by_span), "graphs": s.graphs,
            "forward_ms_by_span": list(s.forward_ms_by_span)}


def spec_time_verify(ctx, spans):
    sp2 = np.ascontiguousarray(np.asarray(spans, np.int32))
    iters, S = sp2.shape
    s, sp = _i32(sp2.reshape(-1))
    ms = np.zeros(iters, np.float32)
    _check(lib().spec_time_verify(ctx, S, iters, sp, ms.ctypes.data_as(C.POINTER(C.c_float))), ctx)
    return ms


def spec_profile_ops(ctx, spans):
    sp2 = np.ascontiguousarray(np.asarray(spans, np.int32))
    iters, S = sp2.shape
    s, sp = _i32(sp2.reshape(-1))
    us = np.zeros(SPEC_OP_COUNT, np.float32)
    n, npp = _i32(np.zeros(SPEC_OP_COUNT, np.int32))
    _check(lib().spec_profile_ops(ctx, S, iters, sp, us.ctypes.data_as(C.POINTER(C.c_float)), npp), ctx)
    return {OPS[i]: (float(us[i]), int(n[i])) for i in range(SPEC_OP_COUNT)}


def spec_time_op(ctx, op, S, reps):
    us = C.c_float()
    _check(lib().spec_time_op(ctx, OPS.index(op) if isinstance(op, str) else op, S, reps, C.byref(us)), ctx)
    return us.value


def spec_measure_read_bw(buf_ptr, nbytes, sink_ptr, reps, stream_ptr):
    g = C.c_double()
    _check(lib().spec_measure_read_bw(C.c_void_p(buf_ptr), nbytes, C.c_void_p(sink_ptr), reps,
                                      C.c_void_p(stream_ptr), C.byref(g)))
    return g.value


def spec_measure_read_chain(buf_ptr, region_bytes, n_regions, grid, sink_ptr, stream_ptr):
    us = C.c_double()
    _check(lib().spec_measure_read_chain(C.c_void_p(buf_ptr), region_bytes, n_regions, grid, C.c_void_p(sink_ptr),
                                         C.c_void_p(stream_ptr), C.byref(us)))
    return us.value


def spec_op_bytes(desc, op, S, ctx_len):
    b = C.c_double()
    _check(lib().spec_op_bytes(C.byref(desc), OPS.index(op) if isinstance(op, str) else op, S, ctx_len,
                               C.byref(b)))
    return b.value


def spec_ngram_create(n_min, n_max, capacity):
    h = C.c_void_p()
    _check(lib().spec_ngram_create(n_min, n_max, capacity, C.byref(h)))
    return h.value


def spec_ngram_destroy(ng):
    return _check(lib().spec_ngram_destroy(ng))


def spec_ngram_append(ng, toks):
    t, tp = _i32(toks)
    return _check(lib().spec_ngram_append(ng, tp, len(t)))


def spec_ngram_truncate(ng, length):
    return _check(lib().spec_ngram_truncate(ng, length))


def spec_ngram_len(ng):
    return _check(lib().spec_ngram_len(ng))


def spec_ngram_propose(ng, K):
    d, dp = _i32(np.zeros(max(K, 1), np.int32))
    c = _check(lib().spec_ngram_propose(ng, K, dp))
    return [int(x) for x in d[:c]]


def spec_adapt_k(k, drafted, accepted, k_cap):
    return int(lib().spec_adapt_k(k, drafted, accepted, k_cap))


def spec_generate(ctx, prompt, n_tokens, spec=True, fixed_k=0, k_cap=7, n_min=2, n_max=4,
                  draft_source=SPEC_DRAFT_NGRAM, ref_stream=None, governed=False):
    p, pp = _i32(prompt)
    out, op = _i32(np.zeros(n_tokens, np.int32))
    ref = None
    if ref_stream is not None:
        ref, refp = _i32(ref_stream)
    params = spec_gen_params(int(spec), fixed_k, k_cap, n_min, n_max, draft_source,
                             refp if ref is not None else None, int(governed))
    st = spec_gen_stats()
    _check(lib().spec_generate(ctx, pp, len(p), n_tokens, C.byref(params), op, C.byref(st)), ctx)
    return out.copy(), _gen_stats_dict(st)


def _gen_stats_dict(st):
    return {"forwards": st.forwards, "drafted": st.drafted, "accepted": st.accepted,
            "accept_hist": list(st.accept_hist), "forwards_by_span": list(st.forwards_by_span),
            "decode_s": st.decode_s, "host_s": st.host_s, "prefill_s": st.prefill_s,
            "plain_steps": st.plain_steps}


GOV_FIELDS = ("wins", "losses", "probes", "spec_steps", "plain_samples", "parked_steps", "state",
              "plain_ms_per_token", "spec_ms_per_token")


def _gov_stats_dict(st):
    return {f: getattr(st, f) for f in GOV_FIELDS}


class Governor:
    """spec_governor_create / should_draft / record / new_request / get_stats."""

    def __init__(self, params=None):
        h = C.c_void_p()
        _check(lib().spec_governor_create(C.byref(params) if params is not None else None, C.byref(h)))
        self.h = h.value

    def should_draft(self):
        return bool(_check(lib().spec_governor_should_draft(self.h)))

    def record(self, speculative, committed, accepted, seconds):
        return _check(lib().spec_governor_record(self.h, int(speculative), int(committed), int(accepted),
                                                 float(seconds)))

    def new_request(self):
        return _check(lib().spec_governor_new_request(self.h))

    def stats(self):
        st = spec_governor_stats()
        _check(lib().spec_governor_get_stats(self.h, C.byref(st)))
        return _gov_stats_dict(st)

    def close(self):
        if self.h:
            lib().spec_governor_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class spec_gen_handle:
    """spec_gen_begin / spec_gen_step / spec_gen_tokens / spec_gen_end."""

    def __init__(self, ctx, prompt, capacity, spec=True, fixed_k=0, k_cap=7, n_min=2, n_max=4,
                 draft_source=SPEC_DRAFT_NGRAM, ref_stream=None, governed=False):
        self.ctx = ctx
        self._p, pp = _i32(prompt)
        self._ref = None
        refp = None
        if ref_stream is not None:
            self._ref, refp = _i32(ref_stream)
        self.params = spec_gen_params(int(spec), fixed_k, k_cap, n_min, n_max, draft_source, refp, int(governed))
        h = C.c_void_p()
        _check(lib().spec_gen_begin(ctx, pp, len(self._p), capacity, C.byref(self.params), C.byref(h)), ctx)
        self.h = h.value
        self.capacity = capacity
        self.st = spec_gen_stats()

    def step(self, rounds):
        return _check(lib().spec_gen_step(self.h, rounds, C.byref(self.st)), self.ctx)

    def stats(self):
        return _gen_stats_dict(self.st)

    def governor_stats(self):
        st = spec_governor_stats()
        _check(lib().spec_gen_governor_stats(self.h, C.byref(st)), self.ctx)
        return _gov_stats_dict(st)

    def tokens(self):
        out, op = _i32(np.zeros(self.capacity, np.int32))
        n = _check(lib().spec_gen_tokens(self.h, op, self.capacity), self.ctx)
        return out[:n].copy()

    def close(self):
        if self.h:
            lib().spec_gen_end(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------- session

class Session:
    """Device buffers, stream and context for one model on cuda:0.

    weights: a callable (kind, layer, name) -> torch tensor in the canonical
    format (see draft_verify_amd.synth), where kind is "layer" (name in
    wq..wd, g_attn, g_ffn) or "global" (emb, lm, g_final)."""

    def __init__(self, shape: dict, weights, max_ctx: int, max_seqs: int = 1, max_rows: int = 16,
                 n_blocks: int = 0, flags: int = 0, device: int = 0, fmt: str = "bf16", static: bool = False):
        """static: the context of spec_create_static (no workspace allocated:
        the library's static scratch serves as the workspace)."""
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("libspecv needs an MI355X (gfx950) GPU; none is visible")
        self.torch = torch
        self.shape = dict(shape)
        self.dev = torch.device("cuda", device)
        wfmt = {"bf16": SPEC_WFMT_BF16, "int4": SPEC_WFMT_INT4G128}[fmt]
        self.desc = make_desc(shape, max_ctx, max_seqs, max_rows, n_blocks, flags, wfmt)
        sz = spec_query_buffers(self.desc)
        self.sizes = sz
        u8 = torch.uint8
        self.w_buf = torch.empty(sz.weights_bytes, dtype=u8, device=self.dev)
        self.kv_buf = torch.empty(sz.kv_bytes, dtype=u8, device=self.dev)
        self.ws_buf = None if static else torch.empty(sz.workspace_bytes, dtype=u8, device=self.dev)
        self.host_buf = torch.empty(sz.host_bytes, dtype=u8, pin_memory=True)
        self.stream = torch.cuda.Stream(device=self.dev)  # default priority
        bufs = spec_device_buffers(self.w_buf.data_ptr(), sz.weights_bytes, self.kv_buf.data_ptr(),
                                   sz.kv_bytes, None if static else self.ws_buf.data_ptr(),
                                   0 if static else sz.workspace_bytes, self.host_buf.data_ptr(), sz.host_bytes)
        torch.cuda.synchronize(self.dev)
        create = spec_create_static if static else spec_create
        self.ctx = create(self.desc, bufs, self.stream.cuda_stream)
        self._load(weights)

    def _load_matrix(self, layer, which, t):
        """One canonical matrix: a bf16 tensor, or an int4 dict {q4, scales}."""
        torch = self.torch
        if isinstance(t, dict):
            q = t["q4"].to(self.dev).contiguous()
            sc = t["scales"].to(self.dev).contiguous()
            torch.cuda.synchronize(self.dev)
            spec_load_matrix(self.ctx, layer, which, q.data_ptr(), sc.data_ptr())
        else:
            t = t.to(self.dev).contiguous()
            torch.cuda.synchronize(self.dev)
            spec_load_matrix(self.ctx, layer, which, t.data_ptr())

    def _load(self, weights):
        torch = self.torch
        sh = self.shape
        with torch.cuda.stream(self.stream):
            for l in range(sh["n_layers"]):
                for name, which in MAT_IDS.items():
                    self._load_matrix(l, which, weights("layer", l, name))
                for name, which in (("g_attn", SPEC_NORM_ATTN), ("g_ffn", SPEC_NORM_FFN)):
                    t = weights("layer", l, name).to(self.dev, torch.float32).contiguous()
                    torch.cuda.synchronize(self.dev)
                    spec_load_norm(self.ctx, l, which, t.data_ptr())
            for name, which in (("emb", SPEC_MAT_EMB), ("lm", SPEC_MAT_LM)):
                self._load_matrix(0, which, weights("global", 0, name))
            t = weights("global", 0, "g_final").to(self.dev, torch.float32).contiguous()
            torch.cuda.synchronize(self.dev)
            spec_load_norm(self.ctx, 0, SPEC_NORM_FINAL, t.data_ptr())
        torch.cuda.synchronize(self.dev)

    def close(self):
        if getattr(self, "ctx", None):
            spec_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def synth_weights(shape: dict, seed: int = 0, device: str = "cpu", fmt: str = "bf16"):
    """Weight provider for Session drawing the seeded synthetic weights."""
    from . import synth

    def get(kind, layer, name):
        if kind == "layer":
            if name in ("g_attn", "g_ffn"):
                return synth.norm_gain(shape, device)
            return synth.matrix(shape, layer, name, seed, fmt, device)
        if name == "emb":
            return synth.embedding(shape, seed, device)
        if name == "lm":
            return synth.lm_head(shape, seed, fmt, device)
        return synth.norm_gain(shape, device)
    return get


def tree_weights(w: dict):
    """Weight provider over an already generated weights tree (synth.weights)."""
    def get(kind, layer, name):
        if kind == "layer":
            return w["layers"][layer][name]
        return w[name]
    return get
