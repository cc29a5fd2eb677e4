"""ctypes wrapper of the fp32 CPU oracle (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  It mirrors the verify transaction the pages
describe:

* verify = one forward over [last, d1..dK] with the trunk argmax per row, then
  accept_greedy and a cache advance of m+1 (pegainfer page "DFlash speculative
  decoding", transaction section and draft-seed alignment paragraph);
* the generation loop: plain greedy (spec off) or propose -> verify -> commit
  (spec on) with the n-gram prompt-lookup proposer and adaptive K (coreai-model-
  zoo note on n-gram spec decoding for dense models, end-to-end and adaptive-K
  sections; TensorSharp speculative decoding page, protocol section).

Weights are passed as numpy arrays in the canonical layout: bf16 bit patterns
(uint16) [rows][cols], or int4 group-128 (uint8 [rows][cols/2] + uint16 bf16
scales [rows][cols/128]); norm gains as float32.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

OK, EINVAL, ECAPACITY, ESTATE, ENAN, ENOMEM = 0, -1, -2, -3, -4, -5
FMT_BF16, FMT_INT4 = 0, 1
WQ, WK, WV, WO, WG, WU, WD = range(7)
MAT_EMB, MAT_LM = 100, 101
NORM_ATTN, NORM_FFN, NORM_FINAL = 0, 1, 2
LAYER_MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


class OracleError(RuntimeError):
    pass


class _Shape(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q", C.c_int32),
                ("n_kv", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("eps", C.c_float), ("rope_theta", C.c_double),
                ("swa_window", C.c_int32), ("swa_layers", C.c_uint64),
                ("rec_layers", C.c_uint64), ("rec_beta", C.c_float)]


_LIBS = {}


def load_lib(path: str = DEFAULT_LIB):
    path = os.path.abspath(path)
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        raise OracleError(f"oracle library not built: {path} (run python oracle/build.py)")
    lib = C.CDLL(path)
    P, I, F, D = C.c_void_p, C.c_int, C.c_float, C.c_double
    i32p, f32p = C.POINTER(C.c_int32), C.POINTER(C.c_float)
    lib.orc_new.restype = P
    lib.orc_new.argtypes = [C.POINTER(_Shape), I, I]
    lib.orc_free.argtypes = [P]
    lib.orc_free.restype = None
    lib.orc_set_matrix.argtypes = [P, I, I, I, I, I, P, P]
    lib.orc_set_norm.argtypes = [P, I, I, P]
    lib.orc_cache_len.argtypes = [P, I]
    lib.orc_rewind.argtypes = [P, I, I]
    lib.orc_forward.argtypes = [P, I, i32p, I, I, f32p, i32p, f32p]
    lib.orc_prefill.argtypes = [P, I, i32p, I, i32p, f32p]
    lib.orc_verify.argtypes = [P, I, i32p, I, i32p, i32p, f32p, f32p]
    lib.orc_accept_greedy.argtypes = [i32p, i32p, I]
    lib.orc_ngram_propose.argtypes = [i32p, I, I, I, I, i32p]
    lib.orc_adapt_k.argtypes = [I, I, I, I]
    lib.orc_rmsnorm.argtypes = [f32p, f32p, I, F, f32p]
    lib.orc_rmsnorm.restype = None
    lib.orc_rope.argtypes = [f32p, I, I, D]
    lib.orc_rope.restype = None
    lib.orc_attend.argtypes = [f32p, f32p, f32p, I, I, I, f32p, f32p]
    lib.orc_attend.restype = None
    lib.orc_silu.argtypes = [F]
    lib.orc_silu.restype = F
    lib.orc_argmax.argtypes = [f32p, I, f32p]
    lib.orc_matvec.argtypes = [I, I, I, P, P, f32p, I, f32p]
    u32p, u64 = C.POINTER(C.c_uint32), C.c_uint64
    lib.orc_philox4x32_10.argtypes = [u32p, u32p, u32p]
    lib.orc_philox4x32_10.restype = None
    lib.orc_uniform01.argtypes = [C.c_uint32]
    lib.orc_uniform01.restype = F
    lib.orc_gumbel.argtypes = [F]
    lib.orc_gumbel.restype = F
    lib.orc_gumbel_noise.argtypes = [u64, I, I, I]
    lib.orc_gumbel_noise.restype = F
    lib.orc_sample_row.argtypes = [f32p, I, F, u64, I, I, f32p]
    lib.orc_verify_sampled.argtypes = [P, I, i32p, I, F, u64, i32p, i32p, f32p, f32p]
    lib.orc_prefill_sampled.argtypes = [P, I, i32p, I, F, u64, i32p, f32p]
    lib.orc_delta_write.argtypes = [f32p, I, f32p, f32p, F]
    lib.orc_delta_write.restype = None
    lib.orc_delta_read.argtypes = [f32p, I, f32p, f32p]
    lib.orc_delta_read.restype = None
    lib.orc_plant.restype = I
    _LIBS[path] = lib
    return lib


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(C.POINTER(C.c_float))


def _check(rc, what):
    if rc < 0:
        raise OracleError(f"{what} failed with code {rc}")
    return rc


# ------------------------------------------------------------ free functions

def ngram_propose(history, n_min, n_max, k, lib=None):
    lib = lib or load_lib()
    h, hp = _i32(history)
    out, op = _i32(np.zeros(max(k, 1), np.int32))
    c = _check(lib.orc_ngram_propose(hp, len(h), n_min, n_max, k, op), "ngram_propose")
    return [int(x) for x in out[:c]]


def adapt_k(k, drafted, accepted, cap, lib=None):
    lib = lib or load_lib()
    return int(lib.orc_adapt_k(k, drafted, accepted, cap))


def accept_greedy(span, argmax, lib=None):
    lib = lib or load_lib()
    s, sp = _i32(span)
    a, ap = _i32(argmax)
    return int(lib.orc_accept_greedy(sp, ap, len(s) - 1))


def rmsnorm(x, g, eps, lib=None):
    lib = lib or load_lib()
    x, xp = _f32(x)
    g, gp = _f32(g)
    y, yp = _f32(np.zeros_like(x))
    lib.orc_rmsnorm(xp, gp, len(x), eps, yp)
    return y


def rope(v, pos, theta, lib=None):
    lib = lib or load_lib()
    v, vp = _f32(np.array(v, np.float32, copy=True))
    lib.orc_rope(vp, len(v), pos, theta)
    return v


def attend(q, K, V, t, lib=None):
    """One head over rows 0..t of K, V ([rows][hd], contiguous)."""
    lib = lib or load_lib()
    q, qp = _f32(q)
    K, kp = _f32(K)
    V, vp = _f32(V)
    hd = q.shape[0]
    o, op = _f32(np.zeros(hd, np.float32))
    sc, scp = _f32(np.zeros(t + 1, np.float32))
    lib.orc_attend(qp, kp, vp, t, hd, hd, op, scp)
    return o


def matvec(mat, X, lib=None):
    """Y = X W^T for one canonical matrix (bf16 uint16 array, or an int4 dict)."""
    lib = lib or load_lib()
    X, xp = _f32(np.atleast_2d(X))
    if isinstance(mat, dict):
        q4 = np.ascontiguousarray(mat["q4"], np.uint8)
        sc = np.ascontiguousarray(mat["scales"], np.uint16)
        rows, cols, fmt, d, s = q4.shape[0], q4.shape[1] * 2, FMT_INT4, q4, sc
    else:
        d = np.ascontiguousarray(mat, np.uint16)
        rows, cols, fmt, s = d.shape[0], d.shape[1], FMT_BF16, None
    if X.shape[1] != cols:
        raise OracleError("matvec: width mismatch")
    Y, yp = _f32(np.zeros((X.shape[0], rows), np.float32))
    _check(lib.orc_matvec(fmt, rows, cols, d.ctypes.data, None if s is None else s.ctypes.data,
                          xp, X.shape[0], yp), "matvec")
    return Y


def philox4x32_10(ctr, key, lib=None):
    lib = lib or load_lib()
    c = (C.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (C.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (C.c_uint32 * 4)()
    lib.orc_philox4x32_10(c, k, out)
    return [int(x) for x in out]


def uniform01(x, lib=None):
    return float((lib or load_lib()).orc_uniform01(int(x) & 0xFFFFFFFF))


def gumbel(u, lib=None):
    return float((lib or load_lib()).orc_gumbel(float(u)))


def gumbel_noise(seed, seq, t, v, lib=None):
    return float((lib or load_lib()).orc_gumbel_noise(int(seed), seq, t, v))


def sample_row(logits, temp, seed, seq, t, lib=None):
    """The token drawn from one row of logits (Gumbel-max at temperature
    temp, Philox noise of (seed, seq, position t)) and the score margin."""
    lib = lib or load_lib()
    v, vp = _f32(logits)
    m = C.c_float(0.0)
    a = lib.orc_sample_row(vp, len(v), float(temp), int(seed), seq, t, C.byref(m))
    if a < 0:
        raise OracleError("sampling a row holding NaN")
    return int(a), float(m.value)


def delta_write(S, k, v, beta, lib=None):
    """One delta-rule write into a copy of the state S [hd][hd]; returns it."""
    lib = lib or load_lib()
    S, sp = _f32(np.array(S, np.float32, copy=True))
    k, kp = _f32(k)
    v, vp = _f32(v)
    lib.orc_delta_write(sp, len(k), kp, vp, float(beta))
    return S


def delta_read(S, q, lib=None):
    lib = lib or load_lib()
    S, sp = _f32(S)
    q, qp = _f32(q)
    o, op = _f32(np.zeros(len(q), np.float32))
    lib.orc_delta_read(sp, len(q), qp, op)
    return o


def silu(x, lib=None):
    lib = lib or load_lib()
    return float(lib.orc_silu(float(x)))


def argmax(v, lib=None):
    lib = lib or load_lib()
    v, vp = _f32(v)
    m = C.c_float(0.0)
    a = lib.orc_argmax(vp, len(v), C.byref(m))
    if a < 0:
        raise OracleError("argmax of a row holding NaN")
    return int(a), float(m.value)


# -------------------------------------------------------------------- model

class Oracle:
    """The trunk plus the verify transaction, over borrowed numpy weights."""

    def __init__(self, shape: dict, weights: dict, max_ctx: int, n_seq: int = 1, lib_path=None):
        self.lib = load_lib(lib_path or DEFAULT_LIB)
        self.shape = dict(shape)
        s = _Shape(shape["n_layers"], shape["hidden"], shape["n_q"], shape["n_kv"],
                   shape["head_dim"], shape["ffn"], shape["vocab"], shape["eps"],
                   shape["rope_theta"], shape.get("swa_window", 0), shape.get("swa_layers", 0),
                   shape.get("rec_layers", 0), shape.get("rec_beta", 0.0))
        self.h = self.lib.orc_new(C.byref(s), max_ctx, n_seq)
        if not self.h:
            raise OracleError("orc_new failed")
        self.max_ctx, self.n_seq = max_ctx, n_seq
        self._keep = []
        for l in range(shape["n_layers"]):
            for w, name in enumerate(LAYER_MATS):
                self._set_mat(l, w, weights["layers"][l][name])
            self._set_norm(l, NORM_ATTN, weights["layers"][l]["g_attn"])
            self._set_norm(l, NORM_FFN, weights["layers"][l]["g_ffn"])
        self._set_mat(0, MAT_EMB, weights["emb"])
        self._set_mat(0, MAT_LM, weights["lm"])
        self._set_norm(0, NORM_FINAL, weights["g_final"])

    def _set_mat(self, layer, which, m):
        if isinstance(m, dict):  # int4 group-128
            q4 = np.ascontiguousarray(m["q4"], np.uint8)
            sc = np.ascontiguousarray(m["scales"], np.uint16)
            self._keep += [q4, sc]
            rows, cols = q4.shape[0], q4.shape[1] * 2
            rc = self.lib.orc_set_matrix(self.h, layer, which, FMT_INT4, rows, cols,
                                         q4.ctypes.data, sc.ctypes.data)
        else:
            w = np.ascontiguousarray(m, np.uint16)
            self._keep.append(w)
            rc = self.lib.orc_set_matrix(self.h, layer, which, FMT_BF16, w.shape[0], w.shape[1],
                                         w.ctypes.data, None)
        _check(rc, "orc_set_matrix")

    def _set_norm(self, layer, which, g):
        g = np.ascontiguousarray(g, np.float32)
        self._keep.append(g)
        _check(self.lib.orc_set_norm(self.h, layer, which, g.ctypes.data), "orc_set_norm")

    def close(self):
        if self.h:
            self.lib.orc_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- transaction ------------------------------------------------------
    def cache_len(self, seq=0):
        return _check(self.lib.orc_cache_len(self.h, seq), "cache_len")

    def rewind(self, length, seq=0):
        _check(self.lib.orc_rewind(self.h, seq, length), "rewind")

    def forward(self, toks, seq=0, lm_from=0, want_logits=False):
        t, tp = _i32(toks)
        n = len(t)
        nl = n - lm_from
        am, ap = _i32(np.zeros(max(nl, 1), np.int32))
        mg, mp = _f32(np.zeros(max(nl, 1), np.float32))
        lg = np.zeros((nl, self.shape["vocab"]), np.float32) if want_logits else None
        lgp = lg.ctypes.data_as(C.POINTER(C.c_float)) if want_logits else None
        _check(self.lib.orc_forward(self.h, seq, tp, n, lm_from, lgp, ap, mp), "forward")
        return am[:nl].copy(), mg[:nl].copy(), lg

    def prefill(self, toks, seq=0, temp=0.0, seed=0):
        """g0 = the argmax of the last prompt row, or (temp > 0) the token
        drawn from it."""
        t, tp = _i32(toks)
        g, gp = _i32(np.zeros(1, np.int32))
        mg, mp = _f32(np.zeros(1, np.float32))
        if temp > 0:
            _check(self.lib.orc_prefill_sampled(self.h, seq, tp, len(t), float(temp), int(seed), gp, mp),
                   "prefill_sampled")
        else:
            _check(self.lib.orc_prefill(self.h, seq, tp, len(t), gp, mp), "prefill")
        return int(g[0]), float(mg[0])

    def verify(self, span, seq=0, want_logits=False, temp=0.0, seed=0):
        """Greedy verify (argmax rows), or sampled (temp > 0: drawn rows).
        Returns (tokens per row, accept length, margins, logits or None)."""
        s, sp = _i32(span)
        K = len(s) - 1
        am, ap = _i32(np.zeros(K + 1, np.int32))
        acc, accp = _i32(np.zeros(1, np.int32))
        mg, mp = _f32(np.zeros(K + 1, np.float32))
        lg = np.zeros((K + 1, self.shape["vocab"]), np.float32) if want_logits else None
        lgp = lg.ctypes.data_as(C.POINTER(C.c_float)) if want_logits else None
        if temp > 0:
            _check(self.lib.orc_verify_sampled(self.h, seq, sp, K, float(temp), int(seed), ap, accp, lgp, mp),
                   "verify_sampled")
        else:
            _check(self.lib.orc_verify(self.h, seq, sp, K, ap, accp, lgp, mp), "verify")
        return am.copy(), int(acc[0]), mg.copy(), lg

    # -- generation loop --------------------------------------------------
    def generate(self, prompt, n_tokens, spec=False, fixed_k=None, k_cap=7, n_min=2, n_max=4,
                 seq=0, drafts_fn=None, temp=0.0, seed=0):
        """Greedy generation of n_tokens tokens counted from g0.

        spec=False: one plain step (K=0) per token.  spec=True: propose with the
        n-gram lookup over prompt + committed tokens, verify, commit.  K is
        fixed_k if given, else adaptive (start 1, cap k_cap).  drafts_fn, if
        given, replaces the proposer (history, K) -> drafts.  A round never
        drafts past the budget; should it commit past it anyway, the commit is
        truncated and the cache rewound to match.
        Returns (tokens, stats)."""
        g0, _ = self.prefill(prompt, seq, temp=temp, seed=seed)
        hist = [int(t) for t in prompt] + [g0]
        out = [g0]
        k = fixed_k if fixed_k is not None else 1
        stats = {"forwards": 0, "drafted": 0, "accepted": 0, "accept_hist": {}}
        while len(out) < n_tokens:
            drafts = []
            if spec:
                kk = max(0, min(k, n_tokens - len(out) - 1))
                drafts = drafts_fn(hist, kk) if drafts_fn else ngram_propose(hist, n_min, n_max, kk, self.lib)
            span = [hist[-1]] + list(drafts)
            p = self.cache_len(seq)
            am, m, _, _ = self.verify(span, seq, temp=temp, seed=seed)
            stats["forwards"] += 1
            stats["drafted"] += len(drafts)
            stats["accepted"] += m
            stats["accept_hist"][m] = stats["accept_hist"].get(m, 0) + 1
            commit = [int(x) for x in am[: m + 1]]
            room = n_tokens - len(out)
            if len(commit) > room:
                commit = commit[:room]
                self.rewind(p + len(commit), seq)
            out += commit
            hist += commit
            if spec and fixed_k is None:
                k = adapt_k(k, len(drafts), m, k_cap, self.lib)
        return out, stats
