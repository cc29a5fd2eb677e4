"""Seeded synthetic inputs: model shapes, random-init weights and prompts.

This module only draws random numbers and lays them out in the canonical
storage formats.  It holds none of the method's arithmetic, and it is the only
code that both the HIP path and the CPU oracle consume.

Canonical weight formats (the oracle reads these directly; the library repacks
them on the device into its own layout):
  * bf16: a [rows, cols] torch.bfloat16 tensor, rows = outputs, cols = inputs;
  * int4 group-128: {"q4": uint8 [rows, cols/2], "scales": bf16 [rows, cols/128]}
    with w = scale * q, q in [-8, 7] two's complement, the low nibble holding
    the even column, groups of 128 consecutive inputs of one output row.

Shapes: the tiny decoder, the Qwen3-4B shape (the trunk of the pegainfer page,
"DFlash speculative decoding") and a 32B-class dense shape (the class of the
trunk measured on the coreai-model-zoo n-gram note).  Conventions the pages do
not fix: RMSNorm epsilon 1e-6 and RoPE base 1e6 (Qwen3 conventions), norm gains
1.0, untied embedding and LM head.
"""
from __future__ import annotations

import numpy as np
import torch

SHAPES = {
    "tiny": dict(n_layers=2, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=128, vocab=256,
                 eps=1e-6, rope_theta=1e6),
    "qwen3_4b": dict(n_layers=36, hidden=2560, n_q=32, n_kv=8, head_dim=128, ffn=9728,
                     vocab=151936, eps=1e-6, rope_theta=1e6),
    # four query heads per kv head: batched spans of 8 rows fill two 16-column
    # query tiles per (sequence, kv head) in attention
    "tiny_g4": dict(n_layers=2, hidden=64, n_q=8, n_kv=2, head_dim=16, ffn=128, vocab=256,
                    eps=1e-6, rope_theta=1e6),
    # the smallest decoder whose GEMM depths hold whole int4 groups of 128
    "tiny_int4": dict(n_layers=2, hidden=128, n_q=4, n_kv=2, head_dim=32, ffn=256, vocab=256,
                      eps=1e-6, rope_theta=1e6),
    "dense_32b": dict(n_layers=64, hidden=5120, n_q=64, n_kv=8, head_dim=128, ffn=25600,
                      vocab=151936, eps=1e-6, rope_theta=1e6),
    # sliding-window layers: the tiny decoder with layer 0 attending only its
    # last 24 positions (layer 1 stays global), and a 4-layer variant of the
    # 4B attention geometry with a 1024-position window on layers 0 and 2
    "tiny_swa": dict(n_layers=2, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=128, vocab=256,
                     eps=1e-6, rope_theta=1e6, swa_window=24, swa_layers=0b01),
    "attn_4b_swa": dict(n_layers=4, hidden=512, n_q=32, n_kv=8, head_dim=128, ffn=512, vocab=1024,
                        eps=1e-6, rope_theta=1e6, swa_window=1024, swa_layers=0b0101),
    # recurrent (delta-rule) layers: a 3-layer tiny decoder whose middle layer
    # is recurrent (write strength 0.5), and a 4-layer variant of the 4B
    # attention geometry (heads of 128) with recurrent layers 1 and 3
    "tiny_rec": dict(n_layers=3, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=128, vocab=256,
                     eps=1e-6, rope_theta=1e6, rec_layers=0b010, rec_beta=0.5),
    "attn_4b_rec": dict(n_layers=4, hidden=512, n_q=32, n_kv=8, head_dim=128, ffn=512, vocab=1024,
                        eps=1e-6, rope_theta=1e6, rec_layers=0b1010, rec_beta=0.5),
    # the attention geometry of the Qwen3-4B shape (32q/8kv heads of 128) and
    # of the 32B-class shape (64q/8kv heads of 128) on a narrow trunk (hidden
    # 512): long contexts at the real head layout, with projections small
    # enough for the CPU oracle to prefill thousands of tokens
    "attn_4b": dict(n_layers=2, hidden=512, n_q=32, n_kv=8, head_dim=128, ffn=512, vocab=1024,
                    eps=1e-6, rope_theta=1e6),
    "attn_32b": dict(n_layers=2, hidden=512, n_q=64, n_kv=8, head_dim=128, ffn=512, vocab=1024,
                     eps=1e-6, rope_theta=1e6),
}

LAYER_MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")
WEIGHT_STD = 0.02
INT4_SCALE = 0.00434  # scale = bf16(INT4_SCALE * U(0.5, 1.5)); effective weight std ~0.02


def shrink(shape: dict, **over) -> dict:
    s = dict(shape)
    s.update(over)
    return s


def matrix_dims(shape: dict) -> dict:
    H, hd, F = shape["hidden"], shape["head_dim"], shape["ffn"]
    return {"wq": (shape["n_q"] * hd, H), "wk": (shape["n_kv"] * hd, H),
            "wv": (shape["n_kv"] * hd, H), "wo": (H, shape["n_q"] * hd),
            "wg": (F, H), "wu": (F, H), "wd": (H, F)}


def _gen(seed: int, idx: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(idx)) & 0x7FFF_FFFF_FFFF)
    return g


def normal_bf16(rows, cols, seed, idx, device="cpu", std=WEIGHT_STD) -> torch.Tensor:
    """N(0, std) drawn in fp32 and rounded once to bf16."""
    g = _gen(seed, idx, device)
    w = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    return (w * std).to(torch.bfloat16)


def int4_g128(rows, cols, seed, idx, device="cpu") -> dict:
    """q uniform over [-8, 7], packed two per byte (low nibble = even column);
    one bf16 scale per 128 consecutive columns of a row."""
    assert cols % 128 == 0
    g = _gen(seed, idx, device)
    q = torch.randint(-8, 8, (rows, cols), generator=g, device=device, dtype=torch.int16)
    nib = (q & 0xF).to(torch.uint8)
    q4 = nib[:, 0::2] | (nib[:, 1::2] << 4)
    u = torch.rand((rows, cols // 128), generator=g, device=device, dtype=torch.float32)
    scales = (INT4_SCALE * (0.5 + u)).to(torch.bfloat16)
    return {"q4": q4.contiguous(), "scales": scales.contiguous()}


def matrix(shape: dict, layer: int, name: str, seed: int = 0, fmt: str = "bf16", device="cpu"):
    """One weight matrix; deterministic in (seed, layer, name) alone, so it can
    be regenerated on demand instead of being held."""
    dims = matrix_dims(shape)
    idx = layer * 16 + LAYER_MATS.index(name)
    rows, cols = dims[name]
    if fmt == "int4":
        return int4_g128(rows, cols, seed, idx, device)
    return normal_bf16(rows, cols, seed, idx, device)


def embedding(shape: dict, seed: int = 0, device="cpu") -> torch.Tensor:
    return normal_bf16(shape["vocab"], shape["hidden"], seed, 1_000_000, device)


def lm_head(shape: dict, seed: int = 0, fmt: str = "bf16", device="cpu"):
    if fmt == "int4":
        return int4_g128(shape["vocab"], shape["hidden"], seed, 1_000_001, device)
    return normal_bf16(shape["vocab"], shape["hidden"], seed, 1_000_001, device)


def norm_gain(shape: dict, device="cpu") -> torch.Tensor:
    return torch.ones(shape["hidden"], dtype=torch.float32, device=device)


def weights(shape: dict, seed: int = 0, fmt: str = "bf16", device="cpu") -> dict:
    """All weights of a model as torch tensors (fits in memory for the shapes
    that are generated whole; large shapes are better streamed with matrix())."""
    layers = []
    for l in range(shape["n_layers"]):
        d = {n: matrix(shape, l, n, seed, fmt, device) for n in LAYER_MATS}
        d["g_attn"] = norm_gain(shape, device)
        d["g_ffn"] = norm_gain(shape, device)
        layers.append(d)
    return {"layers": layers, "emb": embedding(shape, seed, device),
            "lm": lm_head(shape, seed, fmt, device), "g_final": norm_gain(shape, device)}


def to_numpy(w):
    """Host numpy view of a weights tree: bf16 -> uint16 bit patterns."""
    if isinstance(w, dict):
        return {k: to_numpy(v) for k, v in w.items()}
    if isinstance(w, list):
        return [to_numpy(v) for v in w]
    t = w.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ------------------------------------------------------------------ prompts

def motif_prompt(seed: int, vocab: int, motif: int = 8, reps: int = 4) -> np.ndarray:
    """A random motif of `motif` tokens repeated `reps` times."""
    rng = np.random.default_rng(seed)
    m = rng.integers(0, vocab, motif, dtype=np.int64)
    return np.tile(m, reps).astype(np.int32)


def uniform_prompt(seed: int, vocab: int, n: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, n, dtype=np.int64).astype(np.int32)


def repetition_prompt(seed: int, vocab: int, n: int, return_stats: bool = False):
    """Repetition-heavy stream: random spans of 16..48 tokens, each occurring
    2..4 times; later copies follow gaps of 0..64 fresh tokens and interleave
    with other spans.  Truncated to exactly n tokens."""
    rng = np.random.default_rng(seed)
    out: list[int] = []
    rep: list[int] = []          # span id per token (-1 = fresh filler)
    pending: list[list] = []     # [tokens, copies left, span id]
    n_spans = 0
    while len(out) < n:
        if pending and rng.random() < 0.6:
            gap = int(rng.integers(0, 65))
            out += [int(x) for x in rng.integers(0, vocab, gap)]
            rep += [-1] * gap
            j = int(rng.integers(0, len(pending)))
            toks, left, sid = pending[j]
            out += toks
            rep += [sid] * len(toks)
            if left <= 1:
                pending.pop(j)
            else:
                pending[j][1] = left - 1
        else:
            L = int(rng.integers(16, 49))
            c = int(rng.integers(2, 5))
            toks = [int(x) for x in rng.integers(0, vocab, L)]
            out += toks
            rep += [n_spans] * L
            pending.append([toks, c - 1, n_spans])
            n_spans += 1
    out, rep = out[:n], rep[:n]
    arr = np.asarray(out, dtype=np.int32)
    if not return_stats:
        return arr
    counts: dict[int, int] = {}
    # a span counts as repeated when at least two of its copies started in range
    starts = [i for i in range(n) if rep[i] >= 0 and (i == 0 or rep[i - 1] != rep[i])]
    for i in starts:
        counts[rep[i]] = counts.get(rep[i], 0) + 1
    repeated = sum(1 for i in range(n) if rep[i] >= 0 and counts.get(rep[i], 0) >= 2)
    return arr, {"repeated_fraction": repeated / n, "spans": n_spans}


def random_drafts(seed: int, vocab: int, count: int, k: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, (count, k), dtype=np.int64).astype(np.int32)
