"""An independent fp64 reference of the trunk built from torch library routines.

It pins the CPU oracle against library definitions rather than against a copy
of its own formulas: RMSNorm is torch.nn.functional.rms_norm, attention is
scaled_dot_product_attention with its own causal (or, for a sliding-window
layer, band) mask built from torch.tril and grouped-query mapping (enable_gqa), the MLP gate uses F.silu, and the rotary embedding is a
complex multiplication (torch.polar) instead of the oracle's real-valued
rotate-half formula.  Only the conventions the pages leave open are shared by
construction: rotate-half pairing (i, i + d/2), base theta, epsilon, untied
embedding and LM head.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F


def _f64(t):
    if isinstance(t, dict):  # int4 group-128 -> dense fp64 weights
        q4 = t["q4"].to(torch.int64)
        lo = q4 & 15
        hi = (q4 >> 4) & 15
        nib = torch.stack([lo, hi], dim=-1).reshape(q4.shape[0], q4.shape[1] * 2)
        q = torch.where(nib >= 8, nib - 16, nib).to(torch.float64)
        s = t["scales"].to(torch.float64).repeat_interleave(128, dim=1)
        return q * s
    return t.to(torch.float64)


def logits(shape: dict, w: dict, tokens) -> np.ndarray:
    """fp64 logits of every position of `tokens` run from an empty cache."""
    H, nq, nkv, hd = shape["hidden"], shape["n_q"], shape["n_kv"], shape["head_dim"]
    eps, theta = shape["eps"], shape["rope_theta"]
    toks = torch.as_tensor(np.asarray(tokens), dtype=torch.long)
    T = toks.shape[0]
    x = _f64(w["emb"])[toks]
    pos = torch.arange(T, dtype=torch.float64)
    freq = theta ** (-2.0 * torch.arange(hd // 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(T, hd // 2, dtype=torch.float64), pos[:, None] * freq[None, :])

    def rope(z):  # [T, heads, hd]
        c = torch.complex(z[..., : hd // 2], z[..., hd // 2:]) * rot[:, None, :]
        return torch.cat([c.real, c.imag], dim=-1)

    W = shape.get("swa_window", 0)
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    # a sliding-window layer: query i sees keys j with i - W < j <= i (a band mask)
    band = causal & ~torch.ones(T, T, dtype=torch.bool).tril(-W) if W else causal
    for li, L in enumerate(w["layers"]):
        u = F.rms_norm(x, (H,), weight=_f64(L["g_attn"]), eps=eps)
        q = rope(F.linear(u, _f64(L["wq"])).view(T, nq, hd))
        k = rope(F.linear(u, _f64(L["wk"])).view(T, nkv, hd))
        v = F.linear(u, _f64(L["wv"])).view(T, nkv, hd)
        if (shape.get("rec_layers", 0) >> li) & 1:
            # delta rule per kv head on unrotated, unit-normalised keys and queries
            q0 = F.normalize(F.linear(u, _f64(L["wq"])).view(T, nq, hd), dim=-1)
            k0 = F.normalize(F.linear(u, _f64(L["wk"])).view(T, nkv, hd), dim=-1)
            beta, G = shape["rec_beta"], nq // nkv
            S = torch.zeros(nkv, hd, hd, dtype=torch.float64)
            o = torch.empty(T, nq, hd, dtype=torch.float64)
            for t in range(T):
                err = v[t] - torch.einsum("gij,gj->gi", S, k0[t])
                S = S + beta * torch.einsum("gi,gj->gij", err, k0[t])
                o[t] = torch.einsum("gij,ghj->ghi", S, q0[t].view(nkv, G, hd)).reshape(nq, hd)
            x = x + F.linear(o.reshape(T, nq * hd), _f64(L["wo"]))
        else:
            local = W and (shape.get("swa_layers", 0) >> li) & 1
            o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                               attn_mask=band if local else causal,
                                               scale=1.0 / math.sqrt(hd), enable_gqa=True)
            x = x + F.linear(o.transpose(0, 1).reshape(T, nq * hd), _f64(L["wo"]))
        u = F.rms_norm(x, (H,), weight=_f64(L["g_ffn"]), eps=eps)
        x = x + F.linear(F.silu(F.linear(u, _f64(L["wg"]))) * F.linear(u, _f64(L["wu"])), _f64(L["wd"]))
    u = F.rms_norm(x, (H,), weight=_f64(w["g_final"]), eps=eps)
    return F.linear(u, _f64(w["lm"])).numpy()
