"""fp64 matrix-form twin of the oracle, for tiny shapes only.

TEST INFRASTRUCTURE ONLY.  It evaluates the same decoder as ``orc.c`` but in a
different form: the whole token sequence at once, in float64, with the causal
mask written as an explicit -inf upper triangle instead of a token-by-token
loop.  Agreement between the two (within the f32 rounding bound) pins the
f32 oracle against errors in loop order, indexing or masking.

Steps follow "Scalar-Native Qwen3 Reference Runtime As The Numerical
Authority", section 2 items 1-7 (RMSNorm, bias-free Q/K/V, per-head QK-Norm,
RoPE, grouped-query scaled dot-product attention with causal mask, o_proj and
residual, SwiGLU MLP and residual, final norm and tied logits).
"""
from __future__ import annotations

import numpy as np


def _bf16(u16):
    return (np.asarray(u16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _mat64(m):
    if m.is_q8:
        return m.codes.astype(np.float64) * np.repeat(m.scales.astype(np.float64), 32, axis=1)
    return _bf16(m.bf16)


def _norm64(w, fmt):
    return _bf16(w) if fmt == 1 else np.asarray(w, np.float64)


def rmsnorm64(x, w, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rope64(x, pos, theta):
    """x [..., T, D]; rotate pairs (i, i + D/2) by pos * theta^(-2i/D)."""
    D = x.shape[-1]
    inv = theta ** (-2.0 * np.arange(D // 2) / D)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def forward64(weights, tokens=None, hidden=None, kv_round_bf16=False):
    """Full-sequence forward from position 0.  Returns (hidden [T,H], logits of the last position or None)."""
    s = weights.shape
    fmt = s.fmt
    if hidden is not None:
        x = np.asarray(hidden, np.float64)
    else:
        x = _mat64(weights.embed)[np.asarray(tokens)]
    T = x.shape[0]
    D, HQ, HKV = s.head_dim, s.n_q_heads, s.n_kv_heads
    g = HQ // HKV
    pos = np.arange(T)
    causal = np.triu(np.full((T, T), -np.inf), k=1)
    for L in weights.layers:
        r = x
        xn = rmsnorm64(x, _norm64(L["attn_norm"], fmt), s.eps)
        q = (xn @ _mat64(L["q"]).T).reshape(T, HQ, D).transpose(1, 0, 2)
        k = (xn @ _mat64(L["k"]).T).reshape(T, HKV, D).transpose(1, 0, 2)
        v = (xn @ _mat64(L["v"]).T).reshape(T, HKV, D).transpose(1, 0, 2)
        q = rope64(rmsnorm64(q, _norm64(L["q_norm"], fmt), s.eps), pos, s.theta)
        k = rope64(rmsnorm64(k, _norm64(L["k_norm"], fmt), s.eps), pos, s.theta)
        if kv_round_bf16:
            k = _round_bf16(k)
            v = _round_bf16(v)
        kk = np.repeat(k, g, axis=0)       # query head h reads KV head h // g
        vv = np.repeat(v, g, axis=0)
        sc = q @ kk.transpose(0, 2, 1) / np.sqrt(D) + causal
        sc = sc - sc.max(axis=-1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(axis=-1, keepdims=True)
        att = (p @ vv).transpose(1, 0, 2).reshape(T, HQ * D)
        x = r + att @ _mat64(L["o"]).T
        r = x
        xn = rmsnorm64(x, _norm64(L["mlp_norm"], fmt), s.eps)
        gt = xn @ _mat64(L["gate"]).T
        up = xn @ _mat64(L["up"]).T
        a = gt / (1.0 + np.exp(-gt)) * up
        x = r + a @ _mat64(L["down"]).T
    logits = None
    if weights.embed is not None:
        xn = rmsnorm64(x[-1], _norm64(weights.final_norm, fmt), s.eps)
        logits = _mat64(weights.embed) @ xn
    return x, logits


def _round_bf16(x64):
    f = x64.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return _bf16(u.astype(np.uint16))
