"""fp64 reference of the attention step of one decoder layer (decode, one token).

"Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
memória em um Mac comum": section "Sem dependências do llama.cpp e MLX"
lists hand-written GPU kernels for attention, RMSNorm and RoPE next to the
MoE ones; section "Qual é o principal truque da arquitetura" keeps the KV
cache for the context resident in FP16. Nothing more is printed, so the
step below is this project's reading (pre-norm block, rotate-half RoPE,
grouped-query attention):

  h      = x / sqrt(mean(x^2) + eps) * w_norm           RMSNorm, learned weight
  [q|k|v] = Wqkv @ h                                     one int4 g32 matrix,
                                                         q rows, then k rows, then v rows
  q_h    = rope(q_h, pos)   for every query head h
  k_g    = rope(k_g, pos)   for every key/value head g
  K[g][pos] = fp16(k_g),  V[g][pos] = fp16(v_g)          cache append (round to nearest even)
  a_h    = sum_t softmax_t(q_h . K[g(h)][t] / sqrt(d)) V[g(h)][t],  t = 0..pos,
           g(h) = h // (n_heads / n_kv_heads)
  y      = x + Wo @ [a_0 | a_1 | ...]

rope(v, p): pairs (i, i + d/2), i < d/2, rotate by the angle p * theta^(-2i/d):
  v_i' = v_i cos - v_{i+d/2} sin,   v_{i+d/2}' = v_{i+d/2} cos + v_i sin.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from . import q4


def rmsnorm_weighted(x, w, eps: float = 1e-6):
    """x / sqrt(mean(x^2) + eps) * w along the last axis, fp64."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def rope_angles(pos: int, d: int, theta: float = 10000.0):
    """Angle of pair i at position pos: pos * theta^(-2i/d), i < d/2."""
    i = np.arange(d // 2, dtype=np.float64)
    return float(pos) * theta ** (-2.0 * i / d)


def rope(v, pos: int, theta: float = 10000.0):
    """Rotate-half RoPE of v [..., d] at position pos (fp64)."""
    v = np.asarray(v, np.float64)
    d = v.shape[-1]
    a = rope_angles(pos, d, theta)
    c, s = np.cos(a), np.sin(a)
    lo, hi = v[..., : d // 2], v[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def fp16_round(x):
    """Round to the nearest fp16 (ties to even), returned as fp64."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def attention(q, k_cache, v_cache, n_ctx: int):
    """Grouped-query attention of one token over cache positions [0, n_ctx).
    q [nh][d]; caches [nkv][>= n_ctx][d]. Returns a [nh][d] (fp64)."""
    q = np.asarray(q, np.float64)
    nh, d = q.shape
    nkv = k_cache.shape[0]
    per = nh // nkv
    out = np.empty((nh, d))
    for h in range(nh):
        g = h // per
        K = np.asarray(k_cache[g, :n_ctx], np.float64)
        V = np.asarray(v_cache[g, :n_ctx], np.float64)
        s = K @ q[h] / np.sqrt(d)
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ V
    return out


def split_qkv(qkv, a):
    """[q rows | k rows | v rows] -> q [nh][d], k [nkv][d], v [nkv][d]."""
    d = a.head_dim
    nq, nk = a.n_heads * d, a.n_kv_heads * d
    return (qkv[:nq].reshape(a.n_heads, d), qkv[nq:nq + nk].reshape(a.n_kv_heads, d),
            qkv[nq + nk:].reshape(a.n_kv_heads, d))


def decode_step(x, w: dict, k_cache, v_cache, pos: int, a) -> dict:
    """One token through the attention step at position pos. The caches (fp16
    arrays [nkv][max_ctx][d]) receive the token's key and value at pos in place.
    Returns y = x + Wo a, and the intermediate q (rotated), k, v, a."""
    if not 0 <= pos < a.max_ctx:
        raise ValueError(f"position {pos} outside [0, {a.max_ctx})")
    h = rmsnorm_weighted(x, w["norm_w"], a.eps)
    qkv = q4.dequant(w["qkv_q"], w["qkv_s"]) @ h
    q, k, v = split_qkv(qkv, a)
    q = rope(q, pos, a.rope_theta)
    k = rope(k, pos, a.rope_theta)
    k_cache[:, pos] = k.astype(np.float16)
    v_cache[:, pos] = v.astype(np.float16)
    att = attention(q, k_cache, v_cache, pos + 1)
    o = q4.dequant(w["o_q"], w["o_s"]) @ att.reshape(-1)
    return {"y": np.asarray(x, np.float64) + o, "o": o, "q": q, "k": k, "v": v, "a": att}


def step_bytes(a, n_ctx: int) -> dict:
    """Bytes one decode step reads: both projections (nibbles + fp16 scales)
    and the K and V rows of n_ctx positions (fp16)."""
    qkv = a.qkv_rows * (a.hidden // 2 + 2 * (a.hidden // a.group))
    o = a.hidden * (a.attn_width // 2 + 2 * (a.attn_width // a.group))
    kv = 2 * a.n_kv_heads * n_ctx * a.head_dim * 2
    return {"qkv": qkv, "o": o, "kv": kv, "total": qkv + o + kv}
