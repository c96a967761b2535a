"""Explicit-loop references used to pin the oracle on tiny shapes.

Written independently of ``oracle`` (no imports from it): byte offsets,
nibble decoding and the FFN are spelled out element by element.
"""
import math

import numpy as np


def _offsets(H, I):
    o_gate_q = 0
    o_up_q = o_gate_q + I * H // 2
    o_down_q = o_up_q + I * H // 2
    o_gate_s = o_down_q + H * I // 2
    o_up_s = o_gate_s + I * (H // 32) * 2
    o_down_s = o_up_s + I * (H // 32) * 2
    end = o_down_s + H * (I // 32) * 2
    return o_gate_q, o_up_q, o_down_q, o_gate_s, o_up_s, o_down_s, end


def _nibble(byte, k):
    n = (byte >> 4) if (k % 2) else (byte & 15)
    return n - 16 if n > 7 else n


def _fp16_at(blob, off):
    return float(np.frombuffer(bytes(blob[off:off + 2]), np.float16)[0])


def matrix_bruteforce(blob, q_off, s_off, rows, cols):
    """W[r][c] for a matrix stored at (q_off, s_off), decoded one element at a time."""
    W = np.zeros((rows, cols))
    for r in range(rows):
        for c in range(cols):
            byte = int(blob[q_off + r * (cols // 2) + c // 2])
            sc = _fp16_at(blob, s_off + 2 * (r * (cols // 32) + c // 32))
            W[r, c] = _nibble(byte, c) * sc
    return W


def expert_weights_bruteforce(blob, H, I):
    gq, uq, dq, gs, us, ds, end = _offsets(H, I)
    assert len(blob) == end
    return (matrix_bruteforce(blob, gq, gs, I, H),
            matrix_bruteforce(blob, uq, us, I, H),
            matrix_bruteforce(blob, dq, ds, H, I))


def gelu_tanh_scalar(z):
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def ffn_loops(Wg, Wu, Wd, u):
    I, H = Wg.shape
    a = [0.0] * I
    for i in range(I):
        g = sum(Wg[i, k] * u[k] for k in range(H))
        v = sum(Wu[i, k] * u[k] for k in range(H))
        a[i] = gelu_tanh_scalar(g) * v
    return np.array([sum(Wd[h, i] * a[i] for i in range(I)) for h in range(H)])


def dense_ffn_bruteforce_weights(blob, H, I, u):
    """Weights by explicit loops, the FFN by numpy BLAS."""
    Wg, Wu, Wd = expert_weights_bruteforce(blob, H, I)
    g = Wg @ u
    v = Wu @ u
    a = np.array([gelu_tanh_scalar(x) for x in g]) * v
    return Wd @ a


def layer_loops(u, E, k, H, I, Is, router, shared, experts, bias=None):
    """Whole layer by explicit loops for one token (tiny shapes only)."""
    z = [sum(float(router[e, c]) * u[c] for c in range(H)) + (float(bias[e]) if bias is not None else 0.0)
         for e in range(E)]
    order = sorted(range(E), key=lambda e: (-z[e], e))[:k]
    m = max(z[e] for e in order)
    ex = [math.exp(z[e] - m) for e in order]
    w = [x / sum(ex) for x in ex]
    y = ffn_loops(*expert_weights_bruteforce(shared, H, Is), u)
    for j, e in enumerate(order):
        y = y + w[j] * ffn_loops(*expert_weights_bruteforce(experts[e], H, I), u)
    return order, w, y
