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


# --------------------------------------------------------------------------- attention step
def q4_matrix_loops(q, s):
    """W[r][c] of an int4 g32 matrix (q uint8 [N][K/2], s fp16 [N][K/32]), element by element."""
    N, K = q.shape[0], 2 * q.shape[1]
    W = np.zeros((N, K))
    for r in range(N):
        for c in range(K):
            W[r, c] = _nibble(int(q[r, c // 2]), c) * float(s[r, c // 32])
    return W


def attn_step_loops(x, w, kc, vc, pos, nh, nkv, d, theta, eps):
    """One decode token through the attention step by explicit loops (tiny
    shapes only). kc/vc (fp16 [nkv][ctx][d]) receive the token's key/value at
    pos. Returns y (list of floats)."""
    H = len(x)
    ss = sum(float(v) * float(v) for v in x) / H
    r = 1.0 / math.sqrt(ss + eps)
    h = [float(x[i]) * r * float(w["norm_w"][i]) for i in range(H)]
    Wqkv = q4_matrix_loops(w["qkv_q"], w["qkv_s"])
    proj = [sum(Wqkv[n, i] * h[i] for i in range(H)) for n in range(Wqkv.shape[0])]

    def rot(vec):
        out = list(vec)
        for i in range(d // 2):
            ang = pos * theta ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            out[i] = vec[i] * c - vec[i + d // 2] * s
            out[i + d // 2] = vec[i + d // 2] * c + vec[i] * s
        return out

    q = [rot(proj[hh * d:(hh + 1) * d]) for hh in range(nh)]
    for g in range(nkv):
        k = rot(proj[nh * d + g * d: nh * d + (g + 1) * d])
        v = proj[(nh + nkv) * d + g * d: (nh + nkv) * d + (g + 1) * d]
        for i in range(d):
            kc[g, pos, i] = np.float16(k[i])
            vc[g, pos, i] = np.float16(v[i])
    att = []
    for hh in range(nh):
        g = hh // (nh // nkv)
        sc = [sum(q[hh][i] * float(kc[g, t, i]) for i in range(d)) / math.sqrt(d) for t in range(pos + 1)]
        m = max(sc)
        e = [math.exp(v - m) for v in sc]
        tot = sum(e)
        att += [sum(e[t] / tot * float(vc[g, t, i]) for t in range(pos + 1)) for i in range(d)]
    Wo = q4_matrix_loops(w["o_q"], w["o_s"])
    return [float(x[n]) + sum(Wo[n, j] * att[j] for j in range(len(att))) for n in range(H)]
