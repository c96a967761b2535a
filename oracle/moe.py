"""fp64 reference of the MoE layer: routing, expert FFNs, combine, stack, prefill.

Per token (decode), following "Como executar um modelo de 26 bilhões de
parâmetros em dois gigabytes de memória em um Mac comum", section "Qual é
o principal truque da arquitetura" (router picks 8 experts per layer; the
shared-expert branch runs for every token):

  z   = Wr @ u (+ bias)                 router logits, fp64 sums
  ids = the k largest z, ties to the lower expert id, in rank order
  w   = exp(z_ids - max) / sum          softmax over the selected logits
        (identical to a softmax over all E followed by renormalising the k)
  o_e = Wd_e @ (gelu_tanh(Wg_e @ u) * (Wu_e @ u))     GeGLU expert FFN
  y   = o_shared + sum_j w_j * o_{ids_j}

gelu_tanh(z) = z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3))), the tanh
form of GELU published by Hendrycks & Gimpel.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import math

import numpy as np

from . import q4

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715


def gelu_tanh(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(SQRT_2_OVER_PI * (z + GELU_CUBIC * z ** 3)))


def rmsnorm(x, eps: float = 1e-6):
    """Weightless RMSNorm: x / sqrt(mean(x^2) + eps) along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


# --------------------------------------------------------------------------- routing
def router_logits(u, wr, bias=None):
    """z[e] = sum_k u[k] * Wr[e][k] (+ bias[e]), fp64. u: [H] or [B][H]; Wr fp16 [E][H]."""
    z = np.asarray(u, np.float64) @ np.asarray(wr).astype(np.float64).T
    if bias is not None:
        z = z + np.asarray(bias, np.float64)
    return z


def top_k(z, k: int):
    """Indices of the k largest entries of z (1-D), ties to the lower index, in rank order."""
    z = np.asarray(z, np.float64)
    ids = np.arange(z.size)
    order = np.lexsort((ids, -z))          # primary key -z, secondary key id
    return order[:k].astype(np.int32)


def route_weights(z, ids):
    """Softmax over the selected logits (max-subtracted)."""
    sel = np.asarray(z, np.float64)[np.asarray(ids)]
    e = np.exp(sel - sel.max())
    return e / e.sum()


def route(u=None, wr=None, k: int = 8, bias=None, logits_in=None):
    """Route B tokens. Returns (ids int32 [B][k], w fp64 [B][k], z fp64 [B][E])."""
    if logits_in is not None:
        z = np.atleast_2d(np.asarray(logits_in, np.float64))
    else:
        z = np.atleast_2d(router_logits(u, wr, bias))
    ids = np.stack([top_k(row, k) for row in z])
    w = np.stack([route_weights(row, i) for row, i in zip(z, ids)])
    return ids, w, z


# --------------------------------------------------------------------------- FFN
def ffn_from_matrices(wg, wu, wd, u):
    """GeGLU FFN on dequantised fp64 matrices; u: [H] or [T][H]."""
    u = np.asarray(u, np.float64)
    g = u @ wg.T
    v = u @ wu.T
    return (gelu_tanh(g) * v) @ wd.T


def expert_ffn(blob, hidden: int, inter: int, u):
    wg, wu, wd = q4.expert_matrices(blob, hidden, inter)
    return ffn_from_matrices(wg, wu, wd, u)


def layer_decode(u, shape, router, shared, experts, bias=None, logits_in=None, residual=None):
    """One MoE layer for B tokens; u fp [B][H] (already normalised if the caller norms).

    ``experts`` is uint8 [E][blob]; ``shared`` uint8 [blob_s]. Each token is
    computed on its own (the result does not depend on batching). Returns a
    dict with ids, w, z, y (fp64 [B][H]) and y_moe (without the residual).
    """
    u = np.atleast_2d(np.asarray(u, np.float64))
    H, I, Is = shape.hidden, shape.inter, shape.shared_inter
    ids, w, z = route(u, router, shape.top_k, bias, logits_in)
    y = expert_ffn(shared, H, Is, u)
    # each selected expert is dequantised once and applied to the tokens that chose it
    for e in np.unique(ids):
        rows, rank = np.nonzero(ids == e)
        o = expert_ffn(experts[e], H, I, u[rows])
        y[rows] += w[rows, rank][:, None] * o
    y_moe = y.copy()
    if residual is not None:
        y = y + np.atleast_2d(np.asarray(residual, np.float64))
    return {"ids": ids, "w": w, "z": z, "y": y, "y_moe": y_moe}


def layer_decode_per_token(u, shape, router, shared, experts, bias=None, logits_in=None):
    """The same layer, token by token and expert by expert, with no grouping."""
    u = np.atleast_2d(np.asarray(u, np.float64))
    ids, w, z = route(u, router, shape.top_k, bias, logits_in)
    H, I, Is = shape.hidden, shape.inter, shape.shared_inter
    ys = []
    for t in range(u.shape[0]):
        yt = expert_ffn(shared, H, Is, u[t])
        for j in range(shape.top_k):
            yt = yt + w[t, j] * expert_ffn(experts[ids[t, j]], H, I, u[t])
        ys.append(yt)
    return {"ids": ids, "w": w, "z": z, "y": np.stack(ys)}


# --------------------------------------------------------------------------- 30-layer stack
def stack_layer_step(h, eps_l, shape, layer, rms_eps: float = 1e-6):
    """One pre-norm block of the stack: h' = h + eps; u = rmsnorm(h'); h'' = h' + MoE(u).

    ``layer`` is a dict with router, bias, shared, experts. ``eps_l`` is the fp16
    perturbation standing in for attention. Returns (h'', record).
    """
    hp = np.atleast_2d(np.asarray(h, np.float64)) + np.asarray(eps_l, np.float16).astype(np.float64)
    u = rmsnorm(hp, rms_eps)
    r = layer_decode(u, shape, layer["router"], layer["shared"], layer["experts"],
                     bias=layer.get("bias"), residual=hp)
    r["u"] = u
    r["h_in"] = hp
    return r["y"], r


def stack_decode(x0, eps, shape, layers, rms_eps: float = 1e-6):
    """Run one token through all layers. eps: fp16 [L][H]. Returns (h_final, records)."""
    h = np.atleast_2d(np.asarray(x0, np.float64))
    recs = []
    for l, lay in enumerate(layers):
        h, r = stack_layer_step(h, eps[l], shape, lay, rms_eps)
        recs.append(r)
    return h, recs


# --------------------------------------------------------------------------- prefill
def bf16_round(x):
    """Round fp64 values to the nearest bf16 value (8 significant bits), ties to even."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # below 2^-126 bf16 is subnormal: fixed spacing 2^-133
    ulp = np.ldexp(1.0, e - 8)
    return np.round(x / ulp) * ulp           # numpy rounds halves to even


def prefill(x, shape, shared, experts, logits_in=None, router=None, bias=None, mirror_bf16=True):
    """Prefill of T tokens with the bf16 rounding points of an MFMA implementation.

    x: fp64 [T][H] holding bf16-exact values. With ``mirror_bf16`` every weight
    matrix is rounded to bf16 and the GeGLU activation a = gelu(g)*v is rounded
    to bf16 before the down projection; sums are fp64. Without it this is the
    decode oracle. Routing uses ``logits_in`` when given.
    """
    x = np.atleast_2d(np.asarray(x, np.float64))
    H, I, Is = shape.hidden, shape.inter, shape.shared_inter
    rnd = bf16_round if mirror_bf16 else (lambda a: a)
    ids, w, z = route(x, router, shape.top_k, bias, logits_in)

    def ffn(blob, inter, rows):
        wg, wu, wd = q4.expert_matrices(blob, H, inter)
        g = rows @ rnd(wg).T
        v = rows @ rnd(wu).T
        a = rnd(gelu_tanh(g) * v)
        return a @ rnd(wd).T

    y = ffn(shared, Is, x)
    for e in np.unique(ids):
        rows, rank = np.nonzero(ids == e)
        y[rows] += w[rows, rank][:, None] * ffn(experts[e], I, x[rows])
    return {"ids": ids, "w": w, "z": z, "y": y}


# --------------------------------------------------------------------------- byte counts
def layer_bytes(shape) -> dict:
    """Algorithmic bytes one B=1 token moves through one layer."""
    H, I, Is, E, k = shape.hidden, shape.inter, shape.shared_inter, shape.n_experts, shape.top_k
    exp = q4.expert_bytes(H, I)
    return {
        "expert_blob": exp,
        "routed": k * exp,
        "shared": q4.expert_bytes(H, Is),
        "router": E * H * 2,
    }
