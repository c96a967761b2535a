"""Seeded generators for every input of the MoE layer workloads.

Every tensor is drawn from its own numpy stream,
``Generator(PCG64(SeedSequence([seed, config_id, tag, *sub])))`` with seed 0,
so a tensor is reproducible on its own and independent of draw order.

Storage formats produced here (both sides read them, neither side shares
code with this module):

* int4 g32 matrix for y = x.W with W logically K x N: ``q`` uint8 [N][K/2]
  (byte j of a row holds element 2j in bits 0-3 and 2j+1 in bits 4-7, each a
  4-bit two's-complement value in -8..7) and ``s`` fp16 [N][K/32] (one scale
  per 32 consecutive K elements). Uniform random bytes give uniform nibbles.
* expert blob, one contiguous byte run per expert:
  ``gate.q [I][H/2] | up.q [I][H/2] | down.q [H][I/2] | gate.s [I][H/32] |
  up.s [I][H/32] | down.s [H][I/32]``, 27*H*I/16 bytes.

The pages fix only "4 bits" and a per-expert byte size near 3.36 MB
("Show HN: mecanismo de código aberto executando Gemma 4 26B em 2 GB de RAM",
section "Abordagem técnica"); everything else above is this project's reading.
"""
from __future__ import annotations

import numpy as np

from .configs import AttnShape, Shape

SEED = 0

# Stream tags, one per tensor family.
TAG_X = 1
TAG_ROUTER = 2
TAG_EXPERT_BYTES = 3
TAG_EXPERT_SCALES = 4
TAG_SHARED_BYTES = 5
TAG_SHARED_SCALES = 6
TAG_EPS = 7
TAG_ZIPF = 8
TAG_LOGITS = 9
TAG_X_BF16 = 10
TAG_ATTN_NORM = 11
TAG_ATTN_QKV_BYTES = 12
TAG_ATTN_QKV_SCALES = 13
TAG_ATTN_O_BYTES = 14
TAG_ATTN_O_SCALES = 15
TAG_KV = 16

SCALE_LO, SCALE_HI = 0.005, 0.02
ROUTER_STD = 0.02


def stream(config_id: int, tag: int, *sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, config_id, tag, *sub])))


# --------------------------------------------------------------------------- layout
def blob_layout(hidden: int, inter: int, group: int = 32) -> dict:
    """Byte offsets and sizes of the six sub-arrays of one expert blob."""
    H, I = hidden, inter
    parts = [
        ("gate_q", I * H // 2), ("up_q", I * H // 2), ("down_q", H * I // 2),
        ("gate_s", I * (H // group) * 2), ("up_s", I * (H // group) * 2),
        ("down_s", H * (I // group) * 2),
    ]
    out, off = {}, 0
    for name, n in parts:
        out[name] = (off, n)
        off += n
    out["total"] = off
    return out


def blob_bytes(hidden: int, inter: int, group: int = 32) -> int:
    return blob_layout(hidden, inter, group)["total"]


def pack_nibbles(v: np.ndarray) -> np.ndarray:
    """Encode int values in -8..7, shape [N][K], into packed bytes [N][K/2]."""
    v = np.asarray(v)
    if v.min(initial=0) < -8 or v.max(initial=0) > 7:
        raise ValueError("nibble values must lie in -8..7")
    u = (v.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def assemble_blob(hidden, inter, gate_q, gate_s, up_q, up_s, down_q, down_s, group=32) -> np.ndarray:
    """Place the six arrays of one expert at their layout offsets."""
    lay = blob_layout(hidden, inter, group)
    blob = np.zeros(lay["total"], np.uint8)
    for name, arr in (("gate_q", gate_q), ("up_q", up_q), ("down_q", down_q),
                      ("gate_s", gate_s), ("up_s", up_s), ("down_s", down_s)):
        off, n = lay[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        if raw.size != n:
            raise ValueError(f"{name}: {raw.size} bytes, layout wants {n}")
        blob[off:off + n] = raw
    return blob


# --------------------------------------------------------------------------- weights
def fill_blobs(out: np.ndarray, hidden: int, inter: int, config_id: int,
               byte_tag: int, scale_tag: int, *sub: int, group: int = 32) -> np.ndarray:
    """Fill ``out`` (uint8 [n][blob]) with random nibbles and U(0.005,0.02) fp16 scales."""
    lay = blob_layout(hidden, inter, group)
    n = out.shape[0]
    assert out.shape == (n, lay["total"]) and out.dtype == np.uint8
    out.reshape(-1)[:] = np.frombuffer(stream(config_id, byte_tag, *sub).bytes(out.size), np.uint8)
    s0 = lay["gate_s"][0]
    n_scales = (lay["total"] - s0) // 2
    sc = stream(config_id, scale_tag, *sub).uniform(SCALE_LO, SCALE_HI, size=(n, n_scales))
    out[:, s0:] = sc.astype(np.float16).view(np.uint8)
    return out


def expert_blobs(shape: Shape, config_id: int, layer: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    nb = blob_bytes(shape.hidden, shape.inter, shape.group)
    if out is None:
        out = np.empty((shape.n_experts, nb), np.uint8)
    return fill_blobs(out, shape.hidden, shape.inter, config_id, TAG_EXPERT_BYTES, TAG_EXPERT_SCALES,
                      layer, group=shape.group)


def shared_blob(shape: Shape, config_id: int, layer: int = 0) -> np.ndarray:
    nb = blob_bytes(shape.hidden, shape.shared_inter, shape.group)
    out = np.empty((1, nb), np.uint8)
    fill_blobs(out, shape.hidden, shape.shared_inter, config_id, TAG_SHARED_BYTES, TAG_SHARED_SCALES,
               layer, group=shape.group)
    return out[0]


def router(shape: Shape, config_id: int, layer: int = 0) -> np.ndarray:
    """fp16 [E][H], N(0, 0.02) drawn in fp64 and rounded to nearest-even fp16."""
    r = stream(config_id, TAG_ROUTER, layer).normal(0.0, ROUTER_STD, size=(shape.n_experts, shape.hidden))
    return r.astype(np.float16)


# --------------------------------------------------------------------------- activations
def x_fp32(rows: int, hidden: int, config_id: int, sub: int = 0) -> np.ndarray:
    return stream(config_id, TAG_X, sub).standard_normal((rows, hidden), dtype=np.float32)


def eps_fp16(layers: int, tokens: int, hidden: int, config_id: int, std: float = 0.1) -> np.ndarray:
    """Residual perturbation standing in for attention: N(0, std) in fp32, rounded to fp16."""
    out = np.empty((layers, tokens, hidden), np.float16)
    for l in range(layers):
        z = stream(config_id, TAG_EPS, l).standard_normal((tokens, hidden), dtype=np.float32)
        out[l] = (z * np.float32(std)).astype(np.float16)
    return out


def zipf_bias(n_experts: int, config_id: int, layer: int, s: float = 1.1) -> np.ndarray:
    """Per-layer popularity prior: log p of a seeded rank permutation, p_r ~ r^-s."""
    ranks = stream(config_id, TAG_ZIPF, layer).permutation(n_experts) + 1
    p = np.arange(1, n_experts + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return np.log(p[ranks - 1]).astype(np.float32)


def logits_uniform(tokens: int, n_experts: int, config_id: int) -> np.ndarray:
    return stream(config_id, TAG_LOGITS).random((tokens, n_experts), dtype=np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns with round-to-nearest-even (finite inputs)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def x_bf16(tokens: int, hidden: int, config_id: int) -> np.ndarray:
    z = stream(config_id, TAG_X_BF16).standard_normal((tokens, hidden), dtype=np.float32)
    return to_bf16_bits(z)


# --------------------------------------------------------------------------- bundles
def layer_inputs(shape: Shape, config_id: int, layer: int = 0) -> dict:
    """Router, shared blob and all expert blobs of one layer."""
    return {
        "router": router(shape, config_id, layer),
        "shared": shared_blob(shape, config_id, layer),
        "experts": expert_blobs(shape, config_id, layer),
    }


# --------------------------------------------------------------------------- attention step
def q4_matrix(rows: int, cols: int, config_id: int, byte_tag: int, scale_tag: int, *sub: int,
              group: int = 32):
    """int4 g32 matrix [rows][cols]: uniform random nibbles (uint8 [rows][cols/2])
    and U(0.005, 0.02) fp16 scales [rows][cols/32], as for the experts."""
    q = np.frombuffer(stream(config_id, byte_tag, *sub).bytes(rows * cols // 2), np.uint8).reshape(rows, cols // 2)
    s = stream(config_id, scale_tag, *sub).uniform(SCALE_LO, SCALE_HI, size=(rows, cols // group))
    return q.copy(), s.astype(np.float16)


def attn_weights(a: AttnShape, config_id: int, layer: int = 0) -> dict:
    """Weights of one attention step: RMSNorm weight fp32 [H] = 1 + N(0, 0.1);
    the fused projection [q rows | k rows | v rows] x H and the output
    projection H x (n_heads * d), both int4 g32."""
    norm_w = (1.0 + 0.1 * stream(config_id, TAG_ATTN_NORM, layer).standard_normal(a.hidden)).astype(np.float32)
    qkv_q, qkv_s = q4_matrix(a.qkv_rows, a.hidden, config_id, TAG_ATTN_QKV_BYTES, TAG_ATTN_QKV_SCALES, layer)
    o_q, o_s = q4_matrix(a.hidden, a.attn_width, config_id, TAG_ATTN_O_BYTES, TAG_ATTN_O_SCALES, layer)
    return {"norm_w": norm_w, "qkv_q": qkv_q, "qkv_s": qkv_s, "o_q": o_q, "o_s": o_s}


def kv_cache(a: AttnShape, n_filled: int, config_id: int, layer: int = 0):
    """fp16 K and V caches [n_kv_heads][max_ctx][d]: positions < n_filled hold
    N(0, 1) values (the keys and values of earlier tokens), the rest zero."""
    k = np.zeros((a.n_kv_heads, a.max_ctx, a.head_dim), np.float16)
    v = np.zeros_like(k)
    r = stream(config_id, TAG_KV, layer)
    k[:, :n_filled] = r.standard_normal((a.n_kv_heads, n_filled, a.head_dim)).astype(np.float16)
    v[:, :n_filled] = r.standard_normal((a.n_kv_heads, n_filled, a.head_dim)).astype(np.float16)
    return k, v
