"""Pins for the oracle's GELU, GeGLU FFN, combine and stack (CPU only)."""
import math

import numpy as np
import scipy.special

from oracle import moe
from synth import gen
from synth.configs import SMALL_LAYER, TINY_LAYER
from tests import bruteforce as bf


def test_gelu_tanh_within_published_bound_of_exact_gelu():
    # the tanh form differs from x*Phi(x) by at most ~4.7e-4 over the real line
    x = np.linspace(-12, 12, 200001)
    exact = x * scipy.special.ndtr(x)
    assert np.max(np.abs(moe.gelu_tanh(x) - exact)) < 5e-4
    assert moe.gelu_tanh(0.0) == 0.0


def test_gelu_tanh_odd_part_identity():
    # gelu(x) - gelu(-x) = x for the tanh form (tanh is odd)
    x = np.random.default_rng(0).standard_normal(1000) * 4
    assert np.allclose(moe.gelu_tanh(x) - moe.gelu_tanh(-x), x, rtol=1e-13, atol=1e-13)


def _structured_blob(H, I, perm_g, perm_u, perm_d):
    """Blob whose gate/up/down rows each hold a single effective weight of 1.

    Row n of gate has its one nonzero at column perm_g[n]; the nibble there is
    2^(g%3) and the scale of that group is 2^-(g%3), so the product is 1 only
    if dequant uses the scale of the right group.
    """
    def mat(rows, cols, perm):
        v = np.zeros((rows, cols), np.int8)
        s = np.full((rows, cols // 32), 0.0078125, np.float16)
        for r in range(rows):
            c = perm[r]
            if c < 0:
                continue
            gidx = c // 32
            v[r, c] = 2 ** (gidx % 3)
            s[r, gidx] = 2.0 ** -(gidx % 3)
            # a different scale in the neighbouring groups
            for g2 in range(cols // 32):
                if g2 != gidx:
                    s[r, g2] = 2.0 ** -((gidx + 1) % 3 + 3)
        return gen.pack_nibbles(v), s
    gq, gs = mat(I, H, perm_g)
    uq, us = mat(I, H, perm_u)
    dq, ds = mat(H, I, perm_d)
    return gen.assemble_blob(H, I, gq, gs, uq, us, dq, ds)


def test_structured_expert_closed_form():
    H, I = 128, 64
    rng = np.random.default_rng(1)
    pg = rng.permutation(H)[:I]
    pu = rng.permutation(H)[:I]
    pd = np.array([rng.integers(0, I) if h % 3 else -1 for h in range(H)])
    blob = _structured_blob(H, I, pg, pu, pd)
    u = rng.standard_normal(H)
    y = moe.expert_ffn(blob, H, I, u)
    a = np.array([bf.gelu_tanh_scalar(u[pg[i]]) * u[pu[i]] for i in range(I)])
    ref = np.array([a[pd[h]] if pd[h] >= 0 else 0.0 for h in range(H)])
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-14)


def test_tiny_layer_against_explicit_loops():
    sh = TINY_LAYER
    d = gen.layer_inputs(sh, 99)
    bias = gen.zipf_bias(sh.n_experts, 99, 0)
    rng = np.random.default_rng(2)
    for t in range(3):
        u = rng.standard_normal(sh.hidden)
        r = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"], bias=bias)
        ids, w, y = bf.layer_loops(u, sh.n_experts, sh.top_k, sh.hidden, sh.inter, sh.shared_inter,
                                   d["router"], d["shared"], d["experts"], bias=bias)
        assert r["ids"][0].tolist() == ids
        assert np.allclose(r["w"][0], w, rtol=1e-12, atol=0)
        assert np.allclose(r["y"][0], y, rtol=1e-11, atol=1e-12)


def test_small_layer_one_hot_against_bruteforce_weights():
    sh = SMALL_LAYER
    d = gen.layer_inputs(sh, 0)
    u = gen.x_fp32(1, sh.hidden, 0)[0].astype(np.float64)
    e = 17
    logits = np.full((1, sh.n_experts), -1e4)
    logits[0, e] = 0.0
    r = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"], logits_in=logits)
    ref = bf.dense_ffn_bruteforce_weights(d["shared"], sh.hidden, sh.shared_inter, u) + \
        bf.dense_ffn_bruteforce_weights(d["experts"][e], sh.hidden, sh.inter, u)
    assert np.allclose(r["y"][0], ref, rtol=1e-12, atol=1e-12)


def test_residual_adds_the_input():
    sh = TINY_LAYER
    d = gen.layer_inputs(sh, 99)
    u = np.random.default_rng(3).standard_normal((2, sh.hidden))
    res = np.random.default_rng(4).standard_normal((2, sh.hidden))
    a = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"])
    b = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"], residual=res)
    assert np.array_equal(b["y"], a["y"] + res)


def test_rmsnorm_closed_form():
    x = np.random.default_rng(5).standard_normal((4, 256)) * 3
    u = moe.rmsnorm(x, 1e-6)
    m = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(u * u, axis=1), m / (m + 1e-6), rtol=1e-13, atol=0)
    # direction is kept: u is a positive multiple of x
    assert np.allclose(u / x, (u / x)[:, :1], rtol=1e-12)


def test_stack_with_zero_weights_is_sum_of_perturbations():
    sh = TINY_LAYER
    L = 4
    zero_blob = np.zeros(gen.blob_bytes(sh.hidden, sh.inter), np.uint8)
    layers = []
    for l in range(L):
        layers.append({
            "router": gen.router(sh, 99, l),
            "bias": gen.zipf_bias(sh.n_experts, 99, l),
            "shared": np.zeros(gen.blob_bytes(sh.hidden, sh.shared_inter), np.uint8),
            "experts": np.stack([zero_blob] * sh.n_experts),
        })
    x0 = gen.x_fp32(1, sh.hidden, 99)
    eps = gen.eps_fp16(L, 1, sh.hidden, 99)[:, 0]
    h, recs = moe.stack_decode(x0, eps, sh, layers)
    ref = x0.astype(np.float64) + eps.astype(np.float64).sum(axis=0)
    assert np.allclose(h, ref, rtol=1e-15, atol=1e-15)
    assert len(recs) == L and all(r["ids"].shape == (1, sh.top_k) for r in recs)


def test_stack_layer_feeds_the_normalised_input():
    sh = TINY_LAYER
    d = gen.layer_inputs(sh, 99)
    d["bias"] = gen.zipf_bias(sh.n_experts, 99, 0)
    h = gen.x_fp32(1, sh.hidden, 99)
    eps = gen.eps_fp16(1, 1, sh.hidden, 99)[0]
    h2, r = moe.stack_layer_step(h, eps, sh, d)
    hp = h.astype(np.float64) + eps.astype(np.float64)
    u = hp / math.sqrt(float(np.mean(hp * hp)) + 1e-6)
    ref = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"], bias=d["bias"])
    assert np.allclose(h2, hp + ref["y"], rtol=1e-13, atol=1e-13)
