"""Pins for the attention-step oracle (CPU only): RMSNorm, RoPE, grouped-query
attention over the fp16 cache and the whole step, against closed forms,
invariants and explicit loops."""
import math

import numpy as np
import pytest

from oracle import attn
from synth import gen
from synth.configs import GEMMA_ATTN, SMALL_ATTN, TINY_ATTN
from tests import bruteforce as bf


def test_rmsnorm_weighted_hand_example():
    y = attn.rmsnorm_weighted([3.0, 4.0], [2.0, 0.5], eps=0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [3 / r * 2, 4 / r * 0.5], rtol=1e-15)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = np.random.default_rng(1).standard_normal(300)
    y = attn.rmsnorm_weighted(x, np.ones(300), eps=0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-13
    assert np.allclose(attn.rmsnorm_weighted(7.5 * x, np.ones(300), eps=0.0), y, rtol=1e-13)
    w = np.random.default_rng(2).standard_normal(300)
    assert np.allclose(attn.rmsnorm_weighted(x, w, eps=0.0), y * w, rtol=1e-13)


def test_rope_position_zero_is_identity():
    v = np.random.default_rng(3).standard_normal((3, 16))
    assert np.array_equal(attn.rope(v, 0), v)


@pytest.mark.parametrize("p", [1, 5, 123])
def test_rope_single_pair_closed_form(p):
    # d = 2: one pair rotated by p radians (theta^0 = 1)
    assert np.allclose(attn.rope([1.0, 0.0], p), [math.cos(p), math.sin(p)], atol=1e-15)
    assert np.allclose(attn.rope([0.0, 1.0], p), [-math.sin(p), math.cos(p)], atol=1e-15)


def test_rope_pairs_and_frequencies():
    # d = 4, theta = 10^4: pairs (0, 2) at p rad and (1, 3) at p / 100 rad
    p = 37
    assert np.allclose(attn.rope([0.0, 1.0, 0.0, 0.0], p), [0, math.cos(p / 100), 0, math.sin(p / 100)],
                       atol=1e-15)
    assert np.allclose(attn.rope([1.0, 0.0, 0.0, 0.0], p), [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    assert np.allclose(attn.rope([0.0, 1.0, 0.0, 0.0], p, theta=100.0), [0, math.cos(p / 10), 0, math.sin(p / 10)],
                       atol=1e-15)


def test_rope_keeps_pair_norms_and_depends_on_relative_position():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    r = attn.rope(q, 900)
    assert np.allclose(r[:32] ** 2 + r[32:] ** 2, q[:32] ** 2 + q[32:] ** 2, rtol=1e-12)
    for m, n in ((900, 13), (50, 50), (7, 0)):
        assert math.isclose(attn.rope(q, m) @ attn.rope(k, n), attn.rope(q, m - n) @ k, rel_tol=1e-10,
                            abs_tol=1e-10)


def _caches(nkv, n, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((nkv, n, d)).astype(np.float16),
            rng.standard_normal((nkv, n, d)).astype(np.float16))


def test_attention_one_position_returns_its_value_per_group():
    kc, vc = _caches(2, 4, 8, 5)
    q = np.random.default_rng(6).standard_normal((4, 8))
    a = attn.attention(q, kc, vc, 1)
    # heads 0, 1 read group 0; heads 2, 3 read group 1
    assert np.array_equal(a[0], vc[0, 0].astype(np.float64)) and np.array_equal(a[1], vc[0, 0])
    assert np.array_equal(a[2], vc[1, 0].astype(np.float64)) and np.array_equal(a[3], vc[1, 0])


def test_attention_equal_keys_average_values():
    kc, vc = _caches(1, 6, 8, 7)
    kc[0, :] = kc[0, 0]
    a = attn.attention(np.random.default_rng(8).standard_normal((1, 8)), kc, vc, 6)
    assert np.allclose(a[0], vc[0].astype(np.float64).mean(axis=0), rtol=1e-13)


def test_attention_two_keys_closed_form():
    d, t = 16, 3.0
    kc = np.zeros((1, 2, d), np.float16)
    kc[0, 0, 0] = 1.0
    vc = np.zeros((1, 2, d), np.float16)
    vc[0, 0, :] = 2.0
    vc[0, 1, :] = -1.0
    q = np.zeros((1, d))
    q[0, 0] = t
    sig = 1.0 / (1.0 + math.exp(-t / math.sqrt(d)))
    assert np.allclose(attn.attention(q, kc, vc, 2)[0], sig * 2.0 + (1 - sig) * -1.0, rtol=1e-14)


def test_attention_ignores_positions_past_the_context():
    kc, vc = _caches(2, 10, 8, 9)
    q = np.random.default_rng(10).standard_normal((4, 8))
    a = attn.attention(q, kc, vc, 6)
    kc[:, 6:] = 1000.0
    vc[:, 6:] = -1000.0
    assert np.array_equal(attn.attention(q, kc, vc, 6), a)


@pytest.mark.parametrize("pos", [0, 3, 5])
def test_decode_step_matches_explicit_loops(pos):
    a = TINY_ATTN
    w = gen.attn_weights(a, 0)
    kc, vc = gen.kv_cache(a, pos, 0)
    kc2, vc2 = kc.copy(), vc.copy()
    x = gen.x_fp32(1, a.hidden, 0, sub=pos)[0]
    r = attn.decode_step(x, w, kc, vc, pos, a)
    y = bf.attn_step_loops(x, w, kc2, vc2, pos, a.n_heads, a.n_kv_heads, a.head_dim, a.rope_theta, a.eps)
    assert np.allclose(r["y"], y, rtol=1e-11, atol=1e-11)
    # the cache entries are the fp16 roundings of the same key and value
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)


def test_decode_step_writes_only_its_position_and_zero_projection_is_identity():
    a = SMALL_ATTN
    w = gen.attn_weights(a, 0)
    w["o_s"] = np.zeros_like(w["o_s"])
    kc, vc = gen.kv_cache(a, 20, 0)
    k0, v0 = kc.copy(), vc.copy()
    x = gen.x_fp32(1, a.hidden, 0)[0]
    r = attn.decode_step(x, w, kc, vc, 20, a)
    assert np.array_equal(r["y"], x.astype(np.float64))
    changed = np.nonzero(np.any(kc != k0, axis=(0, 2)) | np.any(vc != v0, axis=(0, 2)))[0]
    assert list(changed) == [20]
    assert np.array_equal(kc[:, 20], r["k"].astype(np.float16))
    with pytest.raises(ValueError):
        attn.decode_step(x, w, kc, vc, a.max_ctx, a)


def test_step_bytes_closed_form():
    b = attn.step_bytes(GEMMA_ATTN, 4096)
    assert b["qkv"] == 8192 * (1408 + 176) == 12_976_128
    assert b["o"] == 2816 * (2048 + 256) == 6_488_064
    assert b["kv"] == 2 * 8 * 4096 * 256 * 2 == 33_554_432
