"""Pins for the oracle's router: top-k, weights, tie rule, invariants (CPU only)."""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import moe
from synth import gen
from synth.configs import SMALL_LAYER, TINY_LAYER


def test_top_k_matches_stable_library_sort():
    rng = np.random.default_rng(0)
    for _ in range(200):
        z = rng.standard_normal(32)
        assert moe.top_k(z, 8).tolist() == np.argsort(-z, kind="stable")[:8].tolist()


def test_top_k_brute_force_small():
    # the chosen set is the unique k-subset whose min beats the max of the rest
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.standard_normal(7)
        best = [S for S in itertools.combinations(range(7), 3)
                if min(z[list(S)]) > max(np.delete(z, list(S)))]
        assert len(best) == 1
        ids = moe.top_k(z, 3)
        assert sorted(ids.tolist()) == list(best[0])
        assert all(z[ids[i]] >= z[ids[i + 1]] for i in range(2))


def test_ties_go_to_lower_id():
    z = np.zeros(32)
    assert moe.top_k(z, 8).tolist() == list(range(8))
    z = np.array([1.0, 2.0, 2.0, 0.5, 2.0])
    assert moe.top_k(z, 2).tolist() == [1, 2]


def test_weights_sum_to_one_and_equal_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    for _ in range(100):
        z = rng.standard_normal(128) * 3
        ids = moe.top_k(z, 8)
        w = moe.route_weights(z, ids)
        assert abs(w.sum() - 1.0) <= 1e-12
        p = scipy.special.softmax(z)
        ref = p[ids] / p[ids].sum()
        assert np.allclose(w, ref, rtol=1e-12, atol=0)
        assert np.all(np.diff(w) <= 0)   # rank order means non-increasing weights


def test_logits_are_an_fp64_dot_with_bias():
    rng = np.random.default_rng(3)
    u = rng.standard_normal(64)
    wr = rng.normal(0, 0.02, (4, 64)).astype(np.float16)
    b = rng.standard_normal(4).astype(np.float32)
    z = moe.router_logits(u, wr, b)
    for e in range(4):
        ref = sum(float(u[k]) * float(wr[e, k]) for k in range(64)) + float(b[e])
        assert abs(z[e] - ref) < 1e-12


def _tiny_inputs(shape, cid=99):
    return gen.layer_inputs(shape, cid)


def test_zero_input_gives_ids_0_to_k_and_zero_output():
    sh = SMALL_LAYER
    d = _tiny_inputs(sh, 0)
    r = moe.layer_decode(np.zeros(sh.hidden), sh, d["router"], d["shared"], d["experts"])
    assert r["ids"][0].tolist() == list(range(sh.top_k))
    assert np.all(r["w"][0] == 1.0 / sh.top_k)
    assert np.all(r["y"] == 0.0)


def test_relabelling_experts_permutes_ids_and_keeps_output():
    sh = TINY_LAYER
    d = _tiny_inputs(sh)
    rng = np.random.default_rng(4)
    u = rng.standard_normal((3, sh.hidden))
    perm = rng.permutation(sh.n_experts)          # new expert e holds old expert perm[e]
    r0 = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"])
    r1 = moe.layer_decode(u, sh, d["router"][perm], d["shared"], d["experts"][perm])
    inv = np.argsort(perm)
    assert np.array_equal(r1["ids"], inv[r0["ids"]])
    assert np.allclose(r1["y"], r0["y"], rtol=1e-12, atol=1e-12)


def test_grouped_layer_equals_per_token_layer():
    sh = TINY_LAYER
    d = _tiny_inputs(sh)
    u = np.random.default_rng(5).standard_normal((5, sh.hidden))
    a = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"])
    b = moe.layer_decode_per_token(u, sh, d["router"], d["shared"], d["experts"])
    assert np.array_equal(a["ids"], b["ids"])
    assert np.allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("e", [0, 3])
def test_one_hot_logits_reduce_to_one_dense_ffn(e):
    sh = TINY_LAYER
    d = _tiny_inputs(sh)
    u = np.random.default_rng(6).standard_normal((1, sh.hidden))
    logits = np.full((1, sh.n_experts), -1e4)
    logits[0, e] = 0.0
    r = moe.layer_decode(u, sh, d["router"], d["shared"], d["experts"], logits_in=logits)
    assert r["ids"][0, 0] == e and r["w"][0, 0] == 1.0 and np.all(r["w"][0, 1:] == 0.0)
    # independent dense reference: weights decoded by explicit loops, products by numpy BLAS
    from tests.bruteforce import dense_ffn_bruteforce_weights
    ref = dense_ffn_bruteforce_weights(d["shared"], sh.hidden, sh.shared_inter, u[0]) + \
        dense_ffn_bruteforce_weights(d["experts"][e], sh.hidden, sh.inter, u[0])
    assert np.allclose(r["y"][0], ref, rtol=1e-12, atol=1e-12)


def test_weights_stay_finite_for_large_logits():
    # softmax of the selected logits must not overflow (max is subtracted)
    z = np.array([1000.0, 999.0, 998.0, -5.0, 997.0])
    ids = moe.top_k(z, 3)
    w = moe.route_weights(z, ids)
    e = np.exp(np.array([0.0, -1.0, -2.0]))
    assert np.allclose(w, e / e.sum(), rtol=1e-14)
