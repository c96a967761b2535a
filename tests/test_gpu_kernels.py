"""GPU parity of the standalone kernels through the C ABI: unpack, GEMV, router."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import moe, q4
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER
from tests.gpu_util import DEV, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu


def _q4(N, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, (N, K // 32)).astype(np.float16)
    return q, s


def test_unpack_bit_exact_all_bytes():
    q = np.tile(np.arange(256, dtype=np.uint8), (3, 1))  # 3 rows x 512 nibbles
    q = np.concatenate([q, np.random.default_rng(0).integers(0, 256, (61, 256), dtype=np.uint8)])
    out = torch.full((64, 512), -100, dtype=torch.int8, device=DEV)
    api.moe_debug_unpack_q4(dev(q), 64, 512, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), q4.unpack_nibbles(q))


@pytest.mark.parametrize("n16,blocks", [(2 * 1024 * 3 + 5, 2), (1024, 1), (16 * 1024 * 3, 3)])
def test_read_floor_reads_every_word(n16, blocks):
    """Each wave's word is the XOR of the 16-byte words its lanes load (word
    i + j * grid threads for lane i, the last word re-read past the end)."""
    data = np.random.default_rng(n16).integers(0, 2**32, (n16, 4), dtype=np.uint32)
    out = torch.zeros(blocks * 16, dtype=torch.int32, device=DEV)
    api.moe_debug_read_floor(dev(data.view(np.int32)), 16 * n16, blocks, out)
    torch.cuda.synchronize()
    G = blocks * 1024
    L = -(-n16 // G)
    fold = np.bitwise_xor.reduce(data, axis=1)
    idx = np.minimum(np.arange(G)[:, None] + G * np.arange(L)[None, :], n16 - 1)
    want = np.bitwise_xor.reduce(fold[idx], axis=1).reshape(-1, 64)
    want = np.bitwise_xor.reduce(want, axis=1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
    us = api.moe_debug_read_floor(dev(np.tile(data, (3, 1)).view(np.int32)), 16 * n16, blocks, out, region_stride=16 * n16,
                                  regions=3, reps=6, timed=True)
    assert 0.0 < us < 1e5


@pytest.mark.parametrize("N,K,M", [(128, 512, 1), (256, 512, 3), (37, 32, 2), (704, 2816, 1),
                                   (2816, 704, 1), (2816, 2112, 1), (300, 2816, 8), (64, 1024, 17),
                                   (5, 16384, 1),
                                   # the limits: N and K up to 16384, M up to 64 token rows
                                   (16384, 512, 64), (333, 16384, 64), (16384, 16384, 2)])
def test_gemv_q4_against_oracle(N, K, M):
    q, s = _q4(N, K, N * 7 + K)
    x = gen.x_fp32(M, K, 50, sub=N)
    y = poisoned((M, N))
    api.moe_expert_gemv_q4(dev(q), dev_u16(s), N, K, dev(x), M, y)
    torch.cuda.synchronize()
    ref = x.astype(np.float64) @ q4.dequant(q, s).T
    assert_close(y.cpu().numpy(), ref, f"gemv N={N} K={K} M={M}")


def test_gemv_q4_special_inputs():
    N, K = 96, 256
    q, s = _q4(N, K, 3)
    x = np.zeros((4, K), np.float32)
    x[1, 40] = 1.0                          # one element: picks a dequantised column
    x[2, :32] = 1e-30                       # tiny group next to zero groups
    x[3] = np.where(np.arange(K) % 2, 1e4, -1e4).astype(np.float32)  # large magnitudes
    y = poisoned((4, N))
    api.moe_expert_gemv_q4(dev(q), dev_u16(s), N, K, dev(x), 4, y)
    torch.cuda.synchronize()
    g = y.cpu().numpy()
    W = q4.dequant(q, s)
    assert np.all(g[0] == 0.0)
    assert_close(g[1], W[:, 40], "one-hot column")
    assert_close(g[2], x[2].astype(np.float64) @ W.T, "tiny")
    assert_close(g[3], x[3].astype(np.float64) @ W.T, "large")


def mixed_groups(M, K, seed):
    """Rows whose groups of 32 mix magnitudes: one entry of +-1e4 next to
    entries of +-1e-3 in the same group, some groups small only, some zero."""
    rng = np.random.default_rng(seed)
    x = (rng.choice([-1.0, 1.0], (M, K)) * rng.uniform(0.5, 1.5, (M, K)) * 1e-3).astype(np.float32)
    g = K // 32
    for m in range(M):
        for j in range(g):
            kind = (m + j) % 4
            if kind == 0 or kind == 1:                       # one large entry among small ones
                x[m, 32 * j + rng.integers(0, 32)] = rng.choice([-1.0, 1.0]) * 1e4
            elif kind == 2:                                  # two large of opposite sign
                i0, i1 = rng.choice(32, 2, replace=False)
                x[m, 32 * j + i0], x[m, 32 * j + i1] = 1e4, -7.5e3
            # kind 3: the group stays at 1e-3
        x[m, :32] = 0.0                                      # one all-zero group
    return x


@pytest.mark.parametrize("N,K,M", [(704, 2816, 1), (2816, 704, 1), (96, 256, 4)])
def test_gemv_q4_mixed_magnitudes_in_a_group(N, K, M):
    q, s = _q4(N, K, N + K)
    x = mixed_groups(M, K, N)
    y = poisoned((M, N))
    api.moe_expert_gemv_q4(dev(q), dev_u16(s), N, K, dev(x), M, y)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), x.astype(np.float64) @ q4.dequant(q, s).T, f"mixed N={N} K={K}")


def test_gemv_q4_deterministic():
    N, K = 2816, 2112
    q, s = _q4(N, K, 9)
    x = dev(gen.x_fp32(1, K, 51))
    a, b = poisoned((1, N)), poisoned((1, N))
    qd, sd = dev(q), dev_u16(s)
    api.moe_expert_gemv_q4(qd, sd, N, K, x, 1, a)
    api.moe_expert_gemv_q4(qd, sd, N, K, x, 1, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape,B", [(SMALL_LAYER, 1), (SMALL_LAYER, 9), (GEMMA_LAYER, 1),
                                     (GEMMA_LAYER, 64)])
def test_route_ids_bit_exact(shape, B):
    cid = 0 if shape is SMALL_LAYER else 1
    wr = gen.router(shape, cid)
    x = gen.x_fp32(B, shape.hidden, cid, sub=B)
    bias = gen.zipf_bias(shape.n_experts, 2, 0)
    for use_bias in (False, True):
        ids = poisoned((B, shape.top_k), torch.int32)
        w = poisoned((B, shape.top_k))
        ws = torch.empty(api.moe_route_workspace_bytes(shape, B), dtype=torch.uint8, device=DEV)
        api.moe_route(shape, dev(x), dev_u16(wr), dev(bias) if use_bias else None, None, B, ids, w, ws)
        torch.cuda.synchronize()
        r_ids, r_w, _ = moe.route(x.astype(np.float64), wr, shape.top_k, bias if use_bias else None)
        assert np.array_equal(ids.cpu().numpy(), r_ids)
        assert_close(w.cpu().numpy(), r_w, "w")
        assert np.allclose(w.cpu().numpy().sum(1), 1.0, atol=1e-6)


def test_route_given_logits_and_ties():
    sh = GEMMA_LAYER
    T = 2048
    logits = gen.logits_uniform(T, sh.n_experts, 4)
    logits[0] = 0.0                              # all tied: ids 0..7, w = 1/8
    logits[1, 5] = logits[1, 9] = 2.0            # a tie at the top goes to the lower id
    logits[2] = -1.0                             # -0.0 and +0.0 are equal: ties by id
    logits[2, 12], logits[2, 7], logits[2, 3] = -0.0, 0.0, -0.0
    logits[3] = -3.5                             # negative ties, one larger value
    logits[3, 40] = -2.0
    ids = poisoned((T, sh.top_k), torch.int32)
    w = poisoned((T, sh.top_k))
    api.moe_route(sh, None, None, None, dev(logits), T, ids, w, None)
    torch.cuda.synchronize()
    r_ids, r_w, _ = moe.route(None, None, sh.top_k, logits_in=logits)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert ids[0].tolist() == list(range(8)) and torch.all(w[0] == 0.125)
    assert ids[1, :2].tolist() == [5, 9]
    assert ids[2].tolist() == [3, 7, 12, 0, 1, 2, 4, 5]
    assert ids[3].tolist() == [40, 0, 1, 2, 3, 4, 5, 6]
    assert_close(w.cpu().numpy(), r_w, "w")


def _order_with_nonfinite(z, k):
    """Rank order of one token's logits as the library takes it for non-finite
    values: +inf above every number, NaN below every number (-inf included),
    -0 equal to +0, ties to the lower id. The oracle is not defined on
    non-finite logits; this is the property the ids must have."""
    def key(e):
        v = z[e]
        if np.isnan(v):
            return (0, 0.0, e)
        return (1, -float(v) if v != 0 else 0.0, e)
    order = sorted(range(len(z)), key=lambda e: (-key(e)[0], key(e)[1], e))
    return order[:k]


def test_route_nonfinite_logits_give_valid_ids():
    sh = GEMMA_LAYER
    T = 6
    logits = gen.logits_uniform(T, sh.n_experts, 8)
    logits[0] = np.nan                                  # all NaN: ids 0..7
    logits[1, 3] = np.inf                               # +inf first, NaNs never chosen
    logits[1, 0:3] = np.nan
    logits[2, ::2] = np.nan                             # half NaN: the top 8 odd experts
    logits[3, 10] = -np.inf                             # -inf below every finite value
    logits[3, :] = np.where(np.arange(sh.n_experts) == 10, -np.inf, -1e30)
    logits[4, 50] = np.inf                              # two +inf: the lower id first
    logits[4, 20] = np.inf
    logits[5] = -np.inf                                 # all -inf: ids 0..7
    ids = poisoned((T, sh.top_k), torch.int32)
    w = poisoned((T, sh.top_k))
    api.moe_route(sh, None, None, None, dev(logits), T, ids, w, None)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(T):
        assert got[t].tolist() == _order_with_nonfinite(logits[t], sh.top_k), t
        assert len(set(got[t].tolist())) == sh.top_k and got[t].min() >= 0 and got[t].max() < sh.n_experts
