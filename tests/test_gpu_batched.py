"""GPU parity of batched decode (tokens grouped by expert, matrix-core products) against the
per-token oracle."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import moe
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER, TINY_LAYER, Shape
from tests.gpu_util import Layer, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu

_CACHE = {}


def layer_data(shape, cid):
    if (shape, cid) not in _CACHE:
        _CACHE[(shape, cid)] = gen.layer_inputs(shape, cid)
    return _CACHE[(shape, cid)]


def decode(L, x, flags=0, add_in=None):
    B = x.shape[0]
    sh = L.shape
    y = poisoned((B, sh.hidden))
    ids = poisoned((B, sh.top_k), torch.int32)
    w = poisoned((B, sh.top_k))
    u = poisoned((B, sh.hidden))
    api.moe_layer_decode(L.h, dev(x), add_in, B, flags, y, ids, w, u)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), u.cpu().numpy()


# B covers one ragged token tile (5, 7), exactly one tile (16), two and four
# tiles per pass (33, 64) and a shared segment of more than 64 tokens, which
# takes two passes over the weights (100), and 160 tokens (1280 assignments:
# top-k and sort in separate launches instead of one block); the tiny shape has K tails (2 of the
# 4 groups of a step are past K) and idle waves (32 rows per block of 64)
@pytest.mark.parametrize("shape,cid,B", [(SMALL_LAYER, 0, 5), (SMALL_LAYER, 0, 16), (SMALL_LAYER, 0, 100), (SMALL_LAYER, 0, 160),
                                         (TINY_LAYER, 99, 7), (GEMMA_LAYER, 3, 16), (GEMMA_LAYER, 3, 33),
                                         (GEMMA_LAYER, 3, 64)])
def test_batched_decode_matches_per_token_oracle(shape, cid, B):
    d = layer_data(shape, cid)
    L = Layer(shape, d, max_B=B)
    x = gen.x_fp32(B, shape.hidden, cid, sub=B)
    y, ids, w, u = decode(L, x)
    r = moe.layer_decode(x.astype(np.float64), shape, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids, r["ids"])
    assert_close(w, r["w"], "w")
    assert_close(y, r["y"], f"y B={B}")
    assert np.array_equal(u, x)
    # every token's row matches a B=1 call of the same token: the routing is
    # identical; the arithmetic differs (fp16 matrix-core products here, 16-bit
    # digit planes at B=1), so the two agree to the oracle bar
    L1 = Layer(shape, d)
    for t in (0, B - 1):
        y1, ids1, _, _ = decode(L1, x[t:t + 1])
        assert np.array_equal(ids1[0], ids[t])
        assert_close(y[t], y1[0], "batched vs single")
    # same inputs, same bits
    y2, _, _, _ = decode(L, x)
    assert np.array_equal(y, y2)
    L.close()
    L1.close()


# Every token is one input row times a power of two: the logits scale with it,
# so every token picks the same k experts (the weights differ), and each of
# them serves all B tokens, more than one 16-token pass of its blocks (small
# layer B = 32: two passes; Gemma layer B = 64: four).
@pytest.mark.parametrize("shape,cid,B", [(SMALL_LAYER, 0, 32), (GEMMA_LAYER, 3, 64)])
def test_batched_all_tokens_on_the_same_experts(shape, cid, B):
    d = layer_data(shape, cid)
    L = Layer(shape, d, max_B=B)
    row = gen.x_fp32(1, shape.hidden, cid, sub=5)[0]
    x = np.stack([row * np.float32(2.0 ** (t % 7 - 3)) for t in range(B)]).astype(np.float32)
    y, ids, w, _ = decode(L, x)
    r = moe.layer_decode(x.astype(np.float64), shape, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids, r["ids"])
    assert all(np.array_equal(ids[t], ids[0]) for t in range(B))
    assert_close(w, r["w"], "w")
    for t in range(B):  # each row at its own scale
        assert_close(y[t], r["y"][t], f"y B={B} token {t}")
    L.close()


def test_batched_norm_residual_perturbation():
    sh = GEMMA_LAYER
    d = layer_data(sh, 3)
    bias = gen.zipf_bias(sh.n_experts, 3, 0)
    B = 16
    L = Layer(sh, d, bias=bias, max_B=B)
    x = gen.x_fp32(B, sh.hidden, 3, sub=99)
    eps = gen.eps_fp16(1, B, sh.hidden, 3)[0]
    y, ids, w, u = decode(L, x, api.MOE_F_RMSNORM_IN | api.MOE_F_RESIDUAL, add_in=dev_u16(eps))
    lay = dict(d, bias=bias)
    h2, rec = moe.stack_layer_step(x, eps, sh, lay)
    assert_close(u, rec["u"], "u")
    r_ids, _, _ = moe.route(u.astype(np.float64), d["router"], sh.top_k, bias)
    assert np.array_equal(ids, r_ids)
    assert_close(y, h2, "y")
    L.close()


def test_batched_zero_input():
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    L = Layer(sh, d, max_B=4)
    y, ids, w, _ = decode(L, np.zeros((4, sh.hidden), np.float32))
    assert np.all(y == 0.0)
    assert all(row.tolist() == list(range(8)) for row in ids)
    L.close()


@pytest.mark.parametrize("scale", [3e4, 1e-3])
def test_batched_input_scale(scale):
    """Without RMSNorm the fp16 staging sees the raw input: a per-token power of
    two keeps it in range for very large and very small magnitudes."""
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    B = 8
    L = Layer(sh, d, max_B=B)
    x = (gen.x_fp32(B, sh.hidden, 0, sub=7) * scale).astype(np.float32)
    y, ids, w, _ = decode(L, x)
    r = moe.layer_decode(x.astype(np.float64), sh, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids, r["ids"])
    assert_close(y, r["y"], f"y scale={scale}")
    L.close()


# K above 4096 (the scales of a block's rows staged in more than one batch,
# above 64 KiB of LDS per block): hidden 8192 (gate/up K = 8192, 128 KiB of
# staged scales at 34 KiB of slices for B above 32) and a down projection of
# K = 4608 (inter) and 4160 (shared_inter), with ragged and full token tiles.
LARGE_K = [Shape(hidden=8192, n_experts=8, top_k=2, inter=64, shared_inter=96),
           Shape(hidden=256, n_experts=8, top_k=2, inter=4608, shared_inter=4160)]


@pytest.mark.parametrize("shape,B", [(LARGE_K[0], 5), (LARGE_K[0], 40), (LARGE_K[1], 7), (LARGE_K[1], 33)],
                         ids=["H8192-B5", "H8192-B40", "I4608-B7", "I4608-B33"])
def test_batched_decode_large_k(shape, B):
    d = layer_data(shape, 11)
    print(f"batched large K: H={shape.hidden} I={shape.inter} Is={shape.shared_inter} B={B}", flush=True)
    L = Layer(shape, d, max_B=B)
    x = gen.x_fp32(B, shape.hidden, 11, sub=B)
    y, ids, w, _ = decode(L, x)
    r = moe.layer_decode(x.astype(np.float64), shape, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids, r["ids"])
    assert_close(w, r["w"], "w")
    assert_close(y, r["y"], f"y B={B}")
    L.close()


# The largest batch a handle takes (max_B = 4096): 32768 assignments, 1024
# tokens per routed expert on average (16 passes of 64 over each block's
# rows) and a shared segment of 4096 tokens.
def test_batched_decode_max_batch():
    shape, B = SMALL_LAYER, 4096
    d = layer_data(shape, 0)
    L = Layer(shape, d, max_B=B)
    x = gen.x_fp32(B, shape.hidden, 0, sub=B)
    y, ids, w, u = decode(L, x)
    r = moe.layer_decode(x.astype(np.float64), shape, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids, r["ids"])
    assert_close(w, r["w"], "w")
    assert_close(y, r["y"], f"y B={B}")
    assert np.array_equal(u, x)
    L.close()
