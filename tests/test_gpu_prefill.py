"""GPU parity of moe_layer_prefill (bf16 MFMA grouped GEMM) against the mirrored oracle."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu, moe
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER, Shape
from tests.gpu_util import DEV, Layer, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu

_CACHE = {}


def layer_data(shape, cid):
    if (shape, cid) not in _CACHE:
        _CACHE[(shape, cid)] = gen.layer_inputs(shape, cid)
    return _CACHE[(shape, cid)]


def run_prefill(L, xb, logits, T):
    sh = L.shape
    y = poisoned((T, sh.hidden))
    ids = poisoned((T, sh.top_k), torch.int32)
    w = poisoned((T, sh.top_k))
    api.moe_layer_prefill(L.h, dev_u16(xb), None if logits is None else dev(logits), T, y, ids, w)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T", [1, 64, 300])
def test_prefill_small_layer_given_logits(T):
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    L = Layer(sh, d, max_T=300)
    xb = gen.x_bf16(T, sh.hidden, 40 + T)
    logits = gen.logits_uniform(T, sh.n_experts, 40 + T)
    y, ids, w = run_prefill(L, xb, logits, T)
    x = gen.bf16_bits_to_f32(xb).astype(np.float64)
    ref = moe.prefill(x, sh, d["shared"], d["experts"], logits_in=logits)
    assert np.array_equal(ids, ref["ids"])
    assert_close(w, ref["w"], "w")
    assert_close(y, ref["y"], f"y T={T}")
    L.close()


# Odd shapes for the GEMM tiles (32-row weight tiles, 64 rows per wave): a
# hidden size of 3 groups (96: the down projection's last wave holds one
# 32-row tile inside H and one past it; the gate/up's K is 3 groups, an odd
# number, so its last step holds one), routed rows of 3 and 5 groups, and
# token counts that leave ragged 32-token tiles.
@pytest.mark.parametrize("shape,T", [
    (Shape(hidden=96, n_experts=8, top_k=2, inter=96, shared_inter=160), 77),
    (Shape(hidden=160, n_experts=4, top_k=2, inter=160, shared_inter=96), 130),
    (Shape(hidden=8192, n_experts=8, top_k=2, inter=64, shared_inter=96), 100),  # the largest hidden size
])
def test_prefill_odd_shapes(shape, T):
    d = gen.layer_inputs(shape, 11)
    L = Layer(shape, d, max_T=T)
    xb = gen.x_bf16(T, shape.hidden, 50 + T)
    logits = gen.logits_uniform(T, shape.n_experts, 50 + T)
    y, ids, w = run_prefill(L, xb, logits, T)
    x = gen.bf16_bits_to_f32(xb).astype(np.float64)
    ref = moe.prefill(x, shape, d["shared"], d["experts"], logits_in=logits)
    assert np.array_equal(ids, ref["ids"])
    assert_close(y, ref["y"], f"y H={shape.hidden} T={T}")
    L.close()


def test_prefill_small_layer_router_logits():
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    L = Layer(sh, d, max_T=128)
    T = 100
    xb = gen.x_bf16(T, sh.hidden, 7)
    y, ids, w = run_prefill(L, xb, None, T)
    x = gen.bf16_bits_to_f32(xb).astype(np.float64)
    ref = moe.prefill(x, sh, d["shared"], d["experts"], router=d["router"])
    assert np.array_equal(ids, ref["ids"])
    assert_close(y, ref["y"], "y")
    L.close()


def test_prefill_full_2048_tokens():
    sh = GEMMA_LAYER
    d = layer_data(sh, 4)
    T = 2048
    L = Layer(sh, d, max_T=T)
    xb = gen.x_bf16(T, sh.hidden, 4)
    logits = gen.logits_uniform(T, sh.n_experts, 4)
    y, ids, w = run_prefill(L, xb, logits, T)
    x = gen.bf16_bits_to_f32(xb).astype(np.float64)
    ref = moe.prefill(x, sh, d["shared"], d["experts"], logits_in=logits)
    assert np.array_equal(ids, ref["ids"])
    assert_close(y, ref["y"], "y T=2048")
    # against the plain fp64 layer (no bf16 rounding points): the workload's
    # bf16 weights and bf16 GeGLU activations put the result 2.7e-3 of the
    # largest output away from it (the CPU model of the same rounding points
    # shows the same), above the 1e-3 bar; checked at bf16's unit roundoff 2^-8
    plain = moe.prefill(x, sh, d["shared"], d["experts"], logits_in=logits, mirror_bf16=False)
    assert_close(y, plain["y"], "y T=2048 against the unrounded layer", rel=2.0 ** -8)
    # deterministic: a second run gives the same bits
    y2, _, _ = run_prefill(L, xb, logits, T)
    assert np.array_equal(y, y2)
    L.close()


@pytest.mark.parametrize("shape,slots,T,source,chunk", [(SMALL_LAYER, 8, 300, "host", 128),
                                                         (SMALL_LAYER, 8, 300, "store", 128),
                                                         (GEMMA_LAYER, 16, 260, "host", 128),
                                                         (SMALL_LAYER, 8, 300, "host", 300),
                                                         # the routing limits: 1024 experts, top 16 (55 groups of 16 per chunk)
                                                         (Shape(hidden=256, n_experts=1024, top_k=16, inter=32, shared_inter=64),
                                                          16, 300, "host", 128)])
def test_prefill_through_slot_pool_matches_resident(tmp_path, shape, slots, T, source, chunk):
    """Chunks of 128 tokens (or one chunk) through the LFU slot pool (ragged last chunk) give
    the resident prefill's bits, ids and weights; the cache ends in the
    simulator's state after one step per group of each chunk's experts, and
    every slot holds its expert's blob; the handle then still decodes."""
    sh = shape
    d = layer_data(sh, 5)
    xb = gen.x_bf16(T, sh.hidden, 77)
    logits = gen.logits_uniform(T, sh.n_experts, 77)
    R = Layer(sh, d, max_T=T)
    y_r, ids_r, w_r = run_prefill(R, xb, logits, T)
    R.close()
    store = None
    if source == "store":
        blob = d["experts"].shape[1]
        padded = np.zeros((sh.n_experts, api.moe_store_stride(blob)), np.uint8)
        padded[:, :blob] = d["experts"]
        path = str(tmp_path / "experts.bin")
        padded.tofile(path)
        store = api.moe_store_open(path, 1, sh.n_experts, blob, 4, True)
    Cm = Layer(sh, d, cache_slots=slots, max_T=T, store=store)
    with pytest.raises(api.MoeError):
        api.moe_layer_prefill_chunk(Cm.h, T + 1)
    with pytest.raises(api.MoeError):
        api.moe_layer_prefill_chunk(Cm.h, 0)
    api.moe_layer_prefill_chunk(Cm.h, chunk)
    y_c, ids_c, w_c = run_prefill(Cm, xb, logits, T)
    # the oracle on the same inputs, then bitwise equality with the resident path
    ref = moe.prefill(gen.bf16_bits_to_f32(xb).astype(np.float64), sh, d["shared"], d["experts"],
                      logits_in=logits)
    assert np.array_equal(ids_c, ref["ids"])
    assert_close(w_c, ref["w"], "w slot pool")
    assert_close(y_c, ref["y"], f"y slot pool T={T} chunk={chunk}")
    assert np.array_equal(ids_c, ids_r) and np.array_equal(w_c, w_r)
    assert np.array_equal(y_c, y_r)
    sim = lfu.LFUCache(slots, sh.n_experts)
    g = min(slots, 16)
    for c0 in range(0, T, chunk):
        ex = sorted(set(ids_r[c0:c0 + chunk].reshape(-1).tolist()))
        for i in range(0, len(ex), g):
            sim.step(np.array(ex[i:i + g]))
    ex_n, fr_n, la_n = api.moe_cache_slots(api.moe_layer_cache(Cm.h), slots)
    assert ex_n.tolist() == sim.expert and fr_n.tolist() == sim.freq and la_n.tolist() == sim.last
    pool = Cm.pool.cpu().numpy()
    for s_, e in enumerate(sim.expert):
        if e >= 0:
            assert np.array_equal(pool[s_], d["experts"][e]), (s_, e)
    y = poisoned((1, sh.hidden))
    api.moe_layer_decode(Cm.h, dev(gen.x_fp32(1, sh.hidden, 5)), None, 1, 0, y)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    Cm.close()
    if store is not None:
        api.moe_store_close(store)


# The largest prefill a handle takes (max_T = 65536 tokens, 524288
# assignments, 16384 rows per expert on average) on the small layer.
def test_prefill_maximum_tokens():
    sh, T = SMALL_LAYER, 65536
    d = layer_data(sh, 0)
    L = Layer(sh, d, max_T=T)
    xb = gen.x_bf16(T, sh.hidden, 91)
    logits = gen.logits_uniform(T, sh.n_experts, 91)
    y, ids, w = run_prefill(L, xb, logits, T)
    L.close()
    ref = moe.prefill(gen.bf16_bits_to_f32(xb).astype(np.float64), sh, d["shared"], d["experts"], logits_in=logits)
    assert np.array_equal(ids, ref["ids"])
    assert_close(w, ref["w"], "w")
    assert_close(y, ref["y"], f"y T={T}")


def test_prefill_needs_max_T_and_empty_is_noop():
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    L = Layer(sh, d, max_T=16)
    y = poisoned((1, sh.hidden))
    api.moe_layer_prefill(L.h, dev_u16(gen.x_bf16(1, sh.hidden, 0)), None, 0, y)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(y))
    with pytest.raises(api.MoeError):
        api.moe_layer_prefill(L.h, dev_u16(gen.x_bf16(17, sh.hidden, 0)), None, 17, y)
    L.close()
    Lc = Layer(sh, d, cache_slots=8)
    with pytest.raises(api.MoeError):
        api.moe_layer_prefill(Lc.h, dev_u16(gen.x_bf16(1, sh.hidden, 0)), None, 1, y)
    Lc.close()
