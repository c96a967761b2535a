"""GPU parity at the routing limits every entry point accepts: 1024 experts and
the top 16 of them (MOE_MAX_EXPERTS, MOE_MAX_TOPK), through one-token decode
(resident, and cache mode with as many slots as ranks), batched decode and
prefill, against the fp64 oracle and the LFU simulator.

"Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
memória em um Mac comum", section "Qual é o principal truque da
arquitetura": a router picks the token's experts, a small LFU expert cache
is checked and misses are loaded; the pages use 8 of 128 experts and 16
slots, the limits here are the library's own.
"""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu, moe
from synth import gen
from synth.configs import Shape
from tests.gpu_util import Layer, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu

WIDE = Shape(hidden=256, n_experts=1024, top_k=16, inter=32, shared_inter=64)
_CACHE = {}


def layer_data():
    if "d" not in _CACHE:
        _CACHE["d"] = gen.layer_inputs(WIDE, 21)
    return _CACHE["d"]


def decode(L, x, trace_k=0):
    B = x.shape[0]
    y = poisoned((B, WIDE.hidden))
    ids = poisoned((B, WIDE.top_k), torch.int32)
    w = poisoned((B, WIDE.top_k))
    tr = api.moe_layer_decode(L.h, dev(x), None, B, 0, y, ids, w, trace_k=trace_k)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), tr


def test_widest_routing_resident_and_cache_mode():
    d = layer_data()
    xs = gen.x_fp32(6, WIDE.hidden, 21, sub=1)
    R = Layer(WIDE, d)
    C = Layer(WIDE, d, cache_slots=WIDE.top_k)
    sim = lfu.LFUCache(WIDE.top_k, WIDE.n_experts)
    for t in range(xs.shape[0]):
        print(f"limits: E=1024 k=16 token {t}", flush=True)
        r = moe.layer_decode(xs[t].astype(np.float64), WIDE, d["router"], d["shared"], d["experts"])
        for L, cache in ((R, False), (C, True)):
            y, ids, w, tr = decode(L, xs[t:t + 1], trace_k=WIDE.top_k if cache else 0)
            assert np.array_equal(ids, r["ids"]), (t, cache)
            assert_close(w, r["w"], f"w t={t}")
            assert_close(y, r["y"], f"y t={t} cache={cache}")
            if cache:
                want = sim.step(ids[0])
                assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in want], t
    pool = C.pool.cpu().numpy()
    for s_, e in enumerate(sim.expert):
        if e >= 0:
            assert np.array_equal(pool[s_], d["experts"][e]), (s_, e)
    R.close()
    C.close()


@pytest.mark.parametrize("B", [3, 40])
def test_widest_routing_batched(B):
    d = layer_data()
    print(f"limits: E=1024 k=16 batched B={B}", flush=True)
    L = Layer(WIDE, d, max_B=B)
    x = gen.x_fp32(B, WIDE.hidden, 21, sub=B)
    y, ids, w, _ = decode(L, x)
    r = moe.layer_decode(x.astype(np.float64), WIDE, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids, r["ids"])
    assert_close(w, r["w"], "w")
    assert_close(y, r["y"], f"y B={B}")
    L.close()


def test_widest_routing_prefill():
    d = layer_data()
    T = 300
    print(f"limits: E=1024 k=16 prefill T={T}", flush=True)
    L = Layer(WIDE, d, max_T=T)
    xb = gen.x_bf16(T, WIDE.hidden, 22)
    y = poisoned((T, WIDE.hidden))
    ids = poisoned((T, WIDE.top_k), torch.int32)
    w = poisoned((T, WIDE.top_k))
    api.moe_layer_prefill(L.h, dev_u16(xb), None, T, y, ids, w)
    torch.cuda.synchronize()
    x = gen.bf16_bits_to_f32(xb).astype(np.float64)
    ref = moe.prefill(x, WIDE, d["shared"], d["experts"], router=d["router"])
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_close(w.cpu().numpy(), ref["w"], "w")
    assert_close(y.cpu().numpy(), ref["y"], f"y T={T}")
    L.close()


# The cache stepped on the device at the limits: 1024 experts, 16 ranks, the
# fewest slots a token needs (16) and more (64), both policies; the trace is
# the simulator's, the outputs the oracle's.
@pytest.mark.parametrize("policy,slots", [("lfu", 16), ("lru", 16), ("lfu", 64)])
def test_widest_routing_device_stepped_cache(policy, slots):
    d = layer_data()
    pol = api.MOE_POLICY_LRU if policy == "lru" else api.MOE_POLICY_LFU
    L = Layer(WIDE, d, cache_slots=slots, cache_policy=pol, cache_on_device=True)
    sim = lfu.LFUCache(slots, WIDE.n_experts, policy=policy)
    xs = gen.x_fp32(8, WIDE.hidden, 23, sub=slots)
    for t in range(xs.shape[0]):
        print(f"limits: device-stepped cache {policy} slots={slots} token {t}", flush=True)
        y, ids, w, tr = decode(L, xs[t:t + 1], trace_k=WIDE.top_k)
        r = moe.layer_decode(xs[t].astype(np.float64), WIDE, d["router"], d["shared"], d["experts"])
        assert np.array_equal(ids, r["ids"]), t
        assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in sim.step(ids[0])], t
        assert_close(y, r["y"], f"y t={t}")
    ex, fr, la, hits, misses, steps = api.moe_layer_cache_state(L.h, slots)
    assert list(ex) == list(sim.expert) and list(fr) == list(sim.freq) and list(la) == list(sim.last)
    assert (hits, misses, steps) == (sim.hits, sim.misses, xs.shape[0])
    pool = L.pool.cpu().numpy()
    for s_, e in enumerate(sim.expert):
        if e >= 0:
            assert np.array_equal(pool[s_], d["experts"][e]), (s_, e)
    L.close()
