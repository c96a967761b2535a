"""GPU tests of the device-stepped expert-slot cache (moe_layer_desc.cache_on_device):
the routing kernel's cache step gives the simulator's trace and final state
for both policies, the same bits as the host-stepped cache, and a decode call
that can be captured in a graph and replayed."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER
from tests.gpu_util import DEV, Layer, dev, poisoned
from tests.test_gpu_layer import layer_data, run_decode

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("policy,slots", [("lfu", 8), ("lru", 8), ("lfu", 16), ("lfu", 32)])
def test_device_step_matches_simulator_and_host_step(policy, slots):
    sh = SMALL_LAYER
    d = layer_data(sh, 6)
    bias = gen.zipf_bias(sh.n_experts, 6, 0)
    pol = api.MOE_POLICY_LRU if policy == "lru" else api.MOE_POLICY_LFU
    Lh = Layer(sh, d, bias=bias, cache_slots=slots, cache_policy=pol)
    Ld = Layer(sh, d, bias=bias, cache_slots=slots, cache_policy=pol, cache_on_device=True)
    sim = lfu.LFUCache(slots, sh.n_experts, policy=policy)
    xs = gen.x_fp32(24, sh.hidden, 6, sub=slots)
    for t in range(24):
        print(f"dcache case policy={policy} slots={slots} token={t}", flush=True)
        yh, idh, _, _, trh = run_decode(Lh, dev(xs[t:t + 1]), flags=api.MOE_F_FILL_KERNEL, trace_k=sh.top_k)
        yd, idd, _, _, trd = run_decode(Ld, dev(xs[t:t + 1]), trace_k=sh.top_k)
        assert np.array_equal(idh, idd), t
        want = [tuple(e) for e in sim.step(idd[0])]
        assert [tuple(e) for e in trd.tolist()] == want, t
        assert [tuple(e) for e in trh.tolist()] == want, t
        assert np.array_equal(yh, yd), t
    ex, fr, la, hits, misses, steps = api.moe_layer_cache_state(Ld.h, slots)
    assert list(ex) == list(sim.expert) and list(fr) == list(sim.freq) and list(la) == list(sim.last)
    assert (hits, misses, steps) == (sim.hits, sim.misses, 24)
    exh, frh, lah, hh, mh, sth = api.moe_layer_cache_state(Lh.h, slots)
    assert np.array_equal(ex, exh) and np.array_equal(fr, frh) and np.array_equal(la, lah)
    assert (hh, mh, sth) == (hits, misses, steps)
    Lh.close()
    Ld.close()


def test_device_step_decode_replays_from_a_graph():
    sh = GEMMA_LAYER
    d = layer_data(sh, 7)
    bias = gen.zipf_bias(sh.n_experts, 7, 0)
    Le = Layer(sh, d, bias=bias, cache_slots=16, cache_on_device=True)
    Lg = Layer(sh, d, bias=bias, cache_slots=16, cache_on_device=True)
    xs = gen.x_fp32(6, sh.hidden, 7)
    xb = dev(xs[0:1])
    yb = torch.empty((1, sh.hidden), device=DEV)
    lib = api.lib()
    cap = torch.cuda.Stream()

    def step():
        rc = lib.moe_layer_decode(Lg.h, xb.data_ptr(), None, 1, 0, yb.data_ptr(), None, None, None, None, None,
                                  torch.cuda.current_stream().cuda_stream)
        assert rc == 0, api.moe_last_error()

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    for t in range(6):
        print(f"dcache graph replay {t}", flush=True)
        xb.copy_(dev(xs[t:t + 1]))
        g.replay()
        torch.cuda.synchronize()
        ye, _, _, _, _ = run_decode(Le, dev(xs[t:t + 1]))
        assert np.array_equal(yb.cpu().numpy(), ye), t
    se = api.moe_layer_cache_state(Le.h, 16)
    sg = api.moe_layer_cache_state(Lg.h, 16)
    assert all(np.array_equal(a, b) for a, b in zip(se[:3], sg[:3])) and se[3:] == sg[3:]
    assert se[5] == 6
    del g
    Le.close()
    Lg.close()


def test_device_step_refuses_prefill_and_store():
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    L = Layer(sh, d, cache_slots=8, cache_on_device=True, max_T=64)
    xb = torch.zeros((4, sh.hidden), dtype=torch.int16, device=DEV)
    y = poisoned((4, sh.hidden))
    with pytest.raises(api.MoeError, match="device"):
        api.moe_layer_prefill(L.h, xb, None, 4, y)
    L.close()
