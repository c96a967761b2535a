"""GPU tests of the miss fill's ordering and failure path (cache mode).

"Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
memória em um Mac comum", section "Qual é o principal truque da arquitetura":
missing experts are loaded while the GPU runs the shared-expert branch, so the
routed expert kernels must wait for their own loads and never read a slot that
is still being filled.

* delayed fills: a long unrelated copy is queued on the copy stream before
  each call, so the misses' copies land long after the shared expert; the
  output, the trace and every slot must still equal the oracle and the blobs;
* a failed copy enqueue (forced from the host by moe_debug_fail_copy, no GPU
  fault): the call returns MOE_EHIP, the cache is back in its pre-call state
  except that slots already written by the call's earlier copies are empty,
  and the next calls are correct again;
* stage times: the timed calls give the oracle's result and plausible times.
"""
import copy

import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu, moe
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER
from tests.gpu_util import Layer, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu

_CACHE = {}


def layer_data(shape, cid):
    if (shape, cid) not in _CACHE:
        _CACHE[(shape, cid)] = gen.layer_inputs(shape, cid)
    return _CACHE[(shape, cid)]


def decode(L, x, flags=0, stats=None):
    sh = L.shape
    y = poisoned((1, sh.hidden))
    ids = poisoned((1, sh.top_k), torch.int32)
    tr = api.moe_layer_decode(L.h, dev(x), None, 1, flags, y, ids, trace_k=sh.top_k, stats=stats)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), tr


def cache_state(L, slots):
    ex, fr, la = api.moe_cache_slots(api.moe_layer_cache(L.h), slots)
    return ex.tolist(), fr.tolist(), la.tolist()


def check_pool(L, d, expert):
    pool = L.pool.cpu().numpy()
    for s_, e in enumerate(expert):
        if e >= 0:
            assert np.array_equal(pool[s_], d["experts"][e]), (s_, e)


@pytest.mark.parametrize("shape,cid,slots", [(SMALL_LAYER, 0, 10), (GEMMA_LAYER, 2, 16)])
def test_delayed_fills_are_waited_for(shape, cid, slots):
    d = layer_data(shape, cid)
    bias = gen.zipf_bias(shape.n_experts, cid, 0)
    L = Layer(shape, d, bias=bias, cache_slots=slots)
    # 256 MiB pinned -> device: several ms on the copy stream ahead of each call's copies
    big_h = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    big_d = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
    xs = gen.x_fp32(6, shape.hidden, cid, sub=21)
    sim = lfu.LFUCache(slots, shape.n_experts)
    n_miss = 0
    for t in range(6):
        print(f"delayed fill H={shape.hidden} token={t}", flush=True)
        with torch.cuda.stream(L.copy_stream):
            big_d.copy_(big_h, non_blocking=True)
        y, ids, tr = decode(L, xs[t:t + 1])
        r = moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"], bias=bias)
        assert np.array_equal(ids, r["ids"]), t
        want = sim.step(ids[0])
        assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in want], t
        n_miss += sum(1 for e in want if not e[2])
        assert_close(y, r["y"], f"y t={t}")
    assert n_miss > 0
    check_pool(L, d, sim.expert)
    L.close()


@pytest.mark.parametrize("nth", [1, 2, 3])
def test_failed_miss_copy_undoes_the_step(nth):
    shape, cid, slots = SMALL_LAYER, 0, 12
    d = layer_data(shape, cid)
    L = Layer(shape, d, cache_slots=slots)
    xs = gen.x_fp32(4, shape.hidden, cid, sub=31)
    refs = [moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"])
            for t in range(4)]
    sim = lfu.LFUCache(slots, shape.n_experts)
    # token 0 decodes normally
    y, ids, tr = decode(L, xs[0:1])
    assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in sim.step(refs[0]["ids"][0])]
    # token 1: its misses' slots in copy order, from a copy of the simulator
    probe = copy.deepcopy(sim)
    ev1 = probe.step(refs[1]["ids"][0])
    miss_slots = [e[1] for e in ev1 if not e[2]]
    assert len(miss_slots) >= nth, "the case needs enough misses"
    print(f"failed copy nth={nth} misses={len(miss_slots)}", flush=True)
    api.moe_debug_fail_copy(L.h, nth)
    with pytest.raises(api.MoeError) as ex:
        decode(L, xs[1:2])
    assert ex.value.status == -4 and "injected" in str(ex.value)
    # the pre-call state, with the slots of the copies enqueued before the failure emptied
    for s_ in miss_slots[:nth - 1]:
        sim.expert[s_], sim.freq[s_], sim.last[s_] = lfu.EMPTY, 0, -1
    assert cache_state(L, slots) == (sim.expert, sim.freq, sim.last)
    check_pool(L, d, sim.expert)
    # the same token again, then the next ones: the oracle's results, the simulator's traces
    for t in (1, 2, 3):
        y, ids, tr = decode(L, xs[t:t + 1])
        assert np.array_equal(ids, refs[t]["ids"]), t
        assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in sim.step(ids[0])], t
        assert_close(y, refs[t]["y"], f"y t={t}")
    assert cache_state(L, slots) == (sim.expert, sim.freq, sim.last)
    check_pool(L, d, sim.expert)
    L.close()


def test_failed_copy_in_slot_pool_prefill_leaves_a_consistent_pool():
    sh, slots, T = SMALL_LAYER, 8, 200
    d = layer_data(sh, 5)
    xb = gen.x_bf16(T, sh.hidden, 78)
    logits = gen.logits_uniform(T, sh.n_experts, 78)
    x = gen.bf16_bits_to_f32(xb).astype(np.float64)
    ref = moe.prefill(x, sh, d["shared"], d["experts"], logits_in=logits)
    L = Layer(sh, d, cache_slots=slots, max_T=T)
    api.moe_debug_fail_copy(L.h, 13)  # the 5th copy of the chunk's second group of 8
    y = poisoned((T, sh.hidden))
    with pytest.raises(api.MoeError) as ex:
        api.moe_layer_prefill(L.h, dev_u16(xb), dev(logits), T, y)
    torch.cuda.synchronize()
    assert ex.value.status == -4
    expert, _, _ = cache_state(L, slots)
    check_pool(L, d, expert)
    # a second prefill over the partly emptied pool is the oracle's result
    api.moe_layer_prefill(L.h, dev_u16(xb), dev(logits), T, y)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), ref["y"], "y after the failed prefill")
    expert, _, _ = cache_state(L, slots)
    check_pool(L, d, expert)
    L.close()


@pytest.mark.parametrize("fill", [0, api.MOE_F_FILL_KERNEL], ids=["copy_engine", "fill_kernel"])
def test_stage_times(fill):
    shape, cid, slots = GEMMA_LAYER, 2, 16
    d = layer_data(shape, cid)
    bias = gen.zipf_bias(shape.n_experts, cid, 0)
    L = Layer(shape, d, bias=bias, cache_slots=slots)
    xs = gen.x_fp32(5, shape.hidden, cid, sub=41)
    sim = lfu.LFUCache(slots, shape.n_experts)
    for t in range(5):
        st = api.moe_decode_stats()
        y, ids, tr = decode(L, xs[t:t + 1], fill | api.MOE_F_STAGE_TIMES, stats=st)
        want = sim.step(ids[0])
        assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in want], t
        r = moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"], bias=bias)
        assert_close(y, r["y"], f"y t={t}")
        n_miss = sum(1 for e in want if not e[2])
        assert st.misses == n_miss and st.calls == 1
        assert 0.0 < st.ms_route < 1e3 and 0.0 < st.ms_total < 1e3
        if n_miss:
            # a 3.35 MB blob takes more than 20 us at under 170 GB/s; the copy
            # engine alternates the misses over two streams
            assert st.ms_fill > 0.0 and st.ms_wait_fill >= 0.0
            if not fill:
                assert st.ms_fill >= 0.02 * ((n_miss + 1) // 2), (st.ms_fill, n_miss)
            assert st.ms_total >= st.ms_wait_fill
        else:
            assert st.ms_fill == 0.0 and st.ms_wait_fill == 0.0
    with pytest.raises(api.MoeError):
        decode(L, xs[0:1], api.MOE_F_STAGE_TIMES, stats=None)
    L.close()
