"""Every entry point on a caller's stream other than the default one: the
library orders its work on the stream it is given (and, in cache mode, the
copies on its side streams after that stream's earlier work), so the results
are those of the default stream, checked against the fp64 oracle and the LFU
simulator.

"Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
memória em um Mac comum", section "Qual é o principal truque da
arquitetura": misses are loaded while the GPU computes the shared-expert
branch, which here runs on the caller's stream.
"""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu, moe
from synth import gen
from synth.configs import SMALL_LAYER
from tests.gpu_util import Layer, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu

SH = SMALL_LAYER
_CACHE = {}


def layer_data():
    if "d" not in _CACHE:
        _CACHE["d"] = gen.layer_inputs(SH, 31)
    return _CACHE["d"]


def on_stream(s, fn):
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = fn()
    s.synchronize()
    return out


@pytest.mark.parametrize("mode", ["resident", "copy_engine", "fill_kernel"])
def test_decode_on_a_user_stream(mode):
    d = layer_data()
    bias = gen.zipf_bias(SH.n_experts, 31, 0)
    cache = mode != "resident"
    L = Layer(SH, d, bias=bias, cache_slots=12 if cache else 0)
    flags = api.MOE_F_FILL_KERNEL if mode == "fill_kernel" else 0
    s = torch.cuda.Stream()
    xs = gen.x_fp32(10, SH.hidden, 31, sub=2)
    sim = lfu.LFUCache(12, SH.n_experts)
    for t in range(xs.shape[0]):
        print(f"streams: {mode} token {t}", flush=True)
        x = dev(xs[t:t + 1])
        y = poisoned((1, SH.hidden))
        ids = poisoned((1, SH.top_k), torch.int32)
        tr = on_stream(s, lambda: api.moe_layer_decode(L.h, x, None, 1, flags, y, ids,
                                                       trace_k=SH.top_k if cache else 0, stream=s))
        r = moe.layer_decode(xs[t].astype(np.float64), SH, d["router"], d["shared"], d["experts"], bias=bias)
        assert np.array_equal(ids.cpu().numpy(), r["ids"]), t
        assert_close(y.cpu().numpy(), r["y"], f"y t={t}")
        if cache:
            want = sim.step(r["ids"][0])
            assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in want], t
    if cache:
        assert sim.hits > 0 and sim.misses > 0
    L.close()


def test_batched_and_prefill_on_a_user_stream():
    d = layer_data()
    s = torch.cuda.Stream()
    B, T = 16, 300
    L = Layer(SH, d, max_B=B, max_T=T)
    x = gen.x_fp32(B, SH.hidden, 31, sub=3)
    xd = dev(x)
    y = poisoned((B, SH.hidden))
    ids = poisoned((B, SH.top_k), torch.int32)
    on_stream(s, lambda: api.moe_layer_decode(L.h, xd, None, B, 0, y, ids, stream=s))
    r = moe.layer_decode(x.astype(np.float64), SH, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert_close(y.cpu().numpy(), r["y"], "batched y")
    xb = gen.x_bf16(T, SH.hidden, 32)
    logits = gen.logits_uniform(T, SH.n_experts, 32)
    xbd, lgd = dev_u16(xb), dev(logits)
    yp = poisoned((T, SH.hidden))
    idp = poisoned((T, SH.top_k), torch.int32)
    on_stream(s, lambda: api.moe_layer_prefill(L.h, xbd, lgd, T, yp, idp, stream=s))
    ref = moe.prefill(gen.bf16_bits_to_f32(xb).astype(np.float64), SH, d["shared"], d["experts"], logits_in=logits)
    assert np.array_equal(idp.cpu().numpy(), ref["ids"])
    assert_close(yp.cpu().numpy(), ref["y"], "prefill y")
    L.close()
