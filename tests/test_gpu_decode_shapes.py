"""GPU parity of one-token decode on hidden sizes that reach every form of the
gate/up kernel: 1 ... 16 chunk columns per lane, 4-wave blocks (up to 8
columns) and 1024-lane blocks (more), row scales that do not start on a
16-byte boundary (an odd number of groups per row), in resident mode (in-kernel
top-k) and cache mode (copy engine and fill kernel).

"Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
memória em um Mac comum", section "Qual é o principal truque da
arquitetura": per token a router picks k experts, each a GeGLU FFN of int4
weights, plus a shared expert; the oracle computes that layer in fp64.
"""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu, moe
from synth import gen
from synth.configs import Shape
from tests.gpu_util import Layer, assert_close, dev, poisoned

pytestmark = pytest.mark.gpu

# hidden -> groups per row (chunk columns per lane = ceil(groups / 16))
SHAPES = [
    Shape(hidden=96, n_experts=8, top_k=2, inter=64, shared_inter=64),     # 3 groups: 1 column, unaligned
    Shape(hidden=992, n_experts=8, top_k=2, inter=64, shared_inter=96),    # 31: 2 columns
    Shape(hidden=1056, n_experts=8, top_k=3, inter=64, shared_inter=64),   # 33: 3 columns
    Shape(hidden=1568, n_experts=8, top_k=2, inter=96, shared_inter=64),   # 49: 4 columns
    Shape(hidden=2336, n_experts=8, top_k=2, inter=64, shared_inter=64),   # 73: 5 -> 6 columns
    Shape(hidden=4096, n_experts=8, top_k=2, inter=64, shared_inter=64),   # 128: 8 columns, 4-wave blocks
    Shape(hidden=4128, n_experts=8, top_k=2, inter=64, shared_inter=64),   # 129: 12 columns, 1024 lanes
    Shape(hidden=8192, n_experts=8, top_k=2, inter=32, shared_inter=64),   # 256: 16 columns
]
IDS = [f"H{s.hidden}" for s in SHAPES]
_CACHE = {}


def layer_data(shape):
    if shape not in _CACHE:
        _CACHE[shape] = gen.layer_inputs(shape, 9)
    return _CACHE[shape]


def decode(L, x, flags=0):
    sh = L.shape
    y = poisoned((1, sh.hidden))
    ids = poisoned((1, sh.top_k), torch.int32)
    tr = api.moe_layer_decode(L.h, dev(x), None, 1, flags, y, ids, trace_k=sh.top_k)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), tr


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_resident_decode_shapes(shape):
    d = layer_data(shape)
    L = Layer(shape, d)
    xs = gen.x_fp32(3, shape.hidden, 9, sub=3)
    for t in range(3):
        print(f"resident H={shape.hidden} token={t}", flush=True)
        y, ids, _ = decode(L, xs[t:t + 1])
        r = moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"])
        assert np.array_equal(ids, r["ids"]), t
        assert_close(y, r["y"], f"y H={shape.hidden} t={t}")
    L.close()


@pytest.mark.parametrize("fill", [0, api.MOE_F_FILL_KERNEL], ids=["copy_engine", "fill_kernel"])
@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_cache_mode_decode_shapes(shape, fill):
    d = layer_data(shape)
    slots = shape.top_k + 1
    L = Layer(shape, d, cache_slots=slots)
    xs = gen.x_fp32(4, shape.hidden, 9, sub=4)
    sim = lfu.LFUCache(slots, shape.n_experts)
    for t in range(4):
        print(f"cache H={shape.hidden} fill={fill} token={t}", flush=True)
        y, ids, tr = decode(L, xs[t:t + 1], fill)
        r = moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"])
        assert np.array_equal(ids, r["ids"]), t
        assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in sim.step(ids[0])], t
        assert_close(y, r["y"], f"y H={shape.hidden} t={t}")
    L.close()


def test_hidden_above_the_one_token_limit_is_refused():
    shape = Shape(hidden=8224, n_experts=4, top_k=1, inter=32, shared_inter=32)
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(api.MoeError) as ex:
        api.moe_layer_create(shape, router=buf, shared_blob=buf, workspace=buf, experts_dev=buf)
    assert ex.value.status == -2 and "8192" in str(ex.value)
