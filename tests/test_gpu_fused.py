"""GPU tests of the fused expert-FFN launch (MOE_F_FUSED: routed gate/up, grid
barrier, down projections and combine in one kernel): the same bits and cache
trace as the two separate launches, with host- and device-stepped caches, at
the small and the Gemma shape; no barrier wait gives up; and the option is
available on a cache-mode layer of either shape on this device."""
import numpy as np
import pytest

from bit_quantized_expert_softmax_amd import api
from oracle import moe
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER
from tests.gpu_util import Layer, assert_close, dev
from tests.test_gpu_layer import layer_data, run_decode

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,cid,slots,tokens,on_device",
                         [(SMALL_LAYER, 8, 8, 16, False), (GEMMA_LAYER, 9, 16, 10, False),
                          (GEMMA_LAYER, 9, 16, 10, True)])
def test_fused_equals_separate_launches(shape, cid, slots, tokens, on_device):
    d = layer_data(shape, cid)
    bias = gen.zipf_bias(shape.n_experts, cid, 0)
    Lf = Layer(shape, d, bias=bias, cache_slots=slots, cache_on_device=on_device)
    Lu = Layer(shape, d, bias=bias, cache_slots=slots, cache_on_device=on_device)
    assert api.moe_layer_fused(Lf.h)
    xs = gen.x_fp32(tokens, shape.hidden, cid)
    base = api.MOE_F_RMSNORM_IN | api.MOE_F_RESIDUAL
    for t in range(tokens):
        print(f"fused case H={shape.hidden} device={on_device} token={t}", flush=True)
        yf, idf, _, uf, trf = run_decode(Lf, dev(xs[t:t + 1]), flags=base | api.MOE_F_FUSED, trace_k=shape.top_k)
        yu, idu, _, _, tru = run_decode(Lu, dev(xs[t:t + 1]), flags=base, trace_k=shape.top_k)
        assert np.array_equal(idf, idu) and np.array_equal(trf, tru), t
        assert np.array_equal(yf, yu), t
    api.moe_layer_check(Lf.h)
    # and the oracle on the last token, from the GPU's normalised input
    r = moe.layer_decode(uf[0].astype(np.float64), shape, d["router"], d["shared"], d["experts"], bias=bias)
    assert np.array_equal(idf[0], r["ids"][0])
    assert_close(yf[0], xs[-1] + r["y"][0], "fused y")
    Lf.close()
    Lu.close()
