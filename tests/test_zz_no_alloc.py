"""moe_route_noalloc, the routing entry point that allocates nothing (its
logits live in the library's own device array), against moe_route with a
caller workspace: the same kernels, so the same bits, and the oracle's ids.
Two calls in a row, the second with fewer tokens; sizes past the array's
limit are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import moe
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER
from tests.gpu_util import DEV, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu


def route_both(shape, x, wr, bias, B):
    ids_a = poisoned((B, shape.top_k), torch.int32)
    w_a = poisoned((B, shape.top_k))
    ws = torch.empty(api.moe_route_workspace_bytes(shape, B), dtype=torch.uint8, device=DEV)
    api.moe_route(shape, x, wr, bias, None, B, ids_a, w_a, ws)
    ids_b = poisoned((B, shape.top_k), torch.int32)
    w_b = poisoned((B, shape.top_k))
    api.moe_route_noalloc(shape, x, wr, bias, None, B, ids_b, w_b)
    torch.cuda.synchronize()
    return ids_a.cpu().numpy(), w_a.cpu().numpy(), ids_b.cpu().numpy(), w_b.cpu().numpy()


@pytest.mark.parametrize("shape,cid", [(GEMMA_LAYER, 1), (SMALL_LAYER, 0)])
def test_noalloc_route_equals_workspace_route(shape, cid):
    wr = gen.router(shape, cid)
    bias = gen.zipf_bias(shape.n_experts, cid, 0)
    wr_d, bias_d = dev_u16(wr), dev(bias)
    for B in (64, 7):  # the second call is smaller than the first
        x = gen.x_fp32(B, shape.hidden, cid, sub=100 + B)
        for use_bias in (False, True):
            print(f"noalloc route H={shape.hidden} B={B} bias={use_bias}", flush=True)
            b = bias_d if use_bias else None
            ids_a, w_a, ids_b, w_b = route_both(shape, dev(x), wr_d, b, B)
            assert np.array_equal(ids_a, ids_b) and np.array_equal(w_a, w_b)
            r_ids, r_w, _ = moe.route(x.astype(np.float64), wr, shape.top_k, bias if use_bias else None)
            assert np.array_equal(ids_b, r_ids)
            assert_close(w_b, r_w, "w")


def test_noalloc_route_given_logits_and_limits():
    sh = GEMMA_LAYER
    T = 300
    logits = gen.logits_uniform(T, sh.n_experts, 9)
    ids = poisoned((T, sh.top_k), torch.int32)
    w = poisoned((T, sh.top_k))
    api.moe_route_noalloc(sh, None, None, None, dev(logits), T, ids, w)
    torch.cuda.synchronize()
    r_ids, r_w, _ = moe.route(None, None, sh.top_k, logits_in=logits)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert_close(w.cpu().numpy(), r_w, "w")
    # past the scratch array: refused, nothing written
    B = api.MOE_ROUTE_NOALLOC_MAX // sh.n_experts + 1
    x = torch.zeros((B, sh.hidden), device=DEV)
    wr = dev_u16(gen.router(sh, 1))
    ids2 = poisoned((B, sh.top_k), torch.int32)
    w2 = poisoned((B, sh.top_k))
    with pytest.raises(api.MoeError) as ex:
        api.moe_route_noalloc(sh, x, wr, None, None, B, ids2, w2)
    assert ex.value.status == -2
    torch.cuda.synchronize()
    assert torch.all(ids2 == -7777)
