"""The resident entry points captured in a HIP graph: one-token decode (with
the RMSNorm prologue and the residual), batched decode and prefill. Each
graph is replayed several times with new inputs copied in, with eager calls of
a second handle and synchronisations between the replays, and every replay
must give the eager call's bits (the library records no memset and no host
round trip on these paths).

"Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
memória em um Mac comum", section "Qual é o principal truque da
arquitetura": per token and layer, routing, the experts and the combine.
"""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER
from tests.gpu_util import DEV, Layer, dev, dev_u16

pytestmark = pytest.mark.gpu


def _replays(capture, eager, inputs, copy_in, out, n=5):
    cap = torch.cuda.Stream()
    copy_in(inputs[0])
    capture()  # once eagerly first (nothing is loaded lazily inside the capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        capture()
    torch.cuda.synchronize()
    for t in range(n):
        print(f"graph replay {t}", flush=True)
        copy_in(inputs[t % len(inputs)])
        g.replay()
        torch.cuda.synchronize()
        want = eager(inputs[t % len(inputs)])
        assert np.array_equal(out().cpu().numpy(), want), t
    del g


@pytest.mark.parametrize("shape", [SMALL_LAYER, GEMMA_LAYER], ids=["small", "gemma"])
def test_resident_decode_replays_equal_eager(shape):
    d = gen.layer_inputs(shape, 41)
    Lg, Le = Layer(shape, d), Layer(shape, d)
    flags = api.MOE_F_RMSNORM_IN | api.MOE_F_RESIDUAL
    xs = [gen.x_fp32(1, shape.hidden, 41, sub=t) for t in range(3)]
    eps = dev_u16(gen.eps_fp16(1, 1, shape.hidden, 41)[0])
    xg = torch.empty((1, shape.hidden), device=DEV)
    yg = torch.empty((1, shape.hidden), device=DEV)

    def capture():
        api.moe_layer_decode(Lg.h, xg, eps, 1, flags, yg, stream=torch.cuda.current_stream())

    def eager(x):
        y = torch.empty((1, shape.hidden), device=DEV)
        api.moe_layer_decode(Le.h, dev(x), eps, 1, flags, y)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    _replays(capture, eager, xs, lambda x: xg.copy_(dev(x)), lambda: yg)
    Lg.close()
    Le.close()


def test_batched_decode_and_prefill_replay_equal_eager():
    sh = SMALL_LAYER
    d = gen.layer_inputs(sh, 42)
    B, T = 24, 200
    Lg, Le = Layer(sh, d, max_B=B, max_T=T), Layer(sh, d, max_B=B, max_T=T)
    xs = [gen.x_fp32(B, sh.hidden, 42, sub=t) for t in range(3)]
    xg = torch.empty((B, sh.hidden), device=DEV)
    yg = torch.empty((B, sh.hidden), device=DEV)

    def eager_b(x):
        y = torch.empty((B, sh.hidden), device=DEV)
        api.moe_layer_decode(Le.h, dev(x), None, B, 0, y)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    _replays(lambda: api.moe_layer_decode(Lg.h, xg, None, B, 0, yg, stream=torch.cuda.current_stream()),
             eager_b, xs, lambda x: xg.copy_(dev(x)), lambda: yg)

    xbs = [gen.x_bf16(T, sh.hidden, 43 + t) for t in range(3)]
    lgs = [gen.logits_uniform(T, sh.n_experts, 43 + t) for t in range(3)]
    xbg = torch.empty((T, sh.hidden), dtype=torch.int16, device=DEV)
    lgg = torch.empty((T, sh.n_experts), device=DEV)
    ypg = torch.empty((T, sh.hidden), device=DEV)

    def copy_p(i):
        xbg.copy_(dev_u16(xbs[i]))
        lgg.copy_(dev(lgs[i]))

    def eager_p(i):
        y = torch.empty((T, sh.hidden), device=DEV)
        api.moe_layer_prefill(Le.h, dev_u16(xbs[i]), dev(lgs[i]), T, y)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    _replays(lambda: api.moe_layer_prefill(Lg.h, xbg, lgg, T, ypg, stream=torch.cuda.current_stream()),
             eager_p, [0, 1, 2], copy_p, lambda: ypg)
    Lg.close()
    Le.close()
