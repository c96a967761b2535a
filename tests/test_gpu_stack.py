"""GPU parity of the full benchmark workload: the 30-layer stack of the
2816x128x704 layer with a 16-slot LFU cache per layer and every expert in
pinned host memory, decoded one token at a time in cache mode with the
RMSNorm prologue and the residual, on the benchmark's own seeded inputs.

Every layer step checks the routing (bit-exact against the oracle's fp64
routing of the GPU's own normalised input) and the cache trace (bit-exact
against the LFU simulator); on the first and the last token every layer's
output is compared with the oracle's step from the GPU's input to that layer
(so rounding differences do not accumulate across layers). At the end every
slot holds a byte-exact copy of the expert its cache says it holds."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu, moe
from synth import gen
from synth.configs import C2
from tests.gpu_util import assert_close, dev, dev_u16, pinned, poisoned

pytestmark = pytest.mark.gpu

TOKENS = 3


def test_stack_30_layers_lfu16_matches_oracle():
    sh = C2.shape
    cid = C2.config_id
    H, E, k = sh.hidden, sh.n_experts, sh.top_k
    n_layers, slots = C2.layers, C2.n_slots
    flags = api.MOE_F_RMSNORM_IN | api.MOE_F_RESIDUAL
    copy_stream = torch.cuda.Stream()
    layers = []
    for l in range(n_layers):
        d = {"router": gen.router(sh, cid, l), "bias": gen.zipf_bias(E, cid, l),
             "shared": gen.shared_blob(sh, cid, l), "experts": gen.expert_blobs(sh, cid, l)}
        d["host"] = pinned(d["experts"])
        d["dev"] = (dev_u16(d["router"]), dev(d["bias"]), dev(d["shared"]))
        d["pool"] = torch.zeros((slots, d["experts"].shape[1]), dtype=torch.uint8, device="cuda:0")
        d["ws"] = torch.zeros(api.moe_layer_workspace_bytes(sh, 1, 0), dtype=torch.uint8, device="cuda:0")
        d["h"] = api.moe_layer_create(sh, router=d["dev"][0], bias=d["dev"][1], shared_blob=d["dev"][2],
                                      workspace=d["ws"], experts_host=d["host"], slot_pool=d["pool"],
                                      n_slots=slots, copy_stream=copy_stream)
        d["sim"] = lfu.LFUCache(slots, E)
        layers.append(d)
    x = gen.x_fp32(TOKENS, H, cid)
    eps = gen.eps_fp16(n_layers, TOKENS, H, cid)
    eps_dev = dev_u16(eps)
    for t in range(TOKENS):
        h = dev(x[t:t + 1])
        for l, d in enumerate(layers):
            print(f"[stack] token {t} layer {l}", flush=True)
            y = poisoned((1, H))
            ids = poisoned((1, k), torch.int32)
            u = poisoned((1, H))
            tr = api.moe_layer_decode(d["h"], h, eps_dev[l, t:t + 1], 1, flags, y, ids, None, u, trace_k=k)
            torch.cuda.synchronize()
            ids_np, u_np = ids.cpu().numpy(), u.cpu().numpy()
            r_ids, _, _ = moe.route(u_np.astype(np.float64), d["router"], k, d["bias"])
            assert np.array_equal(ids_np, r_ids), (t, l)
            want = d["sim"].step(ids_np[0])
            assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in want], (t, l)
            if t in (0, TOKENS - 1):
                lay = {"router": d["router"], "bias": d["bias"], "shared": d["shared"], "experts": d["experts"]}
                h_ref, rec = moe.stack_layer_step(h.cpu().numpy()[0], eps[l, t], sh, lay)
                assert_close(u_np, rec["u"], f"u t={t} l={l}")
                assert_close(y.cpu().numpy(), h_ref, f"y t={t} l={l}")
            h = y
    for l, d in enumerate(layers):
        pool = d["pool"].cpu().numpy()
        for s_, e in enumerate(d["sim"].expert):
            if e >= 0:
                assert np.array_equal(pool[s_], d["experts"][e]), (l, s_, e)
        api.moe_layer_destroy(d["h"])
    assert sum(d["sim"].misses for d in layers) > 0 and sum(d["sim"].hits for d in layers) > 0
