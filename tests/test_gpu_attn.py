"""GPU parity of the attention step (moe_attn_decode) against the fp64 oracle:
the output y = x + Wo a, the key and value appended to the fp16 cache at pos,
the rest of the cache untouched; one and several context splits, ragged last
splits, the largest position, 1, 2 and 4 query heads per key/value head, head
widths 64, 128 and 256, consecutive steps filling an empty cache."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import attn
from synth import gen
from synth.configs import GEMMA_ATTN, SMALL_ATTN, AttnShape
from tests.gpu_util import DEV, assert_close, dev, dev_u16

pytestmark = pytest.mark.gpu

# d = 128 with 4 query heads per group; d = 64 with one (plain multi-head)
WIDE_GROUP = AttnShape(hidden=1024, n_heads=8, n_kv_heads=2, head_dim=128, max_ctx=1024)
MHA = AttnShape(hidden=256, n_heads=2, n_kv_heads=2, head_dim=64, max_ctx=2048)
# one query head of width 64: a combine grid of one partly used block
ONE_HEAD = AttnShape(hidden=128, n_heads=1, n_kv_heads=1, head_dim=64, max_ctx=1100)
# the widest step the library takes: hidden 4096, 32 query heads of 256 over 8
# key/value heads (n_heads * d = 8192)
WIDEST = AttnShape(hidden=4096, n_heads=32, n_kv_heads=8, head_dim=256, max_ctx=640)


class Step:
    def __init__(self, a, cid=5, layer=0, filled=0):
        self.a = a
        self.w_np = gen.attn_weights(a, cid, layer)
        self.w = {"norm_w": dev(self.w_np["norm_w"]), "qkv_q": dev(self.w_np["qkv_q"]),
                  "qkv_s": dev_u16(self.w_np["qkv_s"]), "o_q": dev(self.w_np["o_q"]),
                  "o_s": dev_u16(self.w_np["o_s"])}
        self.kc_np, self.vc_np = gen.kv_cache(a, filled, cid, layer)
        self.kc, self.vc = dev_u16(self.kc_np), dev_u16(self.vc_np)
        self.ws = torch.zeros(api.moe_attn_workspace_bytes(a), dtype=torch.uint8, device=DEV)

    def run(self, x_np, pos, in_place=False):
        x = dev(x_np.astype(np.float32))
        y = x if in_place else torch.full_like(x, float("nan"))
        api.moe_attn_decode(self.a, self.w, self.kc, self.vc, pos, x, y, self.ws)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def cache(self):
        return (self.kc.cpu().numpy().view(np.float16), self.vc.cpu().numpy().view(np.float16))


def check(st, pos, sub, in_place=False):
    a = st.a
    x = gen.x_fp32(1, a.hidden, 5, sub=sub)[0]
    kc0, vc0 = st.cache()
    y = st.run(x, pos, in_place)
    ref = attn.decode_step(x, st.w_np, st.kc_np, st.vc_np, pos, a)
    print(f"attn case H={a.hidden} nh={a.n_heads} nkv={a.n_kv_heads} d={a.head_dim} pos={pos}", flush=True)
    assert_close(y - x.astype(np.float64), ref["o"], f"o pos={pos}")
    assert_close(y, ref["y"], f"y pos={pos}")
    kc, vc = st.cache()
    assert_close(kc[:, pos], ref["k"], f"k[{pos}]")
    assert_close(vc[:, pos], ref["v"], f"v[{pos}]")
    others = np.ones(a.max_ctx, bool)
    others[pos] = False
    assert np.array_equal(kc[:, others], kc0[:, others]) and np.array_equal(vc[:, others], vc0[:, others])
    # continue from the GPU's own cache row (both sides then hold the same bits)
    st.kc_np[:, pos], st.vc_np[:, pos] = kc[:, pos], vc[:, pos]
    return y


@pytest.mark.parametrize("pos", [0, 1, 37, 511])
def test_small_shape_one_split(pos):
    st = Step(SMALL_ATTN, filled=pos)
    check(st, pos, pos)


@pytest.mark.parametrize("pos", [0, 127, 128, 1000, 4095])
def test_gemma_shape_splits(pos):
    # 128 positions per split at d = 256: pos 128 leaves a last split of one
    # position, 4095 fills 32 splits
    st = Step(GEMMA_ATTN, filled=pos)
    check(st, pos, pos)


# The longest context the Gemma-shaped step takes (max_ctx = 128 splits of
# 128 positions at d = 256): half of it and its last position.
@pytest.mark.parametrize("pos", [8192, 16383])
def test_gemma_shape_longest_context(pos):
    a = AttnShape(hidden=GEMMA_ATTN.hidden, n_heads=GEMMA_ATTN.n_heads, n_kv_heads=GEMMA_ATTN.n_kv_heads,
                  head_dim=GEMMA_ATTN.head_dim, max_ctx=16384)
    st = Step(a, filled=pos)
    check(st, pos, pos)


@pytest.mark.parametrize("a,pos", [(WIDE_GROUP, 300), (WIDE_GROUP, 1023), (MHA, 1500), (MHA, 3),
                                   (ONE_HEAD, 1099), (ONE_HEAD, 600), (WIDEST, 639), (WIDEST, 64)])
def test_group_sizes_and_widths(a, pos):
    st = Step(a, filled=pos)
    check(st, pos, pos)


def test_consecutive_steps_fill_an_empty_cache_and_run_in_place():
    st = Step(SMALL_ATTN, filled=0)
    for pos in range(12):
        check(st, pos, 100 + pos, in_place=pos % 2 == 1)
    kc, vc = st.cache()
    assert np.all(kc[:, 12:] == 0) and np.all(vc[:, 12:] == 0)


def test_same_inputs_same_bits_across_split_counts():
    st = Step(GEMMA_ATTN, filled=2000)
    x = gen.x_fp32(1, GEMMA_ATTN.hidden, 5, sub=7)[0]
    y1 = st.run(x, 2000)
    y2 = st.run(x, 2000)
    assert np.array_equal(y1, y2)


def test_captured_step_replays_equal_eager_calls():
    """A graph of two layers' attention steps at a fixed position, replayed
    with new inputs, gives the eager calls' bits (and writes the same cache row)."""
    a = GEMMA_ATTN
    pos = 700
    eager = [Step(a, layer=l, filled=pos) for l in range(2)]
    graph = [Step(a, layer=l, filled=pos) for l in range(2)]
    xg = torch.empty((a.hidden,), device=DEV)
    mid = torch.empty_like(xg)
    yg = torch.empty_like(xg)
    cap = torch.cuda.Stream()

    def run(steps, x, m, y, stream=None):
        api.moe_attn_decode(a, steps[0].w, steps[0].kc, steps[0].vc, pos, x, m, steps[0].ws, stream=stream)
        api.moe_attn_decode(a, steps[1].w, steps[1].kc, steps[1].vc, pos, m, y, steps[1].ws, stream=stream)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run(graph, xg, mid, yg, stream=cap)
    torch.cuda.synchronize()
    for t in range(3):
        print(f"attn graph replay {t}", flush=True)
        x = dev(gen.x_fp32(1, a.hidden, 5, sub=50 + t)[0])
        xg.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        m2, y2 = torch.empty_like(x), torch.empty_like(x)
        run(eager, x, m2, y2)
        torch.cuda.synchronize()
        assert torch.equal(yg, y2), t
        for se, sg in zip(eager, graph):
            ke, ve = se.cache()
            kg, vg = sg.cache()
            assert np.array_equal(ke[:, pos], kg[:, pos]) and np.array_equal(ve[:, pos], vg[:, pos])
    del g
