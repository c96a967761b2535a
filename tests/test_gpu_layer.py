"""GPU parity of moe_layer_decode (resident and LFU cache mode) against the oracle."""
import numpy as np
import pytest
import torch

from bit_quantized_expert_softmax_amd import api
from oracle import lfu, moe
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER
from tests.gpu_util import DEV, Layer, assert_close, dev, dev_u16, poisoned

pytestmark = pytest.mark.gpu

_CACHE = {}


def layer_data(shape, cid):
    key = (shape, cid)
    if key not in _CACHE:
        _CACHE[key] = gen.layer_inputs(shape, cid)
    return _CACHE[key]


def run_decode(L, x, flags=0, add_in=None, trace_k=0, stats=None):
    B = x.shape[0]
    sh = L.shape
    y = poisoned((B, sh.hidden))
    ids = poisoned((B, sh.top_k), torch.int32)
    w = poisoned((B, sh.top_k))
    u = poisoned((B, sh.hidden))
    tr = api.moe_layer_decode(L.h, x, add_in, B, flags, y, ids, w, u, trace_k=trace_k, stats=stats)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), u.cpu().numpy(), tr


@pytest.mark.parametrize("shape,cid,tokens", [(SMALL_LAYER, 0, 8), (GEMMA_LAYER, 1, 4)])
def test_resident_decode_b1(shape, cid, tokens):
    d = layer_data(shape, cid)
    L = Layer(shape, d)
    xs = gen.x_fp32(tokens, shape.hidden, cid)
    for t in range(tokens):
        y, ids, w, u, _ = run_decode(L, dev(xs[t:t + 1]))
        r = moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"])
        assert np.array_equal(ids, r["ids"]), t
        assert_close(w, r["w"], f"w t={t}")
        assert_close(y, r["y"], f"y t={t}")
        assert np.array_equal(u, xs[t:t + 1])
    L.close()


@pytest.mark.parametrize("cache", [False, True], ids=["resident", "cache_mode"])
def test_decode_mixed_magnitudes_in_a_group(cache):
    """u's groups of 32 mix 1e4 with 1e-3 (so do the GeGLU activations that follow)."""
    from tests.test_gpu_kernels import mixed_groups
    shape = GEMMA_LAYER
    d = layer_data(shape, 1)
    L = Layer(shape, d, cache_slots=16 if cache else 0)
    xs = mixed_groups(3, shape.hidden, 5)
    for t in range(3):
        y, ids, w, u, _ = run_decode(L, dev(xs[t:t + 1]), trace_k=shape.top_k if cache else 0)
        r = moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"])
        assert np.array_equal(ids, r["ids"]), t
        assert_close(w, r["w"], f"w t={t}")
        assert_close(y, r["y"], f"y t={t}")
    L.close()


def test_resident_decode_batched_call():
    shape = GEMMA_LAYER
    d = layer_data(shape, 1)
    L = Layer(shape, d, max_B=3)
    x = gen.x_fp32(3, shape.hidden, 1, sub=7)
    y, ids, w, _, _ = run_decode(L, dev(x))
    r = moe.layer_decode(x.astype(np.float64), shape, d["router"], d["shared"], d["experts"])
    assert np.array_equal(ids, r["ids"])
    assert_close(y, r["y"], "y B=3")
    L.close()


def test_zero_input_and_determinism():
    shape = SMALL_LAYER
    d = layer_data(shape, 0)
    L = Layer(shape, d)
    y, ids, w, _, _ = run_decode(L, torch.zeros((1, shape.hidden), device=DEV))
    assert np.all(y == 0.0) and ids[0].tolist() == list(range(8)) and np.all(w == 0.125)
    x = dev(gen.x_fp32(1, shape.hidden, 0, sub=3))
    y1 = run_decode(L, x)[0]
    y2 = run_decode(L, x)[0]
    assert np.array_equal(y1, y2)
    L.close()


@pytest.mark.parametrize("shape,cid", [(SMALL_LAYER, 0), (GEMMA_LAYER, 2)])
def test_norm_residual_perturbation(shape, cid):
    d = layer_data(shape, cid)
    bias = gen.zipf_bias(shape.n_experts, cid, 0)
    L = Layer(shape, d, bias=bias)
    xs = gen.x_fp32(3, shape.hidden, cid)
    eps = gen.eps_fp16(1, 3, shape.hidden, cid)[0]
    lay = dict(d, bias=bias)
    for t in range(3):
        y, ids, w, u, _ = run_decode(L, dev(xs[t:t + 1]), api.MOE_F_RMSNORM_IN | api.MOE_F_RESIDUAL,
                                     add_in=dev_u16(eps[t:t + 1]))
        h2, rec = moe.stack_layer_step(xs[t], eps[t], shape, lay)
        assert_close(u, rec["u"], "u")
        # routing decided on the GPU's own u (both sides select in fp64 from it)
        r_ids, r_w, _ = moe.route(u.astype(np.float64), d["router"], shape.top_k, bias)
        assert np.array_equal(ids, r_ids)
        assert np.array_equal(ids, rec["ids"])
        assert_close(w, r_w, "w")
        assert_close(y, h2, "y")
    L.close()


@pytest.mark.parametrize("fill", [0, api.MOE_F_FILL_KERNEL], ids=["copy_engine", "fill_kernel"])
@pytest.mark.parametrize("shape,cid,slots,tokens", [(SMALL_LAYER, 0, 10, 60), (GEMMA_LAYER, 2, 16, 10)])
def test_cache_mode_trace_and_output(shape, cid, slots, tokens, fill):
    d = layer_data(shape, cid)
    bias = gen.zipf_bias(shape.n_experts, cid, 0)
    L = Layer(shape, d, bias=bias, cache_slots=slots)
    xs = gen.x_fp32(tokens, shape.hidden, cid, sub=11)
    sim = lfu.LFUCache(slots, shape.n_experts)
    stats = api.moe_decode_stats()
    check = set(range(0, tokens, max(1, tokens // 6))) | {tokens - 1}
    for t in range(tokens):
        y, ids, w, u, tr = run_decode(L, dev(xs[t:t + 1]), flags=fill, trace_k=shape.top_k, stats=stats)
        r_ids, r_w, _ = moe.route(xs[t:t + 1].astype(np.float64), d["router"], shape.top_k, bias)
        assert np.array_equal(ids, r_ids), t
        want = sim.step(ids[0])
        assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in want], t
        if t in check:
            r = moe.layer_decode(xs[t].astype(np.float64), shape, d["router"], d["shared"], d["experts"],
                                 bias=bias)
            assert_close(y, r["y"], f"y t={t}")
    assert stats.hits == sim.hits and stats.misses == sim.misses and stats.calls == tokens
    assert stats.h2d_bytes == sim.misses * d["experts"].shape[1]
    assert 0 < sim.hits
    # every slot holds a bit-exact copy of the expert the cache says it holds
    pool = L.pool.cpu().numpy()
    for s_, e in enumerate(sim.expert):
        if e >= 0:
            assert np.array_equal(pool[s_], d["experts"][e]), (s_, e)
    ex, fr, la = api.moe_cache_slots(api.moe_layer_cache(L.h), slots)
    assert ex.tolist() == sim.expert and fr.tolist() == sim.freq
    L.close()


def test_fill_kernel_matches_copy_engine_bitwise():
    """Both fill paths leave the same slots and give the same bits."""
    sh = GEMMA_LAYER
    d = layer_data(sh, 2)
    bias = gen.zipf_bias(sh.n_experts, 2, 0)
    La = Layer(sh, d, bias=bias, cache_slots=16)
    Lb = Layer(sh, d, bias=bias, cache_slots=16)
    xs = gen.x_fp32(6, sh.hidden, 2, sub=12)
    for t in range(6):
        ya, ida, _, _, tra = run_decode(La, dev(xs[t:t + 1]), trace_k=sh.top_k)
        yb, idb, _, _, trb = run_decode(Lb, dev(xs[t:t + 1]), flags=api.MOE_F_FILL_KERNEL, trace_k=sh.top_k)
        assert np.array_equal(ida, idb) and np.array_equal(tra, trb), t
        assert np.array_equal(ya, yb), t
    assert np.array_equal(La.pool.cpu().numpy(), Lb.pool.cpu().numpy())
    La.close()
    Lb.close()


@pytest.mark.parametrize("flags", [0, api.MOE_F_FILL_KERNEL], ids=["copy_engine", "fill_kernel"])
def test_cache_mode_matches_resident_bitwise(flags):
    """Cache mode (top-k in its own block, the hit ranks' gate/up ahead of the
    copies and the missed ranks' after them) gives the resident path's bits,
    ids and weights, on tokens with all hits, all misses and a mix."""
    sh = GEMMA_LAYER
    d = layer_data(sh, 2)
    bias = gen.zipf_bias(sh.n_experts, 2, 0)
    R = Layer(sh, d, bias=bias)
    C = Layer(sh, d, bias=bias, cache_slots=16)
    xs = gen.x_fp32(12, sh.hidden, 2, sub=13)
    kinds = set()
    for t in range(12):
        x = dev(xs[t:t + 1])
        print(f"cache vs resident t={t} flags={flags}", flush=True)
        yr, idr, wr, _, _ = run_decode(R, x)
        yc, idc, wc, _, tr = run_decode(C, x, flags=flags, trace_k=sh.top_k)
        hits = int(sum(e[2] for e in tr.tolist()))
        kinds.add("all hit" if hits == sh.top_k else "all miss" if hits == 0 else "mixed")
        assert np.array_equal(idr, idc) and np.array_equal(wr, wc), t
        assert np.array_equal(yr, yc), t
    assert {"all miss", "mixed"} <= kinds, kinds
    R.close()
    C.close()


@pytest.mark.parametrize("flags", [0, api.MOE_F_FILL_KERNEL], ids=["copy_engine", "fill_kernel"])
def test_file_store_matches_host_memory_bitwise(tmp_path, flags):
    """Misses read from an expert file (parallel pread into pinned staging,
    layer 1 of a 2-layer file) leave the same slots and give the same bits as
    misses copied from pinned host memory, with the simulator's cache trace."""
    sh = SMALL_LAYER
    d = layer_data(sh, 2)
    bias = gen.zipf_bias(sh.n_experts, 2, 0)
    blob = d["experts"].shape[1]
    stride = api.moe_store_stride(blob)
    padded = np.zeros((2, sh.n_experts, stride), np.uint8)
    padded[0, :, :blob] = np.random.default_rng(3).integers(0, 256, (sh.n_experts, blob), dtype=np.uint8)
    padded[1, :, :blob] = d["experts"]
    path = str(tmp_path / "experts.bin")
    padded.tofile(path)
    store = api.moe_store_open(path, 2, sh.n_experts, blob, 4, True)
    La = Layer(sh, d, bias=bias, cache_slots=8)
    Lb = Layer(sh, d, bias=bias, cache_slots=8, store=store, store_layer=1)
    sim = lfu.LFUCache(8, sh.n_experts)
    xs = gen.x_fp32(12, sh.hidden, 2, sub=5)
    for t in range(12):
        ya, ida, _, _, tra = run_decode(La, dev(xs[t:t + 1]), flags=flags, trace_k=sh.top_k)
        yb, idb, _, _, trb = run_decode(Lb, dev(xs[t:t + 1]), flags=flags, trace_k=sh.top_k)
        assert np.array_equal(ida, idb) and np.array_equal(tra, trb), t
        assert [tuple(e) for e in trb.tolist()] == [tuple(e) for e in sim.step(idb[0])], t
        assert np.array_equal(ya, yb), t
    assert sim.misses > 8 and sim.hits > 0
    assert np.array_equal(La.pool.cpu().numpy(), Lb.pool.cpu().numpy())
    La.close()
    Lb.close()
    api.moe_store_close(store)


def test_lru_policy_layer_trace_and_bits():
    """A layer with the LRU policy variant follows the simulator's LRU trace
    and gives the same bits as the LFU layer (the policy only decides which
    slot holds an expert)."""
    sh = SMALL_LAYER
    d = layer_data(sh, 4)
    bias = gen.zipf_bias(sh.n_experts, 4, 0)
    La = Layer(sh, d, bias=bias, cache_slots=8)
    Lr = Layer(sh, d, bias=bias, cache_slots=8)
    api.moe_layer_destroy(Lr.h)
    Lr.h = api.moe_layer_create(sh, router=Lr.router, shared_blob=Lr.shared, workspace=Lr.ws, bias=Lr.bias,
                                experts_host=Lr.host, slot_pool=Lr.pool, n_slots=8, copy_stream=Lr.copy_stream,
                                cache_policy=api.MOE_POLICY_LRU)
    sim = lfu.LFUCache(8, sh.n_experts, policy="lru")
    xs = gen.x_fp32(16, sh.hidden, 4, sub=9)
    differs = False
    for t in range(16):
        ya, ida, _, _, tra = run_decode(La, dev(xs[t:t + 1]), trace_k=sh.top_k)
        yr, idr, _, _, trr = run_decode(Lr, dev(xs[t:t + 1]), trace_k=sh.top_k)
        assert np.array_equal(ida, idr) and np.array_equal(ya, yr), t
        assert [tuple(e) for e in trr.tolist()] == [tuple(e) for e in sim.step(idr[0])], t
        differs |= not np.array_equal(tra, trr)
    assert differs  # the two policies did take different slots on this trace
    with pytest.raises(api.MoeError):
        api.moe_layer_create(sh, router=Lr.router, shared_blob=Lr.shared, workspace=Lr.ws, experts_host=Lr.host,
                             slot_pool=Lr.pool, n_slots=8, copy_stream=Lr.copy_stream, cache_policy=7)
    La.close()
    Lr.close()


def test_fill_kernel_needs_cache_mode():
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    L = Layer(sh, d)
    y = poisoned((1, sh.hidden))
    with pytest.raises(api.MoeError):
        api.moe_layer_decode(L.h, dev(gen.x_fp32(1, sh.hidden, 0)), None, 1, api.MOE_F_FILL_KERNEL, y)
    L.close()


def test_empty_call_and_errors():
    shape = SMALL_LAYER
    d = layer_data(shape, 0)
    L = Layer(shape, d)
    x = dev(gen.x_fp32(1, shape.hidden, 0))
    y = poisoned((1, shape.hidden))
    api.moe_layer_decode(L.h, x, None, 0, 0, y)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(y))
    with pytest.raises(api.MoeError):
        api.moe_layer_decode(L.h, x, None, 2, 0, y)     # B above max_B
    with pytest.raises(api.MoeError):
        api.moe_layer_decode(L.h, x, None, 1, 16, y)    # unknown flag
    with pytest.raises(api.MoeError):
        api.moe_layer_decode(L.h, x, None, 1, 0, x)     # y aliases x
    L.close()


@pytest.mark.parametrize("mode", ["resident", "copy_engine", "batched"])
def test_nonfinite_input_gives_valid_ids_and_the_handle_recovers(mode):
    """A token whose input holds a NaN: every logit is NaN, so the ids are the
    lowest k (NaN ranks below every number, ties to the lower id), the output
    is not finite, nothing faults, and the next finite tokens decode as the
    oracle says (in cache mode the NaN token's ids step the cache like any
    other). The oracle is not defined on NaN inputs; this is a property."""
    sh = SMALL_LAYER
    d = layer_data(sh, 0)
    cache = mode == "copy_engine"
    B = 4 if mode == "batched" else 1
    L = Layer(sh, d, cache_slots=sh.top_k if cache else 0, max_B=B)
    sim = lfu.LFUCache(sh.top_k, sh.n_experts)
    xs = gen.x_fp32(3 * B, sh.hidden, 0, sub=13)
    xs[0:B, 5] = np.nan
    for t in range(3):
        x = xs[t * B:(t + 1) * B]
        y, ids, w, u, tr = run_decode(L, dev(x), trace_k=sh.top_k if cache else 0)
        if t == 0:
            assert all(ids[b].tolist() == list(range(sh.top_k)) for b in range(B))
            assert not np.isfinite(y).all()
        else:
            r = moe.layer_decode(x.astype(np.float64), sh, d["router"], d["shared"], d["experts"])
            assert np.array_equal(ids, r["ids"]), t
            assert_close(y, r["y"], f"y t={t}")
        if cache:
            assert [tuple(e) for e in tr.tolist()] == [tuple(e) for e in sim.step(ids[0])], t
    L.close()
