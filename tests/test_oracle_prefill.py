"""Pins for the oracle's bf16 rounding and prefill (CPU only)."""
import numpy as np
import torch

from oracle import moe, q4
from synth import gen
from synth.configs import SMALL_LAYER, TINY_LAYER


def test_bf16_round_matches_library_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        rng.uniform(-1e-3, 1e-3, 1000).astype(np.float32),
        # exact halfway cases between neighbouring bf16 values
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, 3.0e38, 1e-38, 5e-40], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(moe.bf16_round(x.astype(np.float64)), ref)


def test_power_of_two_scales_are_bf16_exact():
    # a 4-bit integer times a power of two needs at most 4 significant bits
    rng = np.random.default_rng(1)
    q = rng.integers(0, 256, (16, 64), dtype=np.uint8)
    s = (2.0 ** rng.integers(-9, -5, (16, 4))).astype(np.float16)
    w = q4.dequant(q, s)
    assert np.array_equal(moe.bf16_round(w), w)


def test_unmirrored_prefill_equals_decode_oracle():
    sh = TINY_LAYER
    d = gen.layer_inputs(sh, 99)
    x = gen.bf16_bits_to_f32(gen.x_bf16(6, sh.hidden, 99)).astype(np.float64)
    logits = gen.logits_uniform(6, sh.n_experts, 99)
    a = moe.prefill(x, sh, d["shared"], d["experts"], logits_in=logits, mirror_bf16=False)
    b = moe.layer_decode_per_token(x, sh, d["router"], d["shared"], d["experts"], logits_in=logits)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)


def test_mirrored_prefill_error_bound_with_exact_weights():
    # with power-of-two scales W is bf16-exact, so only the rounding of the
    # activation a differs: |dy| <= 2^-9 * sum |w_j| |Wd| |a|
    sh = SMALL_LAYER
    d = gen.layer_inputs(sh, 0)
    lay_s = gen.blob_layout(sh.hidden, sh.shared_inter)
    lay_e = gen.blob_layout(sh.hidden, sh.inter)
    rng = np.random.default_rng(2)

    def pow2_scales(blob, lay):
        s0 = lay["gate_s"][0]
        n = (lay["total"] - s0) // 2
        blob[s0:] = (2.0 ** rng.integers(-8, -5, n)).astype(np.float16).view(np.uint8)
    shared = d["shared"].copy()
    pow2_scales(shared, lay_s)
    experts = d["experts"].copy()
    for e in range(sh.n_experts):
        pow2_scales(experts[e], lay_e)
    x = gen.bf16_bits_to_f32(gen.x_bf16(8, sh.hidden, 0)).astype(np.float64)
    logits = gen.logits_uniform(8, sh.n_experts, 0)
    a = moe.prefill(x, sh, shared, experts, logits_in=logits, mirror_bf16=True)
    b = moe.prefill(x, sh, shared, experts, logits_in=logits, mirror_bf16=False)
    # bound built from the unrounded pieces
    bound = np.zeros_like(b["y"])
    def absffn(blob, inter, rows):
        wg, wu, wd = q4.expert_matrices(blob, sh.hidden, inter)
        act = np.abs(moe.gelu_tanh(rows @ wg.T) * (rows @ wu.T))
        return act @ np.abs(wd).T
    bound += absffn(shared, sh.shared_inter, x)
    for t in range(8):
        for j in range(sh.top_k):
            bound[t] += a["w"][t, j] * absffn(experts[a["ids"][t, j]], sh.inter, x[t:t + 1])[0]
    diff = np.abs(a["y"] - b["y"])
    assert np.all(diff <= 2.0 ** -9 * bound + 1e-12)
    assert diff.max() > 0   # the activation rounding is really applied
