"""Checks on the seeded input generators (CPU only)."""
import numpy as np

from synth import gen
from synth.configs import SMALL_LAYER, GEMMA_LAYER


def test_generators_are_deterministic():
    a = gen.layer_inputs(SMALL_LAYER, 0)
    b = gen.layer_inputs(SMALL_LAYER, 0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert np.array_equal(gen.x_fp32(3, 512, 0), gen.x_fp32(3, 512, 0))
    assert not np.array_equal(gen.x_fp32(1, 512, 0), gen.x_fp32(1, 512, 1))


def test_value_distributions():
    sh = SMALL_LAYER
    ex = gen.expert_blobs(sh, 0)
    lay = gen.blob_layout(sh.hidden, sh.inter)
    s = ex[:, lay["gate_s"][0]:].copy().view(np.float16).astype(np.float64)
    assert s.min() >= 0.005 - 1e-5 and s.max() <= 0.02 + 1e-5
    q = ex[:, :lay["gate_s"][0]]
    hist = np.bincount((q & 15).reshape(-1), minlength=16)
    assert hist.min() > 0.9 * hist.mean()
    r = gen.router(sh, 0).astype(np.float64)
    assert abs(r.std() - 0.02) < 0.001
    eps = gen.eps_fp16(1, 4, 512, 2).astype(np.float64)
    assert abs(eps.std() - 0.1) < 0.01


def test_zipf_bias_is_log_of_a_normalised_power_law():
    b = gen.zipf_bias(128, 2, 0).astype(np.float64)
    p = np.exp(b)
    assert abs(p.sum() - 1.0) < 1e-5
    srt = np.sort(p)[::-1]
    r = np.arange(1, 129)
    assert np.allclose(srt / srt[0], r ** -1.1, rtol=1e-5)
    assert not np.array_equal(b, gen.zipf_bias(128, 2, 1))


def test_bf16_bits_round_trip():
    x = gen.x_bf16(4, 64, 4)
    f = gen.bf16_bits_to_f32(x)
    assert np.array_equal(gen.to_bf16_bits(f), x)


def test_blob_size_at_full_shape():
    assert gen.blob_bytes(GEMMA_LAYER.hidden, GEMMA_LAYER.inter) == 3_345_408
