"""Pins for the oracle's int4 unpack, dequant and blob parsing (CPU only)."""
import os

import numpy as np
import pytest

from oracle import q4
from synth import gen
from synth.configs import GEMMA_LAYER, SMALL_LAYER, TINY_LAYER

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_nibbles():
    rows = []
    with open(os.path.join(GOLDEN, "nibbles.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                b, lo, hi = line.split()
                rows.append((int(b, 16), int(lo), int(hi)))
    return rows


def test_worked_bytes():
    for b, lo, hi in _golden_nibbles():
        v = q4.unpack_nibbles(np.array([[b]], np.uint8))
        assert v.tolist() == [[lo, hi]], hex(b)


def test_exhaustive_256_bytes_against_bit_arithmetic():
    # brute force: every byte, each nibble decoded as sum of weighted bits
    # (bit 3 carries weight -8 in 4-bit two's complement)
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    v = q4.unpack_nibbles(allb)[0]
    for b in range(256):
        for half in (0, 1):
            nib = (b >> (4 * half)) & 0xF
            val = -8 * ((nib >> 3) & 1) + 4 * ((nib >> 2) & 1) + 2 * ((nib >> 1) & 1) + (nib & 1)
            assert v[2 * b + half] == val


def test_round_trip_with_independent_packer():
    allb = np.arange(256, dtype=np.uint8).reshape(16, 16)
    assert np.array_equal(gen.pack_nibbles(q4.unpack_nibbles(allb)), allb)
    rng = np.random.default_rng(5)
    vals = rng.integers(-8, 8, size=(7, 64)).astype(np.int8)
    assert np.array_equal(q4.unpack_nibbles(gen.pack_nibbles(vals)), vals)


def test_dequant_uses_the_scale_of_each_group():
    # row 0: element k has nibble 1 everywhere; scale of group g is 2^g
    K = 128
    q = gen.pack_nibbles(np.ones((1, K), np.int8))
    s = np.array([[1.0, 2.0, 4.0, 8.0]], np.float16)
    w = q4.dequant(q, s)
    assert w.shape == (1, K)
    for k in range(K):
        assert w[0, k] == 2.0 ** (k // 32)


def test_dequant_exact_in_fp32():
    # a 4-bit integer times an fp16 scale needs at most 15 significant bits
    rng = np.random.default_rng(1)
    q = rng.integers(0, 256, size=(64, 256), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(64, 16)).astype(np.float16)
    w64 = q4.dequant(q, s)
    assert np.array_equal(w64.astype(np.float32).astype(np.float64), w64)


@pytest.mark.parametrize("shape", [TINY_LAYER, SMALL_LAYER])
def test_blob_parts_match_assembled_blob(shape):
    H, I = shape.hidden, shape.inter
    rng = np.random.default_rng(2)
    parts = {
        "gate_q": rng.integers(0, 256, (I, H // 2), dtype=np.uint8),
        "up_q": rng.integers(0, 256, (I, H // 2), dtype=np.uint8),
        "down_q": rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
        "gate_s": rng.uniform(0.005, 0.02, (I, H // 32)).astype(np.float16),
        "up_s": rng.uniform(0.005, 0.02, (I, H // 32)).astype(np.float16),
        "down_s": rng.uniform(0.005, 0.02, (H, I // 32)).astype(np.float16),
    }
    blob = gen.assemble_blob(H, I, parts["gate_q"], parts["gate_s"], parts["up_q"], parts["up_s"],
                             parts["down_q"], parts["down_s"])
    got = q4.blob_parts(blob, H, I)
    for k, v in parts.items():
        assert np.array_equal(got[k], v), k


def test_closed_form_bytes():
    assert q4.expert_bytes(2816, 704) == 3_345_408 == 27 * 2816 * 704 // 16
    assert q4.expert_bytes(512, 128) == 110_592
    assert q4.expert_bytes(2816, 2112) == 10_036_224
    assert gen.blob_bytes(2816, 704) == q4.expert_bytes(2816, 704)
    # every sub-array of the big blob starts on a 256-byte boundary
    lay = gen.blob_layout(GEMMA_LAYER.hidden, GEMMA_LAYER.inter)
    for name in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s"):
        assert lay[name][0] % 256 == 0


def _pages():
    out = {}
    with open(os.path.join(GOLDEN, "pages_numbers.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, val = line.split()[:2]
                out[key] = float(val)
    return out


def test_bytes_against_the_pages():
    p = _pages()
    blob = q4.expert_bytes(2816, 704)
    # payload 3.345 MB; padded to 16 KiB pages it is 3.36 MB as printed
    assert abs(blob / 1e6 - p["expert_read_mb"]) / p["expert_read_mb"] < 0.005
    padded = -(-blob // 16384) * 16384
    assert round(padded / 1e6, 2) == p["expert_read_mb"]
    # 30 layers x 128 experts plus the resident core comes to the printed 4-bit model size
    total_gb = 30 * 128 * blob / 1e9 + p["shared_core_gb"]
    assert abs(total_gb - p["model_4bit_gb"]) / p["model_4bit_gb"] < 0.01
    # the printed hit rate and read volume per token agree with 30 x 8 lookups per token
    lo = 30 * p["experts_per_token"] * (1 - p["hit_rate_hi"]) * blob / 1e6
    hi = 30 * p["experts_per_token"] * (1 - p["hit_rate_lo"]) * blob / 1e6
    assert abs(lo - p["read_per_token_lo_mb"]) / p["read_per_token_lo_mb"] < 0.05
    assert abs(hi - p["read_per_token_hi_mb"]) / p["read_per_token_hi_mb"] < 0.05


def test_layer_bytes_closed_form_and_generated_arrays():
    """The algorithmic bytes of one B=1 token-layer: k expert blobs, the shared
    blob and the fp16 router, checked against the closed form and against the
    sizes of the arrays the generator actually builds."""
    from oracle import moe
    lb = moe.layer_bytes(GEMMA_LAYER)
    assert lb == {"expert_blob": 3_345_408, "routed": 8 * 3_345_408, "shared": 10_036_224, "router": 720_896}
    assert lb["routed"] + lb["shared"] + lb["router"] == 37_520_384
    # thirty such layers per token with every expert resident
    assert 30 * (lb["routed"] + lb["shared"] + lb["router"]) == 1_125_611_520
    for sh in (SMALL_LAYER, GEMMA_LAYER):
        d = gen.layer_inputs(sh, 0) if sh is SMALL_LAYER else None
        lb = moe.layer_bytes(sh)
        if d is not None:
            assert d["experts"][0].nbytes == lb["expert_blob"]
            assert d["shared"].nbytes == lb["shared"]
            assert d["router"].nbytes == lb["router"]
            assert lb["routed"] == sh.top_k * d["experts"][0].nbytes
        # a blob is its six arrays: gate and up [I][H/2] + down [H][I/2] nibbles, one fp16 per 32
        H, I = sh.hidden, sh.inter
        assert lb["expert_blob"] == 3 * H * I // 2 + 3 * H * I // 32 * 2
