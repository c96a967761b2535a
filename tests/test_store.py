"""The expert file store (host only): blobs read back with parallel pread equal
the bytes written, for every reader count, with and without unbuffered reads,
from concurrent callers; bad arguments and short files are refused."""
import os
import threading

import numpy as np
import pytest

from bit_quantized_expert_softmax_amd import api
from synth import gen
from synth.configs import SMALL_LAYER

LAYERS, E = 3, SMALL_LAYER.n_experts
BLOB = gen.blob_bytes(SMALL_LAYER.hidden, SMALL_LAYER.inter)


def aligned(n, align=4096):
    """A host buffer of n bytes whose address is a multiple of align."""
    raw = np.empty(n + align, np.uint8)
    off = (-raw.ctypes.data) % align
    return raw[off:off + n]


@pytest.fixture(scope="module")
def store_file(tmp_path_factory):
    stride = api.moe_store_stride(BLOB)
    rng = np.random.default_rng(7)
    data = rng.integers(0, 256, (LAYERS, E, stride), dtype=np.uint8)
    path = str(tmp_path_factory.mktemp("store") / "experts.bin")
    data.tofile(path)
    return path, data


def test_stride_is_whole_16k_pages():
    s = api.moe_store_stride(BLOB)
    assert s % 16384 == 0 and BLOB <= s < BLOB + 16384
    # the Gemma blob padded to 16 KiB pages is the pages' 3.36 MB
    assert api.moe_store_stride(3_345_408) == 3_358_720


@pytest.mark.parametrize("threads", [1, 3, 8])
@pytest.mark.parametrize("direct", [True, False])
def test_reads_equal_written_bytes(store_file, threads, direct):
    path, data = store_file
    stride = data.shape[2]
    h = api.moe_store_open(path, LAYERS, E, BLOB, threads, direct)
    try:
        rng = np.random.default_rng(threads)
        for layer in range(LAYERS):
            ids = [int(v) for v in rng.choice(E, 5, replace=False)]
            bufs = [aligned(stride) for _ in ids]
            api.moe_store_read(h, layer, ids, [b.ctypes.data for b in bufs])
            for e, b in zip(ids, bufs):
                assert np.array_equal(b, data[layer, e]), (layer, e)
        api.moe_store_read(h, 0, [], [])  # nothing to read
    finally:
        api.moe_store_close(h)


def test_concurrent_callers_are_serialised(store_file):
    path, data = store_file
    stride = data.shape[2]
    h = api.moe_store_open(path, LAYERS, E, BLOB, 4, True)
    errors = []

    def worker(seed):
        try:
            rng = np.random.default_rng(seed)
            for _ in range(20):
                layer = int(rng.integers(LAYERS))
                ids = [int(v) for v in rng.choice(E, 3, replace=False)]
                bufs = [aligned(stride) for _ in ids]
                api.moe_store_read(h, layer, ids, [b.ctypes.data for b in bufs])
                for e, b in zip(ids, bufs):
                    if not np.array_equal(b, data[layer, e]):
                        errors.append((seed, layer, e))
        except Exception as ex:  # noqa: BLE001 - reported below
            errors.append(repr(ex))

    ts = [threading.Thread(target=worker, args=(s,)) for s in range(3)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    api.moe_store_close(h)
    assert not errors, errors[:3]


def test_errors(store_file, tmp_path):
    path, data = store_file
    stride = data.shape[2]
    with pytest.raises(api.MoeError, match="cannot open"):
        api.moe_store_open(str(tmp_path / "missing.bin"), 1, E, BLOB)
    short = str(tmp_path / "short.bin")
    data[0].reshape(-1)[: E * stride - 1].tofile(short)
    with pytest.raises(api.MoeError, match="need"):
        api.moe_store_open(short, 1, E, BLOB)
    with pytest.raises(api.MoeError):
        api.moe_store_open(path, LAYERS, E, BLOB, threads=0)
    h = api.moe_store_open(path, LAYERS, E, BLOB, 2, True)
    try:
        buf = aligned(stride)
        with pytest.raises(api.MoeError, match="expert"):
            api.moe_store_read(h, 0, [E], [buf.ctypes.data])
        with pytest.raises(api.MoeError, match="layer"):
            api.moe_store_read(h, LAYERS, [0], [buf.ctypes.data])
        if api.moe_store_is_direct(h):
            odd = aligned(stride + 8)[8:]
            with pytest.raises(api.MoeError, match="aligned"):
                api.moe_store_read(h, 0, [1], [odd.ctypes.data])
    finally:
        api.moe_store_close(h)
    api.moe_store_close(None)


def test_file_layout_matches_blob_generator(tmp_path):
    """A store written from the seeded generator returns each expert's blob as
    its first blob_bytes bytes (the rest is padding)."""
    stride = api.moe_store_stride(BLOB)
    blobs = gen.expert_blobs(SMALL_LAYER, 0, 0)
    padded = np.zeros((E, stride), np.uint8)
    padded[:, :BLOB] = blobs
    path = str(tmp_path / "layer.bin")
    padded.tofile(path)
    h = api.moe_store_open(path, 1, E, BLOB, 3, True)
    try:
        bufs = [aligned(stride) for _ in range(E)]
        api.moe_store_read(h, 0, list(range(E)), [b.ctypes.data for b in bufs])
        for e in range(E):
            assert np.array_equal(bufs[e][:BLOB], blobs[e])
    finally:
        api.moe_store_close(h)
    assert os.path.getsize(path) == E * stride
