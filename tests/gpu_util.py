"""Helpers for the GPU parity tests: upload seeded inputs, poison outputs, compare."""
import numpy as np
import torch

from bit_quantized_expert_softmax_amd import api

DEV = "cuda:0"


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_u16(a: np.ndarray) -> torch.Tensor:
    """fp16 / bf16 bit patterns as an int16 device tensor."""
    return dev(np.ascontiguousarray(a).view(np.int16))


def pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = a
    return t


def poisoned(shape, dtype=torch.float32) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=DEV)
    if dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(-7777)
    return t


def assert_close(gpu, ref, what="", rel=1e-3, abs_=1e-5):
    """max|gpu - ref| <= rel * max|ref| + abs_ (the parity bar for floating point)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.max(np.abs(g - r)) if g.size else 0.0
    bound = rel * (np.max(np.abs(r)) if r.size else 0.0) + abs_
    assert err <= bound, f"{what}: max err {err:.3e} > bound {bound:.3e}"
    return err / max(bound, 1e-300)


class Layer:
    """Owns the device copies of one layer's inputs and a libmoedecode handle."""

    def __init__(self, shape, d, *, bias=None, cache_slots=0, max_B=1, max_T=0, copy_stream=None,
                 store=None, store_layer=0, cache_policy=0, cache_on_device=False):
        self.shape = shape
        self.router = dev_u16(d["router"])
        self.shared = dev(d["shared"])
        self.bias = dev(bias) if bias is not None else None
        self.ws = torch.zeros(api.moe_layer_workspace_bytes(shape, max_B, max_T), dtype=torch.uint8,
                              device=DEV)
        if cache_slots:
            # misses from pinned host memory, or (store given) from an expert file
            self.host = pinned(d["experts"]) if store is None else None
            self.pool = torch.zeros((cache_slots, d["experts"].shape[1]), dtype=torch.uint8, device=DEV)
            self.copy_stream = copy_stream or torch.cuda.Stream()
            self.h = api.moe_layer_create(shape, router=self.router, shared_blob=self.shared,
                                          workspace=self.ws, bias=self.bias, experts_host=self.host,
                                          slot_pool=self.pool, n_slots=cache_slots,
                                          copy_stream=self.copy_stream, max_B=max_B, max_T=max_T,
                                          store=store, store_layer=store_layer, cache_policy=cache_policy,
                                          cache_on_device=cache_on_device)
        else:
            self.experts = dev(d["experts"])
            self.h = api.moe_layer_create(shape, router=self.router, shared_blob=self.shared,
                                          workspace=self.ws, bias=self.bias, experts_dev=self.experts,
                                          max_B=max_B, max_T=max_T)

    def close(self):
        if self.h:
            api.moe_layer_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
