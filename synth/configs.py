"""Layer shapes and workloads.

The Gemma-4-26B-A4B-shaped layer follows the engine described on
"Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
memória em um Mac comum" (section "Qual é o principal truque da
arquitetura": a router per layer picks 8 experts, a 16-slot LFU cache,
a shared-expert branch) with hidden 2816, 128 experts, expert
intermediate 704 and shared intermediate 2112; the small parity layer uses
hidden 512, 32 experts, intermediate 128 and shared intermediate 256.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Shape:
    hidden: int          # H, model width
    n_experts: int       # E
    top_k: int           # k experts per token
    inter: int           # I, routed expert intermediate width
    shared_inter: int    # I_s, shared expert intermediate width
    group: int = 32      # quantisation group along the input (K) axis

    def check(self) -> None:
        for k in (self.hidden, self.inter, self.shared_inter):
            if k % self.group:
                raise ValueError(f"dimension {k} is not a multiple of group {self.group}")
        if not (1 <= self.top_k <= self.n_experts):
            raise ValueError("top_k must be in [1, n_experts]")


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int       # seed-stream selector (see synth.gen)
    shape: Shape
    kind: str            # "decode", "stack", "batched", "prefill"
    tokens: int = 1
    layers: int = 1
    batches: tuple = (1,)
    n_slots: int = 0     # LFU slots per layer (stack workload)
    notes: dict = field(default_factory=dict)


@dataclass(frozen=True)
class AttnShape:
    """Attention step next to the MoE layer of one decoder layer. The pages
    name the attention, RoPE and RMSNorm kernels and an fp16 KV cache but no
    head counts; the Gemma-shaped reading below is 16 query heads sharing 8
    key/value heads (2 per group) of width 256."""
    hidden: int          # H
    n_heads: int         # query heads
    n_kv_heads: int      # key/value heads (n_heads / n_kv_heads query heads share one)
    head_dim: int        # d
    max_ctx: int         # positions the KV cache holds
    rope_theta: float = 10000.0
    eps: float = 1e-6    # RMSNorm epsilon
    group: int = 32

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def attn_width(self) -> int:
        return self.n_heads * self.head_dim


GEMMA_LAYER = Shape(hidden=2816, n_experts=128, top_k=8, inter=704, shared_inter=2112)
SMALL_LAYER = Shape(hidden=512, n_experts=32, top_k=8, inter=128, shared_inter=256)
# A hand-checkable shape for brute-force tests (explicit Python loops).
TINY_LAYER = Shape(hidden=64, n_experts=4, top_k=2, inter=32, shared_inter=64)

GEMMA_ATTN = AttnShape(hidden=2816, n_heads=16, n_kv_heads=8, head_dim=256, max_ctx=4096)
SMALL_ATTN = AttnShape(hidden=512, n_heads=4, n_kv_heads=2, head_dim=64, max_ctx=512)
# hand-checkable shape for the explicit-loop pins of the attention oracle
TINY_ATTN = AttnShape(hidden=64, n_heads=4, n_kv_heads=2, head_dim=8, max_ctx=6)

C0 = Workload("small_layer_decode_b1", 0, SMALL_LAYER, "decode", tokens=1)
C1 = Workload("gemma_layer_decode_b1", 1, GEMMA_LAYER, "decode", tokens=1000)
C2 = Workload("gemma_30layer_lfu16_decode_b1", 2, GEMMA_LAYER, "stack",
              tokens=512, layers=30, n_slots=16,
              notes={"zipf_s": 1.1, "eps_std": 0.1, "rms_eps": 1e-6})
C3 = Workload("gemma_layer_batched_decode", 3, GEMMA_LAYER, "batched",
              batches=(16, 64))
C4 = Workload("gemma_layer_prefill_2048", 4, GEMMA_LAYER, "prefill", tokens=2048)
TINY = Workload("tiny_layer", 99, TINY_LAYER, "decode", tokens=4)

CONFIGS = {w.name: w for w in (C0, C1, C2, C3, C4, TINY)}


def shape_of(name: str) -> Shape:
    return CONFIGS[name].shape
