"""fp64 CPU oracle for the decode-time int4 Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call,
link or execute anything in this package; only the tests, the smoke entry
point and the benchmark's CPU-baseline leg do. It shares no code with the
HIP library (no kernels, headers, helpers or constant tables); the only
common code is the seeded input generators in ``synth``.

What is computed, and where the pages describe it:

* the router of each layer picks the 8 experts of the current token, a
  16-slot LFU expert cache is checked, misses are loaded while the GPU runs
  the shared-expert branch -- "Como executar um modelo de 26 bilhões de
  parâmetros em dois gigabytes de memória em um Mac comum", section
  "Qual é o principal truque da arquitetura" (and its German twin, section
  "Was ist der Haupt-Architekturtrick?");
* 4-bit expert weights and custom quantisation / GEMV / MoE / RMSNorm
  kernels -- same page, section "Sem dependências do llama.cpp e MLX";
* the cache keeps about 16 slots with a 60-70 % hit rate -- "Show HN:
  mecanismo de código aberto executando Gemma 4 26B em 2 GB de RAM",
  section "Abordagem técnica (MoE + streaming por SSD)";
* prefill groups rows so that one loaded expert serves a group of rows --
  the first article, section "Desempenho no mundo real".

The pages leave the arithmetic open; the readings taken (signed nibbles,
one fp16 scale per 32 inputs, softmax over the selected logits, GELU-tanh
GeGLU, weight-1 shared expert, weightless RMSNorm in the 30-layer stack,
LFU tie-breaks, bf16 rounding points of prefill) are listed with the pins
that check them in the design notes and in ``tests/test_oracle_*.py``.

Modules: ``q4`` (unpack, dequant, blob parsing), ``moe`` (routing, FFN,
combine, stack, prefill), ``lfu`` (slot-cache simulator).
"""
from . import lfu, moe, q4  # noqa: F401
