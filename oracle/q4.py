"""int4 group-quantised weights: unpack, dequantise, parse an expert blob.

The pages say only that expert weights are 4-bit ("Como executar um modelo
de 26 bilhões de parâmetros ...", section "Qual é o principal truque da
arquitetura") and that one expert is a single ~3.36 MB read ("Show HN:
mecanismo de código aberto executando Gemma 4 26B em 2 GB de RAM", section
"Abordagem técnica"). Reading taken here:

* a row of ``q`` (uint8 [N][K/2]) holds element 2j in the low 4 bits of byte j
  and element 2j+1 in the high 4 bits; each nibble is two's complement, -8..7;
* ``s`` (fp16 [N][K/32]) scales elements [32g, 32g+32) of its row;
* W[n][k] = nibble[n][k] * s[n][k // 32], and y = W @ x (row n is output n);
* blob = gate.q [I][H/2], up.q [I][H/2], down.q [H][I/2],
  gate.s [I][H/32], up.s [I][H/32], down.s [H][I/32], back to back.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def unpack_nibbles(q: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> int8 [..., K] of signed 4-bit values."""
    q = np.asarray(q, dtype=np.uint8)
    lo = (q & 0x0F).astype(np.int16)
    hi = (q >> 4).astype(np.int16)
    # two's complement of a 4-bit field: codes 8..15 stand for -8..-1
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(q.shape[:-1] + (2 * q.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant(q: np.ndarray, s: np.ndarray, group: int = GROUP) -> np.ndarray:
    """fp64 W [N][K] = nibble * scale of its group (exact: 4-bit x 11-bit)."""
    v = unpack_nibbles(q).astype(np.float64)
    n, k = v.shape
    sc = np.asarray(s).view(np.float16).astype(np.float64)
    if sc.shape != (n, k // group):
        raise ValueError(f"scale shape {sc.shape} does not match W {v.shape} with group {group}")
    return v * np.repeat(sc, group, axis=1)


def blob_parts(blob: np.ndarray, hidden: int, inter: int, group: int = GROUP) -> dict:
    """Views of the six arrays of one expert blob (uint8, 27*H*I/16 bytes)."""
    H, I = hidden, inter
    sizes = {
        "gate_q": (I, H // 2), "up_q": (I, H // 2), "down_q": (H, I // 2),
        "gate_s": (I, H // group), "up_s": (I, H // group), "down_s": (H, I // group),
    }
    blob = np.asarray(blob, dtype=np.uint8).reshape(-1)
    out, off = {}, 0
    for name in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s"):
        r, c = sizes[name]
        if name.endswith("_q"):
            nbytes = r * c
            out[name] = blob[off:off + nbytes].reshape(r, c)
        else:
            nbytes = r * c * 2
            out[name] = blob[off:off + nbytes].view(np.float16).reshape(r, c)
        off += nbytes
    if off != blob.size:
        raise ValueError(f"blob has {blob.size} bytes, layout needs {off}")
    return out


def expert_matrices(blob: np.ndarray, hidden: int, inter: int, group: int = GROUP):
    """Dequantised (Wg [I][H], Wu [I][H], Wd [H][I]) in fp64."""
    p = blob_parts(blob, hidden, inter, group)
    return (dequant(p["gate_q"], p["gate_s"], group),
            dequant(p["up_q"], p["up_s"], group),
            dequant(p["down_q"], p["down_s"], group))


def expert_bytes(hidden: int, inter: int) -> int:
    """Closed form of the blob size: 3 matrices of H*I nibbles plus 3*H*I/32 fp16 scales."""
    return 3 * hidden * inter // 2 + 3 * (hidden * inter // GROUP) * 2
