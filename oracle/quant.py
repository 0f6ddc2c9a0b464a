"""Weight-only int8 and int4 quantisation of the oracle (test infrastructure only).

"Inside an LLM: Pure Python Inference for Qwen3-0.6B on MLX", "What the script leaves
out": production inference stores the weights in 8 or 4 bits. The pages give no scheme,
so the plainest one is read: symmetric, one scale per output row of each matrix (every
projection, and the embedding matrix that is also the tied LM head), no zero point.

For a row w_0 .. w_{K-1} (float32 values of the given weights) and Q = 2^(bits-1) - 1
(127 for 8 bits, 7 for 4 bits: a symmetric code range, the most negative code unused):
    s = fl32(max_k |w_k| / Q)                         (one float32 division)
    q_k = clamp(round_half_even(fl32(w_k / s)), -Q, Q)   (q = 0 for an all-zero row)
and the model then runs with the weights s * q_k. Each step is one correctly rounded
IEEE float32 operation, so any implementation of the rule gives the same codes. The
4-bit rule is the 8-bit one with Q = 7 (one scale per row as well: the pages name no
group size, and the plainest reading keeps the scheme of the 8-bit weights).
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

F32 = np.float32
QMAX = 127
QMAX4 = 7


def quantize_rows(w: np.ndarray, qmax: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric codes in [-qmax, qmax] of a [rows, K] float32 matrix: (q int8
    [rows, K], s float32 [rows])."""
    w = np.asarray(w, dtype=F32)
    amax = np.max(np.abs(w), axis=-1)
    s = (amax / F32(qmax)).astype(F32)
    safe = np.where(s > 0, s, F32(1))
    q = np.rint((w / safe[..., None]).astype(F32))
    q = np.clip(q, -qmax, qmax)
    q[s == 0] = 0
    return q.astype(np.int8), s


def quantize_rows_i8(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8 codes (Q = 127)."""
    return quantize_rows(w, QMAX)


def quantize_rows_i4(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int4 codes (Q = 7), held one per int8."""
    return quantize_rows(w, QMAX4)


def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The weights the quantised model computes with: s * q, float32."""
    return (q.astype(F32) * np.asarray(s, dtype=F32)[..., None]).astype(F32)


def is_quantized_matrix(name: str) -> bool:
    """Every matrix of the model: the embedding (tied LM head) and the seven projections
    of each layer; norm weights stay as given."""
    return not name.endswith("norm.weight") and not name.endswith("layernorm.weight")


def quantized_weights(weights: Dict[str, np.ndarray], bits: int = 8) -> Dict[str, np.ndarray]:
    """The weights of the int8 (bits = 8) or int4 (bits = 4) model as float32 arrays (s * q
    for every matrix, norm weights unchanged), under the same names; bf16 inputs are
    widened first (exact)."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    from .model import bf16_bits_to_f32
    out = {}
    for name, a in weights.items():
        a = np.asarray(a)
        f = bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(F32, copy=False)
        if is_quantized_matrix(name):
            q, s = quantize_rows(f, QMAX if bits == 8 else QMAX4)
            out[name] = dequantize_rows(q, s)
        else:
            out[name] = f
    return out
