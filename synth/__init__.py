"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This module holds none of the decoder's arithmetic. It only describes the five
workloads (shapes, step counts, sampling settings) and draws their inputs from
NumPy's seeded generators:

* weights ~ N(0, 0.02) under the Qwen3 tensor names, RMSNorm weights = 1
  (stored as float32 for an fp32 model, or as bf16 bit patterns, round to
  nearest even, for a bf16 model);
* prompt token ids, uniform over the vocabulary;
* the uniforms that drive the sampler's draws;
* for the batched-decode workload: first tokens, per-sequence position
  offsets and a pre-filled K/V cache ~ N(0, 1) per head.

Every array depends only on (base seed, stream id, indices), so any subset can
be regenerated on its own (e.g. the K/V of one layer of one sequence).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "weight_names", "weight_shapes",
    "make_weights", "prompt_tokens", "uniforms", "batch_first_tokens",
    "batch_offsets", "batch_kv", "f32_to_bf16_bits", "normal", "integers",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float
    rope_theta: float
    weight_dtype: str       # "f32" | "bf16"
    kv_dtype: str           # "f32" | "bf16"
    batch: int
    prompt_len: int         # tokens prefilled per sequence (0: cache pre-filled instead)
    prefilled: int          # K/V slots pre-filled with synthetic data per sequence
    decode_steps: int
    temperature: float
    top_p: float

    @property
    def max_seq(self) -> int:
        # prompt (or pre-filled cache) plus one slot per decode step
        return self.prompt_len + self.prefilled + self.decode_steps

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_QWEN3_06B = dict(n_layers=28, hidden=1024, n_heads=16, n_kv_heads=8, head_dim=128,
                  ffn=3072, vocab=151936, rms_eps=1e-6, rope_theta=1e6,
                  weight_dtype="bf16", kv_dtype="bf16")

WORKLOADS: Dict[str, Workload] = {
    # Toy Qwen3-shaped decoder: 2 layers, vocab 8192, fp32 weights; 5-token prompt,
    # then 8 greedy decode steps.
    "toy": Workload(name="toy", seed=1001, n_layers=2, hidden=1024, n_heads=16,
                    n_kv_heads=8, head_dim=128, ffn=3072, vocab=8192, rms_eps=1e-6,
                    rope_theta=1e6, weight_dtype="f32", kv_dtype="f32", batch=1,
                    prompt_len=5, prefilled=0, decode_steps=8, temperature=0.0,
                    top_p=1.0),
    # Qwen3-0.6B shape, batch 1: 5-token prompt, 128 greedy decode steps.
    "bs1_short": Workload(name="bs1_short", seed=1002, batch=1, prompt_len=5,
                          prefilled=0, decode_steps=128, temperature=0.0, top_p=1.0,
                          **_QWEN3_06B),
    # Qwen3-0.6B shape, batch 1: 2048-token prefill, 256 decode steps at T=0.7, top-p 0.9.
    "prefill2k": Workload(name="prefill2k", seed=1003, batch=1, prompt_len=2048,
                          prefilled=0, decode_steps=256, temperature=0.7, top_p=0.9,
                          **_QWEN3_06B),
    # Qwen3-0.6B shape: 64 sequences, each with 4096 pre-filled K/V slots, 64 greedy steps.
    "bs64_ctx4k": Workload(name="bs64_ctx4k", seed=1004, batch=64, prompt_len=0,
                           prefilled=4096, decode_steps=64, temperature=0.0, top_p=1.0,
                           **_QWEN3_06B),
    # Qwen3-0.6B shape, batch 1: 32768-token prefill, 512 decode steps at T=1.0, top-p 0.95.
    "prefill32k": Workload(name="prefill32k", seed=1005, batch=1, prompt_len=32768,
                           prefilled=0, decode_steps=512, temperature=1.0, top_p=0.95,
                           **_QWEN3_06B),
}

# Position offsets of the batched workload are drawn from [0, OFFSET_MAX]: the largest
# offset keeps the last decode position (offset + 4096 + 63) below 32768.
OFFSET_MAX = 28608


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def weight_names(n_layers: int) -> List[str]:
    """Tensor names in the fixed order that also indexes the weight seeds."""
    names = ["model.embed_tokens.weight"]
    for i in range(n_layers):
        p = f"model.layers.{i}"
        names += [
            f"{p}.input_layernorm.weight",
            f"{p}.self_attn.q_proj.weight",
            f"{p}.self_attn.k_proj.weight",
            f"{p}.self_attn.v_proj.weight",
            f"{p}.self_attn.q_norm.weight",
            f"{p}.self_attn.k_norm.weight",
            f"{p}.self_attn.o_proj.weight",
            f"{p}.post_attention_layernorm.weight",
            f"{p}.mlp.gate_proj.weight",
            f"{p}.mlp.up_proj.weight",
            f"{p}.mlp.down_proj.weight",
        ]
    names.append("model.norm.weight")
    return names


def weight_shapes(w: Workload) -> Dict[str, Tuple[int, ...]]:
    d, hq, hkv, dh, f, v = w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn, w.vocab
    shapes: Dict[str, Tuple[int, ...]] = {}
    for name in weight_names(w.n_layers):
        leaf = name.split(".")[-2]
        shapes[name] = {
            "embed_tokens": (v, d),
            "input_layernorm": (d,),
            "post_attention_layernorm": (d,),
            "norm": (d,),
            "q_proj": (hq * dh, d),
            "k_proj": (hkv * dh, d),
            "v_proj": (hkv * dh, d),
            "q_norm": (dh,),
            "k_norm": (dh,),
            "o_proj": (d, hq * dh),
            "gate_proj": (f, d),
            "up_proj": (f, d),
            "down_proj": (d, f),
        }[leaf]
    return shapes


def is_norm_weight(name: str) -> bool:
    return name.endswith("norm.weight") or name.endswith("layernorm.weight")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns the uint16 bit patterns."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 22                      # work in 16 MiB slices to bound temporaries
    lsb = np.empty(min(step, flat_u.size), dtype=np.uint32)
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        t = lsb[:c.size]
        np.right_shift(c, 16, out=t)
        t &= np.uint32(1)
        c += np.uint32(0x7FFF)
        c += t
        c >>= np.uint32(16)
        flat_o[s:s + step] = c
    return out


def normal(key, shape, scale: float = 1.0) -> np.ndarray:
    """float32 N(0, scale^2) drawn from the generator seeded by `key` (a tuple of ints)."""
    rng = np.random.default_rng(list(key))
    out = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def integers(key, low: int, high: int, n: int) -> np.ndarray:
    return np.random.default_rng(list(key)).integers(low, high, n).astype(np.int32)


def make_weights(w: Workload, names: List[str] | None = None) -> Dict[str, np.ndarray]:
    """Weights of workload `w`: float32 arrays ("f32") or uint16 bf16 bit patterns ("bf16").

    Tensor i of `weight_names` is drawn from the generator seeded by (seed, 0, i).
    """
    shapes = weight_shapes(w)
    order = weight_names(w.n_layers)
    wanted = set(order if names is None else names)
    out: Dict[str, np.ndarray] = {}
    for i, name in enumerate(order):
        if name not in wanted:
            continue
        shape = shapes[name]
        if is_norm_weight(name):
            arr = np.ones(shape, dtype=np.float32)
        else:
            arr = normal((w.seed, 0, i), shape, 0.02)
        out[name] = f32_to_bf16_bits(arr) if w.weight_dtype == "bf16" else arr
    return out


def prompt_tokens(w: Workload, n: int | None = None, seq: int = 0) -> np.ndarray:
    """Prompt ids (int32), uniform over [0, vocab), for sequence `seq`."""
    n = w.prompt_len if n is None else n
    return integers((w.seed, 1, seq), 0, w.vocab, n)


def forced_tokens(w: Workload, n: int, seq: int = 0) -> np.ndarray:
    """A seeded token stream that can stand in for generated tokens (teacher forcing)."""
    return integers((w.seed, 6, seq), 0, w.vocab, n)


def uniforms(w: Workload, n: int | None = None, seq: int = 0) -> np.ndarray:
    """Per-step uniforms in [0, 1) (float32) that drive the sampler's draws."""
    n = (w.decode_steps + 1) if n is None else n
    return np.random.default_rng([w.seed, 4, seq]).random(n, dtype=np.float32)


def batch_first_tokens(w: Workload) -> np.ndarray:
    return integers((w.seed, 2), 0, w.vocab, w.batch)


def batch_offsets(w: Workload) -> np.ndarray:
    """Distinct position offsets s_b in [0, OFFSET_MAX]; sequence b decodes at s_b + prefilled + t."""
    rng = np.random.default_rng([w.seed, 5])
    return np.sort(rng.choice(OFFSET_MAX + 1, size=w.batch, replace=False)).astype(np.int32)


def batch_kv(w: Workload, layer: int, seq: int, length: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Pre-filled cache of one (layer, sequence): K, V as bf16 bits [n_kv_heads, length, head_dim]."""
    length = w.prefilled if length is None else length
    kv = normal((w.seed, 3, layer, seq), (2, w.n_kv_heads, length, w.head_dim))
    bits = f32_to_bf16_bits(kv)
    return bits[0], bits[1]
