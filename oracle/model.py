"""NumPy float32 oracle of the Qwen3-shaped decoder (test infrastructure only).

Written from "Inside an LLM: Pure Python Inference for Qwen3-0.6B on MLX",
Steps 2-9. The forward pass composes, in the article's order:

  embedding lookup (Step 2)
  -> per block (Step 7): x += attention(rms_norm(x)); x += ffn(rms_norm(x))
       attention (Step 5): Q/K/V projections, head split, QK-norm (per head,
       before RoPE), RoPE (Step 4), KV-cache append, GQA (q head h reads kv
       head h // (n_heads / n_kv_heads)), scaled scores, causal mask, softmax,
       weighted sum of V, head merge, output projection
       ffn (Step 6): silu(x Wg^T) * (x Wu^T), then Wd
  -> final RMSNorm and LM head (Step 8), tied to the embedding matrix.

Readings of points the article leaves open (each also listed in the design notes):
* ``forward(ids, cache, pos)`` is called but never printed (Step 9). It is read
  as the composition above with positions pos, pos+1, ..., pos+len(ids)-1.
* ``seq_len`` / ``total`` in the mask are the new-row count and the cache length
  after the append. A new row i (absolute slot t0+i) sees cache slots j <= t0+i;
  this equals the article's upper-triangular mask when the cache starts empty
  and is "no mask" for a single decode row.
* The additive -1e9 mask is applied as exclusion: in float32 exp(-1e9 - max)
  is exactly 0, so both give the same probabilities.
* RoPE frequencies f_i = fl32(theta^(-i/half)) (one rounding from float64);
  angles fl32(fl32(p) * f_i) (a single float32 multiply, as the article builds
  them in float32); cos/sin evaluated in float64 and rounded to float32.
* The LM head is tied: lm_head = embed_tokens.
* A bf16 KV cache stores round_to_bf16(k) (after QK-norm and RoPE) and
  round_to_bf16(v); an fp32 cache stores them unrounded.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

F32 = np.float32


@dataclasses.dataclass(frozen=True)
class Config:
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6      # Step 3: EPS = 1e-6
    rope_theta: float = 1e6    # Step 4: THETA = 1,000,000
    kv_bf16: bool = True

    @classmethod
    def from_workload(cls, w) -> "Config":
        return cls(n_layers=w.n_layers, hidden=w.hidden, n_heads=w.n_heads,
                   n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn,
                   vocab=w.vocab, rms_eps=w.rms_eps, rope_theta=w.rope_theta,
                   kv_bf16=(w.kv_dtype == "bf16"))


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32; exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 precision (nearest, ties to even); result stays float32."""
    u = np.array(x, dtype=F32, copy=True).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(F32)


# ----------------------------------------------------------------------------
# Step 3: RMSNorm
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x*x over the last axis) + eps), then times the per-feature weight w.

    No mean subtraction and no bias (Step 3). Evaluated as (x * r) * w with
    r = 1 / sqrt(mean + eps), all in float32.
    """
    x = np.asarray(x, dtype=F32)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    r = F32(1.0) / np.sqrt(ms + F32(eps))
    return (x * r) * np.asarray(w, dtype=F32)


# ----------------------------------------------------------------------------
# Step 4: RoPE on split halves
# ----------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """f_i = theta^(-i/half) for i < half = head_dim/2, rounded once to float32."""
    half = head_dim // 2
    return np.array([theta ** (-(i / half)) for i in range(half)], dtype=np.float64).astype(F32)


def apply_rope(x: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """Rotate each (i, i+half) pair of the last axis by angle position * f_i.

    x: [..., n, head_dim] float32, positions: [n] ints. The first half x1 and the
    second half x2 become (x1 cos - x2 sin, x1 sin + x2 cos) (Step 4).
    """
    half = x.shape[-1] // 2
    ang = np.asarray(positions).astype(F32)[:, None] * inv_freq[None, :]   # float32 product
    ang64 = ang.astype(np.float64)
    cos = np.cos(ang64).astype(F32)
    sin = np.sin(ang64).astype(F32)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


# ----------------------------------------------------------------------------
# Step 5: attention core (scaled scores, causal visibility, softmax, weighted V)
# ----------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, t0: int,
           row_block: int = 512) -> np.ndarray:
    """Grouped-query attention of new rows over a KV cache.

    q: [Hq, M, dh] (rotated queries of M new rows whose slots are t0 .. t0+M-1),
    K, V: [Hkv, T, dh] with T >= t0 + M (rotated keys, values). Query head h reads
    kv head h // (Hq // Hkv): the article repeats each kv head in place.
    Scores are (q . k) * fl32(dh^-0.5); row i sees slots j <= t0 + i.
    Returns the merged heads [M, Hq*dh] (head h in columns h*dh .. h*dh+dh-1).
    Rows are independent, so they are evaluated in blocks of `row_block` rows to
    bound memory; no sum is split or reordered by this.
    """
    Hq, M, dh = q.shape
    Hkv = K.shape[0]
    group = Hq // Hkv
    scale = F32(dh ** -0.5)
    out = np.empty((M, Hq * dh), dtype=F32)
    for r0 in range(0, M, row_block):
        r1 = min(M, r0 + row_block)
        T = t0 + r1                                   # keys any row of this block may see
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(T)[None, :]
        hidden = cols > (t0 + rows)                   # causal exclusion
        for h in range(Hq):
            g = h // group
            s = (q[h, r0:r1] @ K[g, :T].T) * scale
            s[hidden] = -np.inf
            m = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - m)
            p = e / np.sum(e, axis=-1, keepdims=True, dtype=F32)
            out[r0:r1, h * dh:(h + 1) * dh] = p @ V[g, :T]
    return out


# ----------------------------------------------------------------------------
# Step 6: SwiGLU feed-forward
# ----------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), float32."""
    with np.errstate(over="ignore"):
        return g * (F32(1.0) / (F32(1.0) + np.exp(-g)))


def ffn_swiglu(h: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    gate = h @ wg.T
    up = h @ wu.T
    return (silu(gate) * up) @ wd.T


# ----------------------------------------------------------------------------
# KV cache (Step 5): per layer, per kv head, slots 0 .. length-1
# ----------------------------------------------------------------------------

class KVCache:
    """Per-sequence cache. Holds the same values the article's concatenated
    arrays would hold, in buffers reserved up to `capacity` slots."""

    def __init__(self, cfg: Config, capacity: int):
        shape = (cfg.n_layers, cfg.n_kv_heads, capacity, cfg.head_dim)
        self.K = np.zeros(shape, dtype=F32)
        self.V = np.zeros(shape, dtype=F32)
        self.length = 0
        self.capacity = capacity

    def load(self, layer: int, k: np.ndarray, v: np.ndarray, length: int) -> None:
        """Pre-fill slots 0 .. length-1 of one layer (k, v: [Hkv, length, dh] float32)."""
        self.K[layer, :, :length] = k
        self.V[layer, :, :length] = v


# ----------------------------------------------------------------------------
# The model
# ----------------------------------------------------------------------------

class Model:
    """Forward pass over float32 weights keyed by the article's tensor names."""

    def __init__(self, cfg: Config, weights: Dict[str, np.ndarray]):
        self.cfg = cfg
        f32 = {}
        for name, a in weights.items():
            a = np.asarray(a)
            f32[name] = bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(F32, copy=False)
        self.W = f32
        self.E = f32["model.embed_tokens.weight"]          # [V, d]; also the tied LM head
        self.inv_freq = rope_inv_freq(cfg.head_dim, cfg.rope_theta)

    def new_cache(self, capacity: int) -> KVCache:
        return KVCache(self.cfg, capacity)

    # Step 5 --------------------------------------------------------------
    def _qkv(self, h: np.ndarray, layer: int, positions: np.ndarray):
        c = self.cfg
        p = f"model.layers.{layer}.self_attn"
        W = self.W
        q = h @ W[f"{p}.q_proj.weight"].T
        k = h @ W[f"{p}.k_proj.weight"].T
        v = h @ W[f"{p}.v_proj.weight"].T
        M = h.shape[0]
        q = q.reshape(M, c.n_heads, c.head_dim).transpose(1, 0, 2)
        k = k.reshape(M, c.n_kv_heads, c.head_dim).transpose(1, 0, 2)
        v = v.reshape(M, c.n_kv_heads, c.head_dim).transpose(1, 0, 2)
        q = rms_norm(q, W[f"{p}.q_norm.weight"], c.rms_eps)   # QK-norm, before RoPE
        k = rms_norm(k, W[f"{p}.k_norm.weight"], c.rms_eps)
        q = apply_rope(q, positions, self.inv_freq)
        k = apply_rope(k, positions, self.inv_freq)
        if c.kv_bf16:
            k = round_to_bf16(k)
            v = round_to_bf16(v)
        return q, k, v

    def attention(self, h, layer, cache: KVCache, positions):
        c = self.cfg
        q, k, v = self._qkv(h, layer, positions)
        t0, M = cache.length, h.shape[0]
        if t0 + M > cache.capacity:
            raise ValueError("KV cache full")
        cache.K[layer, :, t0:t0 + M] = k
        cache.V[layer, :, t0:t0 + M] = v
        o = attend(q, cache.K[layer, :, :t0 + M], cache.V[layer, :, :t0 + M], t0)
        return o @ self.W[f"model.layers.{layer}.self_attn.o_proj.weight"].T

    # Step 6 --------------------------------------------------------------
    def ffn(self, h, layer):
        p = f"model.layers.{layer}.mlp"
        W = self.W
        return ffn_swiglu(h, W[f"{p}.gate_proj.weight"], W[f"{p}.up_proj.weight"],
                          W[f"{p}.down_proj.weight"])

    # Step 7 --------------------------------------------------------------
    def block(self, x, layer, cache, positions):
        p = f"model.layers.{layer}"
        eps = self.cfg.rms_eps
        h = rms_norm(x, self.W[f"{p}.input_layernorm.weight"], eps)
        x = x + self.attention(h, layer, cache, positions)
        h = rms_norm(x, self.W[f"{p}.post_attention_layernorm.weight"], eps)
        return x + self.ffn(h, layer)

    # Step 8 --------------------------------------------------------------
    def lm_head(self, x):
        h = rms_norm(x, self.W["model.norm.weight"], self.cfg.rms_eps)
        return h @ self.E.T

    # Step 9's forward(ids, cache, pos) -----------------------------------
    def forward(self, ids: Sequence[int], cache: KVCache, pos: int,
                all_logits: bool = False) -> np.ndarray:
        """Run len(ids) new tokens at positions pos.. through the model, appending
        their K/V to `cache`. Returns logits of the last row [V] (or all rows)."""
        ids = np.asarray(ids, dtype=np.int64)
        positions = pos + np.arange(len(ids))
        x = self.E[ids]                                     # Step 2: table lookup
        for layer in range(self.cfg.n_layers):
            x = self.block(x, layer, cache, positions)
        cache.length += len(ids)
        return self.lm_head(x) if all_logits else self.lm_head(x[-1:])[0]

    def forward_batch(self, ids: Sequence[int], caches: Sequence[KVCache],
                      positions: Sequence[int]) -> np.ndarray:
        """One decode row per independent sequence: row b is token ids[b] at
        position positions[b] appended to caches[b]. The projections of all rows
        share one matrix product; attention runs per row. Returns logits [B, V]."""
        c = self.cfg
        ids = np.asarray(ids, dtype=np.int64)
        pos = np.asarray(positions, dtype=np.int64)
        B = len(ids)
        x = self.E[ids]
        W = self.W
        for layer in range(c.n_layers):
            p = f"model.layers.{layer}"
            h = rms_norm(x, W[f"{p}.input_layernorm.weight"], c.rms_eps)
            o = np.empty((B, c.n_heads * c.head_dim), dtype=F32)
            # per-row QK-norm / RoPE need each row's own position
            pa = f"{p}.self_attn"
            qp = h @ W[f"{pa}.q_proj.weight"].T
            kp = h @ W[f"{pa}.k_proj.weight"].T
            vp = h @ W[f"{pa}.v_proj.weight"].T
            for b in range(B):
                q = qp[b].reshape(1, c.n_heads, c.head_dim).transpose(1, 0, 2)
                k = kp[b].reshape(1, c.n_kv_heads, c.head_dim).transpose(1, 0, 2)
                v = vp[b].reshape(1, c.n_kv_heads, c.head_dim).transpose(1, 0, 2)
                q = rms_norm(q, W[f"{pa}.q_norm.weight"], c.rms_eps)
                k = rms_norm(k, W[f"{pa}.k_norm.weight"], c.rms_eps)
                q = apply_rope(q, pos[b:b + 1], self.inv_freq)
                k = apply_rope(k, pos[b:b + 1], self.inv_freq)
                if c.kv_bf16:
                    k = round_to_bf16(k)
                    v = round_to_bf16(v)
                cache = caches[b]
                t0 = cache.length
                if t0 + 1 > cache.capacity:
                    raise ValueError("KV cache full")
                cache.K[layer, :, t0:t0 + 1] = k
                cache.V[layer, :, t0:t0 + 1] = v
                o[b] = attend(q, cache.K[layer, :, :t0 + 1], cache.V[layer, :, :t0 + 1], t0)[0]
            x = x + o @ W[f"{pa}.o_proj.weight"].T
            h = rms_norm(x, W[f"{p}.post_attention_layernorm.weight"], c.rms_eps)
            x = x + self.ffn(h, layer)
        for cache in caches:
            cache.length += 1
        return self.lm_head(x)
