"""Plain CPU oracle of the Qwen3-shaped decoder forward pass and its sampler.

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``decoder_only_amd``) never imports, calls or links it, and this package imports
nothing from the product path: the two share no code. Inputs come from ``synth``,
which holds no arithmetic of the method.

Source pages: "Inside an LLM: Pure Python Inference for Qwen3-0.6B on MLX"
(reactapp.top, English page; French and Russian translations of the same
article). Every function cites the step of that article it restates.

Arithmetic:
* model: NumPy float32 activations and float32 accumulation, from the same
  weights the GPU receives (bf16 weights are widened to float32, which is exact);
  RoPE angles in float32 as the article builds them;
* sampler: float64 masses and prefix sums;
* optional bf16 rounding (round to nearest even) of K and V as they enter the
  cache, for models whose cache is stored in bf16.

Pins: every function here is checked by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, invariants, brute-force float64
loops on tiny shapes and library special cases (torch CPU ``rms_norm``,
``scaled_dot_product_attention``, ``silu`` and the transformers Qwen3 model).
The only part without a pin is the trained-model behaviour quoted by the article
(the "Paris" probability table and the prompt's token ids): parity unpinned,
since the trained weights and the tokenizer are not available.
"""
from .model import (  # noqa: F401
    Config, KVCache, Model, apply_rope, attend, bf16_bits_to_f32, ffn_swiglu,
    rms_norm, rope_inv_freq, round_to_bf16, silu,
)
from .sampler import sample, sample_margin  # noqa: F401
