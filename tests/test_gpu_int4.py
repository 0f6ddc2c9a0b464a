"""Weight-only int4 decode ("Inside an LLM ...", "What the script leaves out": production
weights in 4 bits): the engine quantises the given weights at load (q3_quantize_i4's rule,
one scale per row, pinned bit-exactly to the oracle's on the CPU), packs two codes per
byte, and the persistent decode kernel streams half a byte per weight plus a scale per
row; the prefill GEMMs take the codes in bf16 with per-column scales. The oracle runs the
model with the same quantised weights. Bar: per step logits within max-abs 2e-2 and
relative L2 1e-3 for the 2-layer toy model, INT4_REL_L2 for the 28-layer one; greedy
tokens identical."""
import pytest

import synth
from e2e import failures, run_ragged, run_single

pytestmark = pytest.mark.gpu

# Relative-L2 bar of the int4 model: 1e-7 relative noise on the residual after every layer
# moves the 28-layer int4 model's logits by up to ~1.9e-3
# (tests/test_oracle_quant.py::test_int4_model_noise_floor), so the bar keeps the bf16 bar's
# ~1.6x margin over that floor.
INT4_REL_L2 = 3e-3


def _report(stats):
    worst = max(stats, key=lambda s: s.rel)
    print(f"steps={len(stats)} worst rel-L2={worst.rel:.2e} (step {worst.step}) "
          f"max-abs={max(s.max_abs for s in stats):.2e}")


@pytest.mark.parametrize("path,prompt,steps", [
    (0, 5, 16),        # short prompt in causal chunks, short-context decode, cooperative launch
    (3, 5, 16),        # the same, ordinary launch
    (3, 512, 12),      # matrix-core prefill with per-column scales, then decode
    (3, 250, 12),      # split-K attention instance
    (3, 8400, 4),      # double-buffered split-K instance (contexts above 8192 slots)
])
def test_toy_int4(path, prompt, steps):
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    stats = run_single(w, prompt, steps, decode_path=path, int4=True)
    _report(stats)
    assert not failures(stats), failures(stats)[:5]      # the 2-layer model: the bf16 bar


def test_toy_int4_from_float32_weights():
    """The engine quantises float32 matrices as well as bf16 ones (the same rule on the
    float32 values): the toy model's float32 weights, short prompt and matrix-core prefill."""
    w = synth.workload("toy").with_(weight_dtype="f32", kv_dtype="bf16")
    for prompt, steps in ((5, 8), (300, 6)):
        stats = run_single(w, prompt, steps, decode_path=3, int4=True)
        _report(stats)
        assert not failures(stats), failures(stats)[:5]


@pytest.mark.parametrize("path", [0, 3])
def test_toy_int4_ragged_rows(path):
    """Three sequences of different lengths (one past the short-context limit) decoded
    together in the persistent kernel, row by row against the oracle."""
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    stats = run_ragged(w, [7, 180, 300], 6, decode_path=path, qbits=4)
    _report(stats)
    assert not failures(stats), failures(stats)[:5]


@pytest.mark.timeout(900)
def test_qwen3_06b_shape_int4_bs1_greedy():
    """The bs1 workload (28 layers, vocab 151936, 5-token prompt, 128 greedy steps) with
    weight-only int4 weights."""
    w = synth.workload("bs1_short")
    stats = run_single(w, w.prompt_len, w.decode_steps, decode_path=3, int4=True)
    _report(stats)
    bad = [s for s in stats if s.max_abs > 2e-2 or s.rel > INT4_REL_L2 or not s.argmax_ok]
    assert not bad, bad[:5]


def test_int4_engine_limits():
    """int4 engines, like int8 ones, decode only in the persistent kernel: the
    per-operation path and more than 4 sequence slots are refused."""
    import torch
    from decoder_only_amd import q3
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16", n_layers=1, vocab=512)
    weights = synth.make_weights(w)
    with pytest.raises(q3.Q3Error) as e:
        q3.Engine(q3.config(w, 5, 16, int4=True), weights)
    assert e.value.code == -1
    eng = q3.Engine(q3.config(w, 4, 16, int4=True), weights)
    with pytest.raises(q3.Q3Error) as e:
        eng.set_decode_path(1)
    assert e.value.code == -7
    toks = torch.tensor([1, 2, 3, 4], dtype=torch.int32, device="cuda")
    eng.decode_step(toks)
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    eng.sample(out, 0.0)
    eng.sync()
    assert ((out >= 0) & (out < w.vocab)).all()
    eng.close()
