"""The seeded input generators are deterministic and have the workloads' shapes."""
import numpy as np

import synth


def test_weights_deterministic_and_shaped():
    w = synth.workload("toy").with_(n_layers=1, vocab=256)
    a = synth.make_weights(w)
    b = synth.make_weights(w)
    shapes = synth.weight_shapes(w)
    assert list(a) == synth.weight_names(1)
    for k in a:
        assert a[k].shape == shapes[k] and np.array_equal(a[k], b[k])
        if k.endswith("norm.weight"):
            assert np.all(a[k] == 1.0)
    e = a["model.embed_tokens.weight"]
    assert abs(float(e.std()) - 0.02) < 1e-3
    # a subset regenerates the same tensors
    sub = synth.make_weights(w, names=["model.layers.0.mlp.up_proj.weight"])
    assert np.array_equal(sub["model.layers.0.mlp.up_proj.weight"], a["model.layers.0.mlp.up_proj.weight"])


def test_bf16_weights_are_rounded_fp32_draws():
    w = synth.workload("toy").with_(n_layers=1, vocab=64, weight_dtype="bf16")
    a = synth.make_weights(w)["model.layers.0.self_attn.q_proj.weight"]
    f = synth.make_weights(w.with_(weight_dtype="f32"))["model.layers.0.self_attn.q_proj.weight"]
    assert a.dtype == np.uint16
    wide = (a.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(wide - f) <= np.abs(f) * 2.0**-8)


def test_batch_workload_inputs():
    w = synth.workload("bs64_ctx4k")
    off = synth.batch_offsets(w)
    assert len(np.unique(off)) == 64 and off.min() >= 0 and off.max() <= synth.OFFSET_MAX
    assert off.max() + w.prefilled + w.decode_steps <= 32768
    t = synth.batch_first_tokens(w)
    assert t.shape == (64,) and t.min() >= 0 and t.max() < w.vocab
    k, v = synth.batch_kv(w, 3, 5, length=16)
    k2, _ = synth.batch_kv(w, 3, 5, length=16)
    assert k.shape == (8, 16, 128) and k.dtype == np.uint16 and np.array_equal(k, k2)


def test_uniforms_in_unit_interval():
    u = synth.uniforms(synth.workload("prefill2k"))
    assert u.shape == (257,) and u.dtype == np.float32 and u.min() >= 0 and u.max() < 1
