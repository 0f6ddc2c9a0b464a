"""The C ABI on the host (no GPU work): the library loads, exports every function the
headers declare, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("q3.h", "q3_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(q3_\w+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    from decoder_only_amd import q3
    if not os.path.exists(q3.LIB_PATH):
        pytest.skip("libq3.so not built")
    return q3.load_library()


def test_every_declared_symbol_is_exported(lib):
    from decoder_only_amd import q3
    declared = _declared()
    assert declared == set(q3.EXPORTS), declared ^ set(q3.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def _tiny(**kw):
    return synth.workload("toy").with_(n_layers=1, vocab=64, **kw)


def _tensors(weights):
    from decoder_only_amd import q3
    keep, arr = [], (q3.Q3Tensor * len(weights))()
    for i, (k, a) in enumerate(weights.items()):
        a = np.ascontiguousarray(a)
        keep.append(a)
        arr[i] = q3.Q3Tensor(k.encode(), a.ctypes.data, 1 if a.dtype == np.uint16 else 0, a.size)
    return arr, keep


def _load(lib, cfg, weights):
    h = ctypes.c_void_p()
    arr, keep = _tensors(weights)
    rc = lib.q3_load(ctypes.byref(cfg), arr, len(weights), None, ctypes.byref(h))
    return rc, h


def test_load_rejects_bad_config(lib):
    from decoder_only_amd import q3
    w = _tiny()
    weights = synth.make_weights(w)
    h = ctypes.c_void_p()
    assert lib.q3_load(None, None, 0, None, ctypes.byref(h)) == -1 and not h.value
    for field, bad in [("head_dim", 64), ("n_kv_heads", 3), ("tie_embeddings", 0), ("max_seq", 0),
                       ("weight_dtype", 7), ("rms_eps", 0.0)]:
        cfg = q3.config(w, 1, 8)
        setattr(cfg, field, bad)
        rc, h = _load(lib, cfg, weights)
        assert rc == -1 and not h.value, field


def test_load_rejects_missing_or_misshaped_tensor(lib):
    from decoder_only_amd import q3
    w = _tiny()
    weights = synth.make_weights(w)
    cfg = q3.config(w, 1, 8)
    partial = dict(weights)
    del partial["model.layers.0.mlp.up_proj.weight"]
    assert _load(lib, cfg, partial)[0] == -2
    wrong = dict(weights)
    wrong["model.norm.weight"] = np.ones(7, np.float32)
    assert _load(lib, cfg, wrong)[0] == -2
    wrong_dtype = dict(weights)
    wrong_dtype["model.layers.0.self_attn.q_proj.weight"] = synth.f32_to_bf16_bits(
        weights["model.layers.0.self_attn.q_proj.weight"])
    assert _load(lib, cfg, wrong_dtype)[0] == -2


def test_load_without_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from decoder_only_amd import q3
    w = _tiny()
    rc, h = _load(lib, q3.config(w, 1, 8), synth.make_weights(w))
    assert rc == -6 and not h.value


def test_null_engine_and_op_argument_errors(lib):
    assert lib.q3_prefill(None, 0, None, 1, None) == -1
    assert lib.q3_decode_step(None, None, None, 1, None) == -1
    assert lib.q3_sample(None, None, 1, 0.0, 1.0, None, None) == -1
    assert lib.q3_sync(None) == -1
    assert lib.q3_seq_len(None, 0) == -1
    assert lib.q3_last_error(None) == b"engine is NULL"
    lib.q3_free(None)
    fake = ctypes.c_void_p(0x1000)    # never dereferenced: shape checks come first
    assert lib.q3_op_gemm(fake, 1, fake, fake, 4, 100, 64, 0, 1, None, None) == -2       # N % 128
    assert lib.q3_op_gemm(fake, 1, fake, fake, 4, 128, 60, 0, 1, None, None) == -2       # K % 64
    assert lib.q3_op_gemm(None, 1, fake, fake, 4, 128, 64, 0, 1, None, None) == -1
    assert lib.q3_op_gemm(fake, 5, fake, fake, 4, 128, 64, 0, 1, None, None) == -1       # bad A dtype
    assert lib.q3_op_gemm(fake, 1, fake, fake, 4, 128, 64, 5, 0, None, None) == -1       # splits < 1
    assert lib.q3_op_gemm(fake, 1, fake, fake, 4, 128, 128, 5, 3, None, None) == -1     # splits > K / 64
    assert lib.q3_op_gemm(fake, 1, fake, fake, 4, 128, 128, 0, 2, None, None) == -1     # splits, not partials
    assert lib.q3_op_gemv(fake, 1, fake, fake, 6, 12, 1, 0, None) == -2         # K % 8
    assert lib.q3_op_attn_decode(fake, fake, fake, 1, 16, fake, 1, 16, 7, 4, fake, None) == -2
    assert lib.q3_op_attn_decode(fake, fake, fake, 1, 16, fake, 1, 16, 8, 17, fake, None) == -1
    assert lib.q3_op_attn_prefill(fake, fake, fake, 10, 8, 3, 16, 8, fake, 0, None) == -1   # t0+M > t_cap
    assert lib.q3_op_attn_prefill(fake, fake, fake, 16, 8, 3, 16, 8, fake, 1, None) == -1   # bad o dtype
    assert lib.q3_op_gemm(fake, 2, fake, fake, 4, 128, 64, 6, 1, None, None) == -1       # bad epilogue
    assert lib.q3_op_sample(fake, 1, 10, -1.0, 0.9, fake, fake, None) == -1
    assert lib.q3_op_sample(fake, 1, 10, 0.7, 0.9, None, fake, None) == -1
