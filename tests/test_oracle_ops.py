"""Pins of the oracle's building blocks (CPU only).

Each test fixes one property that the article or mathematics determines, chosen
so that a plausible slip (wrong eps, dropped weight, interleaved instead of
split-half RoPE, wrong rotation sign, wrong GQA head map, missing causal mask,
wrong scale) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle

F32 = np.float32


# ---------------------------------------------------------------- bf16 format

def test_round_to_bf16_ties_to_even_and_exact_values():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 1.5 * 2**-8, -2.5, 0.0, -0.0,
                  3.3895314e38], dtype=F32)
    r = oracle.round_to_bf16(x)
    expect = np.array([1.0, 1.0, 1.0 + 4 * 2**-8, 1.0 + 2**-7, -2.5, 0.0, -0.0,
                       3.3895314e38], dtype=F32)
    assert np.array_equal(r.view(np.uint32), expect.view(np.uint32))
    # widening is exact and round-trips
    bits = (r.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f32(bits).view(np.uint32), r.view(np.uint32))


def test_round_to_bf16_error_bound():
    x = np.random.default_rng(0).standard_normal(100000).astype(F32)
    r = oracle.round_to_bf16(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0**-8 + 1e-38)
    assert np.all(r.view(np.uint32) & 0xFFFF == 0)


# ---------------------------------------------------------------- RMSNorm (Step 3)

def test_rmsnorm_eps_closed_form():
    one = np.ones(1024, F32)
    y = oracle.rms_norm(np.full(1024, 1e-4, F32), one, 1e-6)
    # 1e-4 / sqrt(1e-8 + 1e-6) = 0.0995037...; eps = 1e-5 would give 0.0316
    assert np.allclose(y, 1e-4 / math.sqrt(1e-8 + 1e-6), rtol=1e-6)
    for c in (0.5, 3.0, 1e-3):
        y = oracle.rms_norm(np.full(128, c, F32), one[:128], 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-6)


def test_rmsnorm_weight_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 1024)).astype(F32)
    w = (1 + 0.1 * rng.standard_normal(1024)).astype(F32)
    unit = oracle.rms_norm(x, np.ones(1024, F32), 1e-6)
    assert np.allclose(oracle.rms_norm(x, w, 1e-6), unit * w, rtol=1e-6, atol=1e-7)
    # mean square of the unit-weight output is 1 (eps negligible at this scale)
    assert np.allclose(np.mean(unit.astype(np.float64) ** 2, axis=-1), 1.0, rtol=1e-5)
    # scale invariance when mean(x^2) >> eps
    assert np.allclose(oracle.rms_norm(7.0 * x, w, 1e-6), oracle.rms_norm(x, w, 1e-6), rtol=1e-5, atol=1e-6)


def test_rmsnorm_matches_torch_library():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 16, 128)).astype(F32) * 0.3
    w = (1 + 0.1 * rng.standard_normal(128)).astype(F32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (128,),
                                       torch.from_numpy(w).double(), eps=1e-6).numpy()
    assert np.allclose(oracle.rms_norm(x, w, 1e-6), ref, rtol=2e-6, atol=2e-7)


# ---------------------------------------------------------------- RoPE (Step 4)

def test_rope_frequencies_closed_form():
    f = oracle.rope_inv_freq(128, 1e6)
    assert f.dtype == F32 and f.shape == (64,)
    assert f[0] == 1.0
    assert abs(f[63] - 1e6 ** (-63 / 64)) <= 1e-7 * f[63] and abs(f[63] - 1.2409e-6) < 1e-10
    assert np.all(np.diff(f) < 0)
    # geometric with ratio theta^(-1/64)
    ratio = (f[1:].astype(np.float64) / f[:-1])
    assert np.allclose(ratio, 1e6 ** (-1 / 64), rtol=1e-6)


def test_rope_identity_at_position_zero_and_unit_vectors():
    f = oracle.rope_inv_freq(128, 1e6)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 1, 128)).astype(F32)
    assert np.array_equal(oracle.apply_rope(x, np.array([0]), f), x)
    p = 37
    for i in (0, 5, 63):
        e = np.zeros((1, 1, 128), F32)
        e[..., i] = 1.0
        y = oracle.apply_rope(e, np.array([p]), f)[0, 0]
        a = float(F32(p) * f[i])
        expect = np.zeros(128)
        expect[i] = math.cos(a)          # split halves: pair (i, i+64)
        expect[i + 64] = math.sin(a)     # counter-clockwise rotation
        assert np.allclose(y, expect, atol=1e-7)
        e2 = np.zeros((1, 1, 128), F32)
        e2[..., i + 64] = 1.0
        y2 = oracle.apply_rope(e2, np.array([p]), f)[0, 0]
        expect2 = np.zeros(128)
        expect2[i] = -math.sin(a)
        expect2[i + 64] = math.cos(a)
        assert np.allclose(y2, expect2, atol=1e-7)


def test_rope_preserves_norm():
    f = oracle.rope_inv_freq(128, 1e6)
    x = np.random.default_rng(4).standard_normal((3, 7, 128)).astype(F32)
    y = oracle.apply_rope(x, np.arange(1000, 1007), f)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-6)


@pytest.mark.parametrize("m,n,s", [(3, 1, 5), (100, 40, 900), (30000, 2, 3000)])
def test_rope_scores_depend_on_relative_position(m, n, s):
    f = oracle.rope_inv_freq(128, 1e6)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 128)).astype(F32)
    k = rng.standard_normal((1, 1, 128)).astype(F32)
    d1 = float(np.dot(oracle.apply_rope(q, np.array([m]), f).ravel().astype(np.float64),
                      oracle.apply_rope(k, np.array([n]), f).ravel()))
    d2 = float(np.dot(oracle.apply_rope(q, np.array([m + s]), f).ravel().astype(np.float64),
                      oracle.apply_rope(k, np.array([n + s]), f).ravel()))
    # float32 angles: each angle is rounded with ulp <= 2^-23 * position
    tol = (np.linalg.norm(q) * np.linalg.norm(k)) * (2.0**-22 * max(m, n) * 2 + 1e-6)
    assert abs(d1 - d2) <= tol


# ---------------------------------------------------------------- attention (Step 5)

def _brute_attention(q, K, V, t0):
    """float64 scalar loops: row i sees slots j <= t0+i; q head h reads kv head h // group."""
    Hq, M, dh = q.shape
    Hkv = K.shape[0]
    group = Hq // Hkv
    out = np.zeros((M, Hq * dh))
    for h in range(Hq):
        g = h // group
        for i in range(M):
            s = []
            for j in range(t0 + i + 1):
                s.append(sum(float(q[h, i, d]) * float(K[g, j, d]) for d in range(dh)) / math.sqrt(dh))
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = sum(e)
            for d in range(dh):
                out[i, h * dh + d] = sum(e[j] * float(V[g, j, d]) for j in range(len(e))) / z
    return out


@pytest.mark.parametrize("M,t0", [(1, 0), (1, 8), (7, 0), (4, 5)])
def test_attention_brute_force_tiny(M, t0):
    rng = np.random.default_rng(6 + M + t0)
    Hq, Hkv, dh = 4, 2, 8
    T = t0 + M
    q = rng.standard_normal((Hq, M, dh)).astype(F32)
    K = rng.standard_normal((Hkv, T + 2, dh)).astype(F32)   # slots beyond T must be ignored
    V = rng.standard_normal((Hkv, T + 2, dh)).astype(F32)
    got = oracle.attend(q, K[:, :T], V[:, :T], t0)
    assert np.allclose(got, _brute_attention(q, K[:, :T], V[:, :T], t0), rtol=1e-5, atol=1e-6)


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 1, 8)).astype(F32)
    K = rng.standard_normal((2, 1, 8)).astype(F32)
    V = rng.standard_normal((2, 1, 8)).astype(F32)
    o = oracle.attend(q, K, V, 0)
    for h in range(4):
        assert np.allclose(o[0, h * 8:(h + 1) * 8], V[h // 2, 0])


def test_attention_zero_query_averages_visible_values():
    # q = 0 makes every visible score equal: row i returns the mean of v_0 .. v_{t0+i}.
    rng = np.random.default_rng(8)
    t0, M = 3, 5
    q = np.zeros((4, M, 8), F32)
    K = rng.standard_normal((2, t0 + M, 8)).astype(F32)
    V = rng.standard_normal((2, t0 + M, 8)).astype(F32)
    o = oracle.attend(q, K, V, t0)
    for i in range(M):
        for h in range(4):
            assert np.allclose(o[i, h * 8:(h + 1) * 8], V[h // 2, :t0 + i + 1].mean(0), atol=1e-6)


def test_attention_gqa_head_map():
    # kv head g carries the constant value c_g: q head h must return c_{h // 2} (not c_{h % 8}).
    rng = np.random.default_rng(9)
    Hq, Hkv, T = 16, 8, 6
    q = rng.standard_normal((Hq, 2, 16)).astype(F32)
    K = rng.standard_normal((Hkv, T, 16)).astype(F32)
    c = np.arange(Hkv, dtype=F32) + 1
    V = np.broadcast_to(c[:, None, None], (Hkv, T, 16)).astype(F32)
    o = oracle.attend(q, K, V, T - 2)
    for h in range(Hq):
        assert np.allclose(o[:, h * 16:(h + 1) * 16], c[h // 2], rtol=1e-6)


def test_attention_matches_torch_sdpa_causal():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(10)
    Hq, Hkv, n, dh = 16, 8, 33, 128
    q = rng.standard_normal((Hq, n, dh)).astype(F32)
    K = rng.standard_normal((Hkv, n, dh)).astype(F32)
    V = rng.standard_normal((Hkv, n, dh)).astype(F32)
    tq = torch.from_numpy(q).double()[None]
    tk = torch.from_numpy(K).double().repeat_interleave(Hq // Hkv, dim=0)[None]
    tv = torch.from_numpy(V).double().repeat_interleave(Hq // Hkv, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0]
    ref = ref.permute(1, 0, 2).reshape(n, Hq * dh).numpy()
    assert np.allclose(oracle.attend(q, K, V, 0), ref, rtol=1e-4, atol=2e-5)
    # the same rows, computed as decode rows against a pre-filled cache
    got = np.concatenate([oracle.attend(q[:, i:i + 1], K[:, :i + 1], V[:, :i + 1], i) for i in range(n)])
    assert np.allclose(got, ref, rtol=1e-4, atol=2e-5)


def test_attention_rows_are_probability_weighted_means():
    # with V = identity-like one-hot columns, each output row is a probability vector
    rng = np.random.default_rng(11)
    T = 8
    q = rng.standard_normal((2, 3, T)).astype(F32) * 3
    K = rng.standard_normal((1, T, T)).astype(F32)
    V = np.eye(T, dtype=F32)[None]
    o = oracle.attend(q, K, V, T - 3)
    probs = o.reshape(3, 2, T)
    assert np.all(probs >= 0)
    assert np.allclose(probs.sum(-1), 1.0, atol=1e-6)
    # causal: row i puts zero weight on slots after t0 + i
    for i in range(3):
        assert np.all(probs[i, :, T - 3 + i + 1:] == 0)


# ---------------------------------------------------------------- SwiGLU (Step 6)

def test_silu_closed_forms_and_library():
    torch = pytest.importorskip("torch")
    g = np.array([0.0, 30.0, -30.0, 1.0, -1.0, 100.0, -100.0], F32)
    y = oracle.silu(g)
    assert y[0] == 0.0
    assert abs(y[1] - 30.0) < 1e-5 and abs(y[2]) < 1e-11 and y[5] == 100.0 and abs(y[6]) < 1e-40
    assert abs(y[3] - 1 / (1 + math.exp(-1))) < 1e-7
    x = np.random.default_rng(12).standard_normal(1000).astype(F32) * 4
    assert np.allclose(oracle.silu(x), torch.nn.functional.silu(torch.from_numpy(x).double()).numpy(),
                       rtol=1e-6, atol=1e-7)


def test_ffn_is_gated_product():
    rng = np.random.default_rng(13)
    h = rng.standard_normal((2, 16)).astype(F32)
    wg = rng.standard_normal((24, 16)).astype(F32)
    wu = rng.standard_normal((24, 16)).astype(F32)
    wd = rng.standard_normal((16, 24)).astype(F32)
    g = h.astype(np.float64) @ wg.T
    u = h.astype(np.float64) @ wu.T
    ref = (g / (1 + np.exp(-g)) * u) @ wd.T
    assert np.allclose(oracle.ffn_swiglu(h, wg, wu, wd), ref, rtol=1e-4, atol=1e-4)
    # swapping gate and up changes the result (the gate is the one passed through SiLU)
    assert not np.allclose(oracle.ffn_swiglu(h, wu, wg, wd), ref, rtol=1e-3, atol=1e-3)
