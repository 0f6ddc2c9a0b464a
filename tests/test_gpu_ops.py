"""Per-kernel parity on the GPU: each q3_op_* call against the oracle on seeded inputs.

Sizes span several tiles and a ragged tail; the full-shape cases check sampled
outputs that the oracle computes one by one.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import announce, bf16_bits, bf16_dev, f32_of_bits, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q3():
    import torch
    from decoder_only_amd import q3 as mod
    mod.load_library()
    torch.cuda.set_device(0)
    return mod


def _bf16(x):
    return synth.f32_to_bf16_bits(x)


def _pair_bits(x):
    """float32 [rows, n] -> bf16 pair rows [rows, 2n]: hi = bf16(x), lo = bf16(x - hi)."""
    hi = _bf16(x)
    lo = _bf16((x - f32_of_bits(hi)).astype(np.float32))
    return np.concatenate([hi, lo], axis=1)


def _pair_value(bits, n):
    """bf16 pair rows [rows, 2n] (as bf16 tensor bits) -> float64 hi + lo."""
    return f32_of_bits(bits[:, :n]).astype(np.float64) + f32_of_bits(bits[:, n:]).astype(np.float64)


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("rows,d", [(1, 1024), (37, 1024), (5, 3072)])
def test_rmsnorm(q3, rows, d):
    import torch
    announce("rmsnorm", rows, d)
    x = synth.normal((1, rows, d), (rows, d), 0.7)
    w = (1 + 0.1 * synth.normal((2, d), (d,))).astype(np.float32)
    ref = oracle.rms_norm(x, w, 1e-6)
    xt, wt = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    out = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    q3.op_rmsnorm(xt, wt, out, 1e-6)
    outb = torch.empty(rows, d, dtype=torch.bfloat16, device="cuda")
    q3.op_rmsnorm(xt, wt, outb, 1e-6)
    torch.cuda.synchronize()
    assert np.allclose(out.cpu().numpy(), ref, rtol=2e-6, atol=1e-6)
    gotb = f32_of_bits(bf16_bits(outb))
    assert np.all(np.abs(gotb - ref) <= np.abs(ref) * 2.0**-8 + 1e-30)
    outp = torch.empty(rows, 2 * d, dtype=torch.bfloat16, device="cuda")
    q3.op_rmsnorm(xt, wt, outp, 1e-6, pair=True)
    torch.cuda.synchronize()
    # the pair carries the float32 result to ~2^-16 of its size
    f = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(_pair_value(bf16_bits(outp), d) - f) <= np.abs(f) * 2.0**-16 + 1e-30)


# ------------------------------------------------------------------ GEMV (decode projections)

@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("N,K,B", [(4096, 1024, 1), (1024, 2048, 3), (1024, 3072, 8), (2048, 1024, 13)])
def test_gemv_store_and_residual(q3, wdt, N, K, B):
    import torch
    announce("gemv", wdt, N, K, B)
    W = synth.normal((3, N, K), (N, K), 0.02)
    if wdt == "bf16":
        Wb = _bf16(W)
        W = f32_of_bits(Wb)
        Wt = bf16_dev(Wb)
    else:
        Wt = torch.from_numpy(W).cuda()
    x = synth.normal((4, B, K), (B, K))
    ref = (x.astype(np.float64) @ W.T.astype(np.float64))
    xt = torch.from_numpy(x).cuda()
    y = torch.empty(B, N, dtype=torch.float32, device="cuda")
    q3.op_gemv(Wt, xt, y, q3.GEMV_STORE)
    r0 = synth.normal((5, B, N), (B, N))
    yr = torch.from_numpy(r0).cuda()
    q3.op_gemv(Wt, xt, yr, q3.GEMV_RESID)
    torch.cuda.synchronize()
    scale = np.sqrt(K) * 0.02
    assert np.abs(y.cpu().numpy() - ref).max() <= 1e-5 * scale
    assert np.abs(yr.cpu().numpy() - (ref + r0)).max() <= 1e-5 * scale + 1e-6


@pytest.mark.parametrize("B", [1, 9])
def test_gemv_swiglu(q3, B):
    import torch
    announce("gemv swiglu", B)
    F, K = 3072, 1024
    g = f32_of_bits(_bf16(synth.normal((6, F, K), (F, K), 0.02)))
    u = f32_of_bits(_bf16(synth.normal((7, F, K), (F, K), 0.02)))
    packed = np.empty((2 * F, K), np.float32)
    for j in range(F // 16):
        packed[32 * j:32 * j + 16] = g[16 * j:16 * j + 16]
        packed[32 * j + 16:32 * j + 32] = u[16 * j:16 * j + 16]
    x = synth.normal((8, B, K), (B, K))
    ref = oracle.silu(x @ g.T) * (x @ u.T)
    y = torch.empty(B, F, dtype=torch.float32, device="cuda")
    q3.op_gemv(bf16_dev(_bf16(packed)), torch.from_numpy(x).cuda(), y, q3.GEMV_SWIGLU)
    torch.cuda.synchronize()
    assert np.allclose(y.cpu().numpy(), ref, rtol=1e-4, atol=1e-5)


# ------------------------------------------------------------------ GEMM (prefill, matrix cores)

def _pack_gate_up(g, u):
    F, K = g.shape
    packed = np.empty((2 * F, K), np.float32)
    for j in range(F // 16):
        packed[32 * j:32 * j + 16] = g[16 * j:16 * j + 16]
        packed[32 * j + 16:32 * j + 32] = u[16 * j:16 * j + 16]
    return packed


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (77, 1024, 2048), (300, 4096, 1024), (129, 1024, 3072)])
def test_gemm_bf16_activations(q3, M, N, K):
    import torch
    announce("gemm bf16-A", M, N, K)
    A = _bf16(synth.normal((10, M, K), (M, K)))
    W = _bf16(synth.normal((11, N, K), (N, K), 0.02))
    ref = f32_of_bits(A).astype(np.float64) @ f32_of_bits(W).T.astype(np.float64)
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    q3.op_gemm(bf16_dev(A), bf16_dev(W), C, q3.GEMM_F32)
    Cb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    q3.op_gemm(bf16_dev(A), bf16_dev(W), Cb, q3.GEMM_BF16)
    torch.cuda.synchronize()
    scale = np.sqrt(K) * 0.02
    assert np.abs(C.cpu().numpy() - ref).max() <= 2e-5 * scale
    gb = f32_of_bits(bf16_bits(Cb))
    assert np.all(np.abs(gb - ref) <= np.abs(ref) * 2.0**-8 + 1e-5 * scale)


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (77, 1024, 2048), (300, 4096, 1024), (129, 1024, 3072)])
def test_gemm_f32_activations_split(q3, M, N, K):
    """float32 A enters as bf16 hi + lo: the product keeps ~16 bits of A."""
    import torch
    announce("gemm f32-A", M, N, K)
    A = synth.normal((19, M, K), (M, K))
    W = _bf16(synth.normal((11, N, K), (N, K), 0.02))
    ref = A.astype(np.float64) @ f32_of_bits(W).T.astype(np.float64)
    At, Wt = torch.from_numpy(A).cuda(), bf16_dev(W)
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    q3.op_gemm(At, Wt, C, q3.GEMM_F32)
    R0 = synth.normal((12, M, N), (M, N))
    Cr = torch.from_numpy(R0).cuda()
    q3.op_gemm(At, Wt, Cr, q3.GEMM_RESID_F32)
    torch.cuda.synchronize()
    scale = np.sqrt(K) * 0.02
    err = np.abs(C.cpu().numpy() - ref).max()
    assert err <= 3e-5 * scale, err
    assert np.abs(Cr.cpu().numpy() - (ref + R0)).max() <= 3e-5 * scale + 1e-6
    # a single bf16 rounding of A would be ~100x worse: the split is really in effect
    single = f32_of_bits(_bf16(A)).astype(np.float64) @ f32_of_bits(W).T.astype(np.float64)
    assert np.abs(single - ref).max() > 20 * err


@pytest.mark.parametrize("M,N,K", [(77, 1024, 2048), (300, 1024, 3072), (2047, 4096, 1024)])
def test_gemm_pair_activations_equal_split(q3, M, N, K):
    """A handed over as bf16 pair rows gives exactly the products of float32 A split while
    staging (same hi / lo parts, same matrix-core sequence); 2047 x 4096 takes 128-row tiles,
    the others 64-row tiles."""
    import torch
    announce("gemm pair-A", M, N, K)
    A = synth.normal((19, M, K), (M, K))
    W = bf16_dev(_bf16(synth.normal((11, N, K), (N, K), 0.02)))
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    q3.op_gemm(torch.from_numpy(A).cuda(), W, C, q3.GEMM_F32)
    Cp = torch.empty(M, N, dtype=torch.float32, device="cuda")
    q3.op_gemm(bf16_dev(_pair_bits(A)), W, Cp, q3.GEMM_F32, a_pair=True)
    torch.cuda.synchronize()
    assert torch.equal(C, Cp)
    rows = [0, M // 2, M - 1]
    ref = A[rows].astype(np.float64) @ f32_of_bits(bf16_bits(W)).T.astype(np.float64)
    assert np.abs(Cp.cpu().numpy()[rows] - ref).max() <= 3e-5 * np.sqrt(K) * 0.02


# Prefill shapes (QKV and gate/up at 2047 rows) and ragged ones.
EPILOGUE_SHAPES = [(2047, 4096, 1024), (2047, 6144, 1024), (1000, 1024, 3072), (129, 256, 2048)]


@pytest.mark.parametrize("M,N,K", EPILOGUE_SHAPES)
def test_gemm_pair_epilogues_equal_split(q3, M, N, K):
    """Every epilogue, with and without column scales (the int8 weights' row scales): pair-A
    products equal, bit for bit, float32-A products split into the same hi / lo parts while
    staging (the same matrix-core sequence per output); sampled rows also against a float64
    product."""
    import torch
    announce("gemm epilogues", M, N, K)
    A = synth.normal((21, M, K), (M, K))
    Wf = f32_of_bits(_bf16(synth.normal((22, N, K), (N, K), 0.02)))
    W = bf16_dev(_bf16(Wf))
    At, Ap = torch.from_numpy(A).cuda(), bf16_dev(_pair_bits(A))
    cs = torch.from_numpy(synth.normal((24, N), (N,)).astype(np.float32)).cuda()
    R = torch.from_numpy(synth.normal((23, M, N), (M, N))).cuda()
    cases = [(q3.GEMM_F32, (M, N), torch.float32), (q3.GEMM_BF16, (M, N), torch.bfloat16),
             (q3.GEMM_SWIGLU_F32, (M, N // 2), torch.float32), (q3.GEMM_SWIGLU_PAIR, (M, N), torch.bfloat16),
             (q3.GEMM_RESID_F32, (M, N), torch.float32)]
    for epi, shape, dt in cases:
        for scale in (None, cs):
            C1 = R.clone() if epi == q3.GEMM_RESID_F32 else torch.empty(shape, dtype=dt, device="cuda")
            C2 = C1.clone()
            q3.op_gemm(At, W, C1, epi, colscale=scale)
            q3.op_gemm(Ap, W, C2, epi, a_pair=True, colscale=scale)
            torch.cuda.synchronize()
            assert torch.equal(C1, C2), (epi, scale is not None)
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    q3.op_gemm(Ap, W, C, q3.GEMM_F32, a_pair=True)
    rows = [0, 1, M // 2, M - 2, M - 1]
    ref = A[rows].astype(np.float64) @ Wf.T.astype(np.float64)
    assert np.abs(C.cpu().numpy()[rows] - ref).max() <= 3e-5 * np.sqrt(K) * 0.02


@pytest.mark.parametrize("M,N,K,S", [(2047, 1024, 2048, 2), (2047, 1024, 3072, 3), (300, 1024, 3072, 4),
                                     (1000, 1024, 2048, 32)])
def test_gemm_split_k_partials(q3, M, N, K, S):
    """Split-K partials (the prefill O and down projections): partial z is the product over
    the 64-wide k-tiles [z n / S, (z+1) n / S), n = K / 64, checked against float64 on
    sampled rows, and equal bit for bit between pair A and float32 A."""
    import torch
    announce("gemm split-K", M, N, K, S)
    A = synth.normal((25, M, K), (M, K))
    Wf = f32_of_bits(_bf16(synth.normal((26, N, K), (N, K), 0.02)))
    W = bf16_dev(_bf16(Wf))
    P1 = torch.empty(S, M, N, dtype=torch.float32, device="cuda")
    P2 = torch.empty_like(P1)
    q3.op_gemm(torch.from_numpy(A).cuda(), W, P1, q3.GEMM_PARTIAL_F32, splits=S)
    q3.op_gemm(bf16_dev(_pair_bits(A)), W, P2, q3.GEMM_PARTIAL_F32, a_pair=True, splits=S)
    torch.cuda.synchronize()
    assert torch.equal(P1, P2)
    got = P2.cpu().numpy()
    n = K // 64
    rows = [0, M // 3, M - 1]
    for z in range(S):
        k0, k1 = 64 * (n * z // S), 64 * (n * (z + 1) // S)
        ref = A[rows, k0:k1].astype(np.float64) @ Wf[:, k0:k1].T.astype(np.float64)
        assert np.abs(got[z][rows] - ref).max() <= 3e-5 * np.sqrt(max(k1 - k0, 1)) * 0.02, z
    with pytest.raises(q3.Q3Error):
        q3.op_gemm(bf16_dev(_pair_bits(A)), W, P2, q3.GEMM_F32, a_pair=True, splits=2)


def test_gemm_swiglu(q3):
    import torch
    announce("gemm swiglu")
    M, F, K = 200, 3072, 1024
    g = f32_of_bits(_bf16(synth.normal((13, F, K), (F, K), 0.02)))
    u = f32_of_bits(_bf16(synth.normal((14, F, K), (F, K), 0.02)))
    A = synth.normal((15, M, K), (M, K))
    ref = oracle.silu(A @ g.T) * (A @ u.T)
    C = torch.empty(M, F, dtype=torch.float32, device="cuda")
    Wp = bf16_dev(_bf16(_pack_gate_up(g, u)))
    q3.op_gemm(torch.from_numpy(A).cuda(), Wp, C, q3.GEMM_SWIGLU_F32)
    Cp = torch.empty(M, 2 * F, dtype=torch.bfloat16, device="cuda")
    q3.op_gemm(torch.from_numpy(A).cuda(), Wp, Cp, q3.GEMM_SWIGLU_PAIR)
    torch.cuda.synchronize()
    f = C.cpu().numpy()
    assert np.allclose(f, ref, rtol=1e-4, atol=2e-5)
    assert np.all(np.abs(_pair_value(bf16_bits(Cp), F) - f) <= np.abs(f) * 2.0**-16 + 1e-30)


def test_gemm_full_prefill_shape_sampled_rows(q3):
    import torch
    announce("gemm 32767x4096x1024 sampled")
    M, N, K = 32767, 4096, 1024
    A = synth.normal((16, M, K), (M, K))
    W = _bf16(synth.normal((17, N, K), (N, K), 0.02))
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    q3.op_gemm(torch.from_numpy(A).cuda(), bf16_dev(W), C, q3.GEMM_F32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(18).integers(0, M, 200), [0, 127, 128, M - 1]]))
    ref = A[rows].astype(np.float64) @ f32_of_bits(W).T.astype(np.float64)
    assert np.abs(C.cpu().numpy()[rows] - ref).max() <= 3e-5 * np.sqrt(K) * 0.02


# ------------------------------------------------------------------ QK-norm + RoPE + KV append

@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_qk_norm_rope_append(q3, kv):
    import torch
    announce("qk_norm_rope", kv)
    B, Hq, Hkv, T = 4, 16, 8, 40
    qkv = synth.normal((20, B), (B, (Hq + 2 * Hkv) * 128), 0.6)
    qn = (1 + 0.1 * synth.normal((21,), (128,))).astype(np.float32)
    kn = (1 + 0.1 * synth.normal((22,), (128,))).astype(np.float32)
    pos = np.array([0, 7, 4097, 33279], np.int32)
    slots = np.array([0, 39, 5, 17], np.int32)
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    kc = torch.zeros(B, Hkv, T, 128, dtype=dt, device="cuda")
    vc = torch.zeros(B, Hkv, T, 128, dtype=dt, device="cuda")
    qo = torch.empty(B, Hq, 128, dtype=torch.float32, device="cuda")
    q3.op_qk_norm_rope(torch.from_numpy(qkv).cuda(), torch.from_numpy(qn).cuda(), torch.from_numpy(kn).cuda(),
                       torch.from_numpy(pos).cuda(), torch.from_numpy(slots).cuda(), Hq, Hkv, 1e-6, 1e6,
                       qo, kc, vc)
    torch.cuda.synchronize()
    f = oracle.rope_inv_freq(128, 1e6)
    kcf = kc.float().cpu().numpy()
    vcf = vc.float().cpu().numpy()
    for b in range(B):
        q = qkv[b, :Hq * 128].reshape(Hq, 1, 128)
        k = qkv[b, Hq * 128:(Hq + Hkv) * 128].reshape(Hkv, 1, 128)
        v = qkv[b, (Hq + Hkv) * 128:].reshape(Hkv, 1, 128)
        qr = oracle.apply_rope(oracle.rms_norm(q, qn, 1e-6), pos[b:b + 1], f)[:, 0]
        kr = oracle.apply_rope(oracle.rms_norm(k, kn, 1e-6), pos[b:b + 1], f)[:, 0]
        assert np.allclose(qo[b].cpu().numpy(), qr, rtol=1e-5, atol=2e-6)
        if kv == "bf16":
            kr_b = oracle.round_to_bf16(kr)
            # rounding may flip by one bf16 ulp where the float32 inputs differ in the last bit
            assert np.all(np.abs(kcf[b, :, slots[b]] - kr_b) <= np.abs(kr_b) * 2.0**-7 + 1e-30)
            assert np.mean(kcf[b, :, slots[b]] == kr_b) > 0.99
            assert np.array_equal(vcf[b, :, slots[b]], oracle.round_to_bf16(v[:, 0]))
        else:
            assert np.allclose(kcf[b, :, slots[b]], kr, rtol=1e-5, atol=2e-6)
            assert np.array_equal(vcf[b, :, slots[b]], v[:, 0])
        others = np.setdiff1d(np.arange(T), [slots[b]])
        assert np.all(kcf[b][:, others] == 0) and np.all(vcf[b][:, others] == 0)


# ------------------------------------------------------------------ decode attention (split-K)

@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("lens", [[1], [1, 300, 1000], [257, 256, 255, 513]])
def test_attn_decode(q3, kv, lens):
    import torch
    announce("attn_decode", kv, lens)
    B, Hq, Hkv = len(lens), 16, 8
    t_cap = max(lens) + 3
    q = synth.normal((30, B), (B, Hq, 128))
    K = synth.normal((31, B), (B, Hkv, t_cap, 128))
    V = synth.normal((32, B), (B, Hkv, t_cap, 128))
    if kv == "bf16":
        K, V = oracle.round_to_bf16(K), oracle.round_to_bf16(V)
        dt = torch.bfloat16
    else:
        dt = torch.float32
    o = torch.empty(B, Hq * 128, dtype=torch.float32, device="cuda")
    q3.op_attn_decode(torch.from_numpy(q).cuda(), torch.from_numpy(K).to(dt).cuda(), torch.from_numpy(V).to(dt).cuda(),
                      torch.tensor(lens, dtype=torch.int32, device="cuda"), o, max(lens))
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    for b, T in enumerate(lens):
        ref = oracle.attend(q[b][:, None, :], K[b, :, :T], V[b, :, :T], T - 1)[0]
        assert np.allclose(got[b], ref, rtol=1e-4, atol=2e-5), (b, np.abs(got[b] - ref).max())


def test_attn_decode_full_shapes_sampled(q3):
    """bs64 at 4097 keys and bs1 at 33280 keys (the batched-decode and long-context shapes)."""
    import torch
    for B, T, rows in [(64, 4097, [0, 17, 63]), (1, 33280, [0])]:
        announce("attn_decode full", B, T)
        Hq, Hkv = 16, 8
        gen = torch.Generator(device="cuda").manual_seed(40 + B)
        K = torch.randn(B, Hkv, T, 128, generator=gen, device="cuda").bfloat16()
        V = torch.randn(B, Hkv, T, 128, generator=gen, device="cuda").bfloat16()
        q = synth.normal((41, B), (B, Hq, 128))
        o = torch.empty(B, Hq * 128, dtype=torch.float32, device="cuda")
        lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
        q3.op_attn_decode(torch.from_numpy(q).cuda(), K, V, lens, o, T)
        torch.cuda.synchronize()
        got = o.cpu().numpy()
        for b in rows:
            Kb = K[b].float().cpu().numpy()
            Vb = V[b].float().cpu().numpy()
            ref = oracle.attend(q[b][:, None, :], Kb, Vb, T - 1)[0]
            assert np.allclose(got[b], ref, rtol=1e-4, atol=2e-5), (B, b, np.abs(got[b] - ref).max())


# ------------------------------------------------------------------ prefill attention (flash, matrix cores)

@pytest.mark.parametrize("M,t0", [(1, 0), (63, 0), (64, 0), (65, 0), (200, 0), (130, 37), (1, 500), (700, 0), (1000, 24),
                                  (4100, 3)])
def test_attn_prefill(q3, M, t0):
    import torch
    announce("attn_prefill", M, t0)
    Hq, Hkv = 16, 8
    t_cap = t0 + M + 5
    q = synth.normal((50, M, t0), (Hq, M, 128))
    K = f32_of_bits(_bf16(synth.normal((51, M, t0), (Hkv, t_cap, 128))))
    V = f32_of_bits(_bf16(synth.normal((52, M, t0), (Hkv, t_cap, 128))))
    o = torch.empty(M, Hq * 128, dtype=torch.float32, device="cuda")
    q3.op_attn_prefill(torch.from_numpy(q).cuda(), torch.from_numpy(K).bfloat16().cuda(),
                       torch.from_numpy(V).bfloat16().cuda(), t0, o)
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    ref = oracle.attend(q, K[:, :t0 + M], V[:, :t0 + M], t0)
    assert np.abs(got - ref).max() <= 1e-4, np.abs(got - ref).max()
    assert rel_l2(got, ref) <= 2e-5, rel_l2(got, ref)
    op = torch.empty(M, 2 * Hq * 128, dtype=torch.bfloat16, device="cuda")
    q3.op_attn_prefill(torch.from_numpy(q).cuda(), torch.from_numpy(K).bfloat16().cuda(),
                       torch.from_numpy(V).bfloat16().cuda(), t0, op, pair=True)
    torch.cuda.synchronize()
    f = got.astype(np.float64)
    assert np.all(np.abs(_pair_value(bf16_bits(op), Hq * 128) - f) <= np.abs(f) * 2.0**-16 + 1e-30)


def test_attn_prefill_long_sampled_rows(q3):
    import torch
    M, t0 = 32767, 0
    announce("attn_prefill long", M)
    Hq, Hkv = 16, 8
    gen = torch.Generator(device="cuda").manual_seed(55)
    q = torch.randn(Hq, M, 128, generator=gen, device="cuda")
    K = torch.randn(Hkv, M, 128, generator=gen, device="cuda").bfloat16()
    V = torch.randn(Hkv, M, 128, generator=gen, device="cuda").bfloat16()
    o = torch.empty(M, Hq * 128, dtype=torch.float32, device="cuda")
    q3.op_attn_prefill(q, K, V, t0, o)
    torch.cuda.synchronize()
    qn, Kn, Vn = q.cpu().numpy(), K.float().cpu().numpy(), V.float().cpu().numpy()
    got = o.cpu().numpy()
    for i in [0, 1, 63, 64, 4095, 20000, M - 1]:
        ref = oracle.attend(qn[:, i:i + 1], Kn[:, :i + 1], Vn[:, :i + 1], i)[0]
        assert np.abs(got[i] - ref).max() <= 1e-4 and rel_l2(got[i], ref) <= 2e-5, i


# ------------------------------------------------------------------ sampler

def _sampler_case(q3, logits, T, p, us):
    import torch
    B, V = logits.shape
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    u = np.asarray(us, np.float32)
    q3.op_sample(torch.from_numpy(logits).cuda(), T, p, torch.from_numpy(u).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    Tf, pf = float(np.float32(T)), float(np.float32(p))
    for b in range(B):
        want = oracle.sample(logits[b], Tf, pf, float(u[b]))
        margin = oracle.sample_margin(logits[b], Tf, pf, float(u[b]))
        if margin > 1e-9:
            assert got[b] == want, (b, got[b], want, margin)


@pytest.mark.parametrize("T,p", [(0.7, 0.9), (1.0, 0.95), (0.0, 0.9), (1.0, 1.0), (0.3, 0.5)])
def test_sampler_matches_oracle(q3, T, p):
    announce("sampler", T, p)
    V, B = 151936, 6
    logits = (synth.normal((60, int(T * 10), int(p * 100)), (B, V)) * 0.64).astype(np.float32)
    us = np.random.default_rng(61).random(B)
    _sampler_case(q3, logits, T, p, us)


def test_sampler_ties_and_degenerate(q3):
    announce("sampler ties")
    V = 8192
    flat = np.zeros((3, V), np.float32)                     # all equal: ordered by id
    _sampler_case(q3, flat, 1.0, 0.5, [0.0, 0.5, 0.999])
    coarse = np.round(synth.normal((62,), (4, V)) * 4) / 4  # many exact ties
    _sampler_case(q3, coarse.astype(np.float32), 0.8, 0.9, [0.1, 0.4, 0.7, 0.95])
    spiky = np.full((2, V), -30.0, np.float32)               # one dominant token
    spiky[:, 1234] = 10.0
    _sampler_case(q3, spiky, 1.0, 0.9, [0.0, 0.9999])
    # full vocabulary: a crossing bucket of 5000 equal logits (more members than the
    # sort holds, so the whole-row refinement runs) and one of a few hundred
    Vf = 151936
    crowd = (synth.normal((63,), (2, Vf)) * 0.5 - 3.0).astype(np.float32)
    crowd[0, 1000:6000] = 1.0
    crowd[1, ::400] = 1.0
    _sampler_case(q3, crowd, 1.0, 0.9, [0.3, 0.8])
