"""Python binding of the q3 C ABI (include/q3.h, include/q3_ops.h) over ctypes.

Argument marshalling only: every step of the forward pass runs in libq3.so's HIP
kernels. Device buffers are torch tensors on the engine's GPU; work is enqueued on
torch's current stream. The library must have been built in-tree
(``python -m decoder_only_amd.build``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int32, c_int64, c_void_p
from typing import Dict, Mapping, Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq3.so")

F32, BF16, I8, I4 = 0, 1, 2, 3
OP_PAIR = 2     # single operations: bf16 pair rows (n hi parts, then n lo parts)
STATUS = {0: "Q3_OK", -1: "Q3_ERR_ARG", -2: "Q3_ERR_SHAPE", -3: "Q3_ERR_TOKEN",
          -4: "Q3_ERR_CAPACITY", -5: "Q3_ERR_OOM", -6: "Q3_ERR_HIP", -7: "Q3_ERR_STATE",
          -8: "Q3_ERR_NUMERIC"}
EXPORTS = [
    "q3_load", "q3_prefill", "q3_decode_step", "q3_sample", "q3_reset", "q3_kv_import", "q3_kv_export", "q3_kv_fork",
    "q3_seq_len", "q3_kv_free_pages", "q3_sync", "q3_last_error", "q3_free", "q3_profile_begin", "q3_profile_end", "q3_quantize_i8", "q3_quantize_i4",
    "q3_set_decode_path", "q3_profile_trace",
    "q3_op_rmsnorm", "q3_op_gemv", "q3_op_gemm", "q3_op_qk_norm_rope", "q3_op_attn_decode",
    "q3_op_attn_prefill", "q3_op_sample", "q3_op_sample_noalloc",
]
GEMV_STORE, GEMV_RESID, GEMV_SWIGLU = 0, 1, 2
PROF_DECODE_STEP, PROF_GEMV, PROF_LMHEAD, PROF_ATTN_DECODE, PROF_GEMM, PROF_ATTN_PREFILL = range(6)
GEMM_F32, GEMM_RESID_F32, GEMM_SWIGLU_F32, GEMM_BF16, GEMM_SWIGLU_PAIR, GEMM_PARTIAL_F32 = 0, 1, 2, 3, 4, 5


class Q3Error(RuntimeError):
    def __init__(self, code: int, msg: str = ""):
        self.code = code
        super().__init__(f"{STATUS.get(code, code)}: {msg}")


class Q3Config(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("hidden", c_int32), ("n_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32),
                ("vocab", c_int32), ("rms_eps", c_float), ("rope_theta", c_float),
                ("tie_embeddings", c_int32), ("weight_dtype", c_int32), ("kv_dtype", c_int32),
                ("max_batch", c_int32), ("max_seq", c_int32), ("kv_pages", c_int32)]


class Q3Tensor(ctypes.Structure):
    _fields_ = [("name", c_char_p), ("data", c_void_p), ("dtype", c_int32), ("numel", c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libq3.so once. torch is imported first so that the library binds to the
    HIP runtime torch already loaded (one runtime per process)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m decoder_only_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, f32 = c_void_p, c_int32, c_float
    sig = {
        "q3_load": ([POINTER(Q3Config), POINTER(Q3Tensor), i32, vp, POINTER(vp)], i32),
        "q3_prefill": ([vp, i32, vp, i32, vp], i32),
        "q3_decode_step": ([vp, vp, vp, i32, vp], i32),
        "q3_sample": ([vp, vp, i32, f32, f32, vp, vp], i32),
        "q3_reset": ([vp, i32], i32),
        "q3_kv_import": ([vp, i32, i32, vp, vp, i32], i32),
        "q3_kv_export": ([vp, i32, i32, vp, vp, i32], i32),
        "q3_kv_fork": ([vp, i32, i32, i32], i32),
        "q3_seq_len": ([vp, i32], i32),
        "q3_kv_free_pages": ([vp], i32),
        "q3_quantize_i8": ([vp, i32, c_int64, c_int64, vp, vp], i32),
        "q3_quantize_i4": ([vp, i32, c_int64, c_int64, vp, vp], i32),
        "q3_sync": ([vp], i32),
        "q3_last_error": ([vp], c_char_p),
        "q3_free": ([vp], None),
        "q3_profile_begin": ([vp, i32], i32),
        "q3_set_decode_path": ([vp, i32], i32),
        "q3_profile_trace": ([vp, vp, i32], i32),
        "q3_profile_end": ([vp, POINTER(ctypes.c_double), POINTER(c_int64), POINTER(ctypes.c_double),
                            POINTER(ctypes.c_double)], i32),
        "q3_op_rmsnorm": ([vp, vp, vp, i32, i32, i32, f32, vp], i32),
        "q3_op_gemv": ([vp, i32, vp, vp, i32, i32, i32, i32, vp], i32),
        "q3_op_gemm": ([vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp], i32),
        "q3_op_qk_norm_rope": ([vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp, vp, i32, i32, vp], i32),
        "q3_op_attn_decode": ([vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, vp, vp], i32),
        "q3_op_attn_prefill": ([vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp], i32),
        "q3_op_sample": ([vp, i32, i32, f32, f32, vp, vp, vp], i32),
        "q3_op_sample_noalloc": ([vp, i32, i32, f32, f32, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, dtype=None) -> Optional[int]:
    """Device pointer of a contiguous torch CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous tensor on the GPU")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"expected dtype {dtype}, got {t.dtype}")
    return t.data_ptr()


def _check(code: int, what: str = "", eng=None) -> None:
    if code != 0:
        msg = what
        if eng is not None:
            msg += ": " + load_library().q3_last_error(eng).decode()
        raise Q3Error(code, msg)


def config(w, max_batch: int, max_seq: int, int8: bool = False, kv_pages: int = 0, int4: bool = False) -> Q3Config:
    """q3_config of a model description with the synth.Workload fields; int8 / int4:
    weight-only int8 / int4 (the engine quantises the given weights at load); kv_pages:
    KV-cache pool size in pages of 256 slots (0: enough for every sequence slot to reach
    max_seq)."""
    if int8 and int4:
        raise ValueError("int8 and int4 exclude each other")
    return Q3Config(n_layers=w.n_layers, hidden=w.hidden, n_heads=w.n_heads,
                    n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn, vocab=w.vocab,
                    rms_eps=w.rms_eps, rope_theta=w.rope_theta, tie_embeddings=1,
                    weight_dtype=I8 if int8 else I4 if int4 else (BF16 if w.weight_dtype == "bf16" else F32),
                    kv_dtype=BF16 if w.kv_dtype == "bf16" else F32,
                    max_batch=max_batch, max_seq=max_seq, kv_pages=kv_pages)


class Engine:
    """One q3 engine (weights, KV cache, workspaces) on the current GPU."""

    def __init__(self, cfg: Q3Config, weights: Mapping[str, np.ndarray], stream: Optional[int] = None):
        L = load_library()
        arrs = []
        tens = (Q3Tensor * len(weights))()
        for i, (name, a) in enumerate(weights.items()):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                dt = BF16
            elif a.dtype == np.float32:
                dt = F32
            else:
                raise TypeError(f"{name}: weights must be float32 or bf16 bits (uint16)")
            arrs.append(a)
            tens[i] = Q3Tensor(name.encode(), a.ctypes.data, dt, a.size)
        self._cfg = cfg
        self._stream = _stream() if stream is None else stream
        h = c_void_p()
        rc = L.q3_load(byref(cfg), tens, len(weights), self._stream, byref(h))
        _check(rc, "q3_load")
        self._h = h
        self.vocab = cfg.vocab

    @property
    def handle(self):
        return self._h

    def close(self) -> None:
        if getattr(self, "_h", None):
            load_library().q3_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, seq: int, tokens, logits=None) -> None:
        import torch
        _check(load_library().q3_prefill(self._h, seq, _ptr(tokens, torch.int32), tokens.numel(),
                                         _ptr(logits, torch.float32)), "q3_prefill", self._h)

    def decode_step(self, tokens, positions=None, logits=None) -> None:
        import torch
        _check(load_library().q3_decode_step(self._h, _ptr(tokens, torch.int32),
                                             _ptr(positions, torch.int32), tokens.numel(),
                                             _ptr(logits, torch.float32)), "q3_decode_step", self._h)

    def sample(self, out, temperature: float, top_p: float = 1.0, uniforms=None, logits=None) -> None:
        import torch
        _check(load_library().q3_sample(self._h, _ptr(logits, torch.float32), out.numel(),
                                        float(temperature), float(top_p),
                                        _ptr(uniforms, torch.float32), _ptr(out, torch.int32)),
               "q3_sample", self._h)

    def reset(self, seq: int) -> None:
        _check(load_library().q3_reset(self._h, seq), "q3_reset", self._h)

    def kv_import(self, seq: int, layer: int, k, v, length: int) -> None:
        """k, v: numpy arrays (host) or torch tensors (device), [n_kv_heads, length, head_dim]."""
        def p(x):
            if isinstance(x, np.ndarray):
                return np.ascontiguousarray(x).ctypes.data
            return _ptr(x)
        kk = np.ascontiguousarray(k) if isinstance(k, np.ndarray) else k
        vv = np.ascontiguousarray(v) if isinstance(v, np.ndarray) else v
        _check(load_library().q3_kv_import(self._h, seq, layer, p(kk), p(vv), length), "q3_kv_import", self._h)

    def kv_fork(self, src: int, dst: int, length: int) -> None:
        """Slot dst becomes a copy of the first `length` cached tokens of slot src."""
        _check(load_library().q3_kv_fork(self._h, src, dst, length), "q3_kv_fork", self._h)

    def kv_export(self, seq: int, layer: int, length: int):
        """Slots 0 .. length-1 of one (sequence, layer) of the cache as two host arrays
        [n_kv_heads, length, head_dim] (uint16 bf16 bit patterns, or float32)."""
        c = self._cfg
        dt = np.uint16 if c.kv_dtype == BF16 else np.float32
        k = np.empty((c.n_kv_heads, length, c.head_dim), dtype=dt)
        v = np.empty_like(k)
        _check(load_library().q3_kv_export(self._h, seq, layer, k.ctypes.data, v.ctypes.data, length),
               "q3_kv_export", self._h)
        return k, v

    def seq_len(self, seq: int) -> int:
        return load_library().q3_seq_len(self._h, seq)

    def kv_free_pages(self) -> int:
        """Pages of 256 token slots in the KV-cache pool that no sequence holds."""
        return load_library().q3_kv_free_pages(self._h)

    def sync(self) -> None:
        _check(load_library().q3_sync(self._h), "q3_sync", self._h)

    def set_decode_path(self, path: int) -> None:
        """0 auto, 1 one launch per operation, 2 always the persistent decode kernel,
        3 auto with the persistent kernel dispatched as an ordinary launch."""
        _check(load_library().q3_set_decode_path(self._h, path), "q3_set_decode_path", self._h)

    def profile_trace(self, buf=None) -> None:
        """Record phase timestamps of the persistent decode kernel into buf (device int64
        [2, n]); None turns it off."""
        n = 0 if buf is None else buf.shape[1]
        _check(load_library().q3_profile_trace(self._h, _ptr(buf), n), "q3_profile_trace", self._h)

    def profile_begin(self, kind: int) -> None:
        _check(load_library().q3_profile_begin(self._h, kind), "q3_profile_begin", self._h)

    def profile_end(self) -> dict:
        ms, n = ctypes.c_double(), c_int64()
        by, fl = ctypes.c_double(), ctypes.c_double()
        _check(load_library().q3_profile_end(self._h, byref(ms), byref(n), byref(by), byref(fl)),
               "q3_profile_end", self._h)
        return {"ms": ms.value, "launches": n.value, "bytes": by.value, "flops": fl.value}


# ------------------------------------------------------------------------- op level

def op_rmsnorm(x, w, out, eps: float, pair: bool = False) -> None:
    """out: float32 or bf16 [rows, d], or (pair) bf16 [rows, 2d]."""
    import torch
    dt = OP_PAIR if pair else (BF16 if out.dtype == torch.bfloat16 else F32)
    rows, d = x.shape
    _check(load_library().q3_op_rmsnorm(_ptr(x, torch.float32), _ptr(w, torch.float32), _ptr(out), dt,
                                        rows, d, eps, _stream()), "q3_op_rmsnorm")


def op_gemv(W, x, y, epilogue: int = GEMV_STORE) -> None:
    import torch
    dt = BF16 if W.dtype == torch.bfloat16 else F32
    N, K = W.shape
    _check(load_library().q3_op_gemv(_ptr(W), dt, _ptr(x, torch.float32), _ptr(y, torch.float32), N, K,
                                     x.shape[0], epilogue, _stream()), "q3_op_gemv")


def op_gemm(A, W, C, epilogue: int = GEMM_F32, a_pair: bool = False, splits: int = 1, colscale=None) -> None:
    """A: bf16 or float32 [M, K], or (a_pair) bf16 pair rows [M, 2K]; W: bf16 [N, K];
    colscale: optional float32 [N] column scales."""
    import torch
    M, K = A.shape
    N = W.shape[0]
    if a_pair:
        K //= 2
    adt = OP_PAIR if a_pair else (F32 if A.dtype == torch.float32 else BF16)
    cs = _ptr(colscale, torch.float32) if colscale is not None else None
    _check(load_library().q3_op_gemm(_ptr(A, (torch.bfloat16, torch.float32)), adt, _ptr(W, torch.bfloat16),
                                     _ptr(C), M, N, K, epilogue, splits, cs, _stream()), "q3_op_gemm")


def op_qk_norm_rope(qkv, q_norm, k_norm, positions, slots, n_heads, n_kv_heads, eps, theta,
                    q_out, k_cache, v_cache) -> None:
    import torch
    dt = BF16 if k_cache.dtype == torch.bfloat16 else F32
    B = qkv.shape[0]
    _check(load_library().q3_op_qk_norm_rope(
        _ptr(qkv, torch.float32), _ptr(q_norm, torch.float32), _ptr(k_norm, torch.float32),
        _ptr(positions, torch.int32), _ptr(slots, torch.int32), B, n_heads, n_kv_heads, eps, theta,
        _ptr(q_out, torch.float32), _ptr(k_cache), _ptr(v_cache), dt, k_cache.shape[2], _stream()),
        "q3_op_qk_norm_rope")


def op_attn_decode(q, k_cache, v_cache, lens, o, max_len: int) -> None:
    import torch
    dt = BF16 if k_cache.dtype == torch.bfloat16 else F32
    B, Hkv, t_cap, _ = k_cache.shape
    _check(load_library().q3_op_attn_decode(_ptr(q, torch.float32), _ptr(k_cache), _ptr(v_cache), dt, t_cap,
                                            _ptr(lens, torch.int32), B, q.shape[1], Hkv, max_len,
                                            _ptr(o, torch.float32), _stream()), "q3_op_attn_decode")


def op_attn_prefill(q, k_cache, v_cache, t0: int, o, pair: bool = False) -> None:
    """o: float32 [M, Hq*128], or (pair) bf16 pair rows [M, 2*Hq*128]."""
    import torch
    Hq, M, _ = q.shape
    Hkv, t_cap, _ = k_cache.shape
    _check(load_library().q3_op_attn_prefill(_ptr(q, torch.float32), _ptr(k_cache, torch.bfloat16),
                                             _ptr(v_cache, torch.bfloat16), t_cap, M, t0, Hq, Hkv,
                                             _ptr(o, torch.bfloat16 if pair else torch.float32),
                                             OP_PAIR if pair else F32, _stream()), "q3_op_attn_prefill")


def op_sample(logits, temperature: float, top_p: float, uniforms, out) -> None:
    import torch
    B, V = logits.shape
    _check(load_library().q3_op_sample(_ptr(logits, torch.float32), B, V, float(temperature), float(top_p),
                                       _ptr(uniforms, torch.float32), _ptr(out, torch.int32), _stream()),
           "q3_op_sample")


def op_sample_noalloc(logits, temperature: float, top_p: float, uniforms, out) -> None:
    """q3_op_sample without allocation (library-owned scratch; at most 4 rows of 262144)."""
    import torch
    B, V = logits.shape
    _check(load_library().q3_op_sample_noalloc(_ptr(logits, torch.float32), B, V, float(temperature),
                                               float(top_p), _ptr(uniforms, torch.float32),
                                               _ptr(out, torch.int32), _stream()), "q3_op_sample_noalloc")
