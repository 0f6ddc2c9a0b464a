"""Helpers shared by the GPU tests (test infrastructure)."""
import sys

import numpy as np


def announce(*parts) -> None:
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    print("[gpu case]", *parts, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype) if t.dtype.itemsize == dtype.itemsize and t.dtype != dtype and a.dtype == np.uint16 else t.to(dtype)
    return t.cuda()


def bf16_dev(bits: np.ndarray):
    """Device bf16 tensor from uint16 bit patterns."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32_of_bits(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
