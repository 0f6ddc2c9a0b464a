"""q3_op_sample_noalloc (sampling with library-owned scratch, no allocation) against
q3_op_sample (the allocating entry point, same kernels): identical tokens, on two
calls in a row where the second is smaller, at temperature 0 and > 0, including a row
whose crossing bucket is too large for the in-memory sort (the refinement passes) and
the largest accepted shape; calls beyond the limits are rejected before any launch."""
import numpy as np
import pytest

from gpu_util import announce

pytestmark = pytest.mark.gpu


def _both(q3, torch, logits, T, p, u):
    B = logits.shape[0]
    a = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    b = torch.full((B,), -2, dtype=torch.int32, device="cuda")
    q3.op_sample(logits, T, p, u, a)
    q3.op_sample_noalloc(logits, T, p, u, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_sample_matches_allocating_entry_point():
    import torch
    from decoder_only_amd import q3
    rng = np.random.default_rng(11)
    # (rows, vocab, temperature, top_p); each call follows the previous one on the same
    # scratch array, the second and fourth with a smaller input than the one before
    cases = [(4, 151936, 0.7, 0.9), (2, 8192, 1.0, 0.95), (4, 262144, 1.0, 0.95), (1, 151936, 0.6, 0.5)]
    for B, V, T, p in cases:
        lg = (rng.standard_normal((B, V)) * 3).astype(np.float32)
        if B >= 2:
            lg[1, :6000] = lg[1].max() - 0.25       # 6000 equal logits near the top: one large bucket
        logits = torch.from_numpy(lg).cuda()
        u = torch.from_numpy(rng.random(B, dtype=np.float32)).cuda()
        for temp in (T, 0.0):
            announce("noalloc sample", B, V, temp, p)
            a, b = _both(q3, torch, logits, temp, p, u)
            assert (a >= 0).all() and (a < V).all(), a
            assert np.array_equal(a, b), (B, V, temp, p, a, b)
            if temp == 0.0:
                assert np.array_equal(a, np.argmax(lg, axis=1)), (a, np.argmax(lg, axis=1))


def test_noalloc_sample_rejects_sizes_beyond_its_scratch():
    import torch
    from decoder_only_amd import q3
    out = torch.empty(5, dtype=torch.int32, device="cuda")
    for B, V in ((5, 1024), (1, 262145)):
        logits = torch.zeros(B, V, dtype=torch.float32, device="cuda")
        with pytest.raises(q3.Q3Error) as e:
            q3.op_sample_noalloc(logits, 0.0, 1.0, None, out[:B])
        assert e.value.code == -2
