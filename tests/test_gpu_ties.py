"""Greedy ties on the GPU: among equal maximal logits the lowest token id wins (Step 8's
argmax; reading: the lowest id among equal maxima).

Random logits never tie, so the ties are built: with the tied LM head, logit v is the
dot product of the final hidden row with embedding row v, so copying the embedding row
of the step's argmax a onto a lower id b (one not fed as an input token) gives the two
ids bit-identical logits -- both the maximum -- and the greedy token must be b. Every
decode path is run: the persistent kernel (cooperative and ordinary launch; its argmax
is packed per workgroup and reduced by its tail kernel), one launch per operation (the
LM-head GEMV's fused argmax), and the batch path of more than 8 rows (LM head on the
matrix cores, then a per-row argmax kernel). The sampler entry points are also given
explicitly tied logits at temperature 0.
"""
import numpy as np
import pytest

import synth
from gpu_util import announce

pytestmark = pytest.mark.gpu


def _toy():
    return synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")


def _with_copied_row(weights, src: int, dst: int):
    ws = dict(weights)
    E = ws["model.embed_tokens.weight"].copy()
    E[dst] = E[src]
    ws["model.embed_tokens.weight"] = E
    return ws


def _lower_unused(a: int, used) -> int:
    for b in range(a - 1, -1, -1):
        if b not in used:
            return b
    raise AssertionError("no free lower id")


def _prefill_greedy(w, weights, prompt, path):
    """Prefill `prompt` into slot 0 and draw the greedy token twice: fused into the decode
    launch (no logits given) and from the returned logits (explicit logits)."""
    import torch
    from decoder_only_amd import q3
    eng = q3.Engine(q3.config(w, 1, 16), weights)
    eng.set_decode_path(path)
    logits = torch.empty(1, w.vocab, dtype=torch.float32, device="cuda")
    fused = torch.empty(1, dtype=torch.int32, device="cuda")
    explicit = torch.empty(1, dtype=torch.int32, device="cuda")
    eng.prefill(0, torch.from_numpy(prompt).cuda(), logits)
    eng.sample(fused, 0.0)
    eng.sample(explicit, 0.0, logits=logits)
    eng.sync()
    out = logits[0].cpu().numpy(), int(fused.item()), int(explicit.item())
    eng.close()
    return out


@pytest.mark.parametrize("path", [0, 1, 2, 3])
def test_greedy_tie_lowest_id_single_row(path):
    w = _toy()
    weights = synth.make_weights(w)
    prompt = synth.prompt_tokens(w, 5)
    announce("greedy tie", "path", path)
    lg, _, _ = _prefill_greedy(w, weights, prompt, path)
    a = int(np.argmax(lg))
    b = _lower_unused(a, set(prompt.tolist()))
    lg2, fused, explicit = _prefill_greedy(w, _with_copied_row(weights, a, b), prompt, path)
    # the two rows give bit-identical logits, and they are the maximum
    assert lg2[a] == lg2[b] == lg2.max(), (lg2[a], lg2[b], lg2.max())
    assert fused == b and explicit == b, (fused, explicit, a, b)


def test_greedy_tie_lowest_id_matrix_core_batch():
    """9 rows (more than the GEMV path takes): every row decodes the same token after the
    same prompt, so all rows tie at the same pair of ids."""
    import torch
    from decoder_only_amd import q3
    w = _toy()
    B = 9
    weights = synth.make_weights(w)
    prompt = synth.prompt_tokens(w, 5)
    nxt = int(prompt[0])

    def run(ws):
        eng = q3.Engine(q3.config(w, B, 16), ws)
        p = torch.from_numpy(prompt).cuda()
        for s in range(B):
            eng.prefill(s, p)
        logits = torch.empty(B, w.vocab, dtype=torch.float32, device="cuda")
        toks = torch.full((B,), nxt, dtype=torch.int32, device="cuda")
        eng.decode_step(toks, None, logits)
        out = torch.empty(B, dtype=torch.int32, device="cuda")
        eng.sample(out, 0.0)
        eng.sync()
        r = logits.cpu().numpy(), out.cpu().numpy()
        eng.close()
        return r

    announce("greedy tie", "matrix-core batch", B)
    lg, _ = run(weights)
    a = int(np.argmax(lg[0]))
    b = _lower_unused(a, set(prompt.tolist()) | {nxt})
    lg2, toks = run(_with_copied_row(weights, a, b))
    for r in range(B):
        assert lg2[r, a] == lg2[r, b] == lg2[r].max(), (r, lg2[r, a], lg2[r, b], lg2[r].max())
    assert (toks == b).all(), (toks, a, b)


def test_sampler_temperature_zero_ties():
    """Explicit ties at temperature 0 (any top_p): the lowest tied id, including ties that
    span the first and the last id and ties of three."""
    import torch
    from decoder_only_amd import q3
    V = 151936
    ties = [(9, 4, 4000), (0, V - 1), (V - 1, V - 2), (77777, 77778, 5)]
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((len(ties), V)).astype(np.float32)
    for r, ids in enumerate(ties):
        lg[r, list(ids)] = lg[r].max() + np.float32(0.5)
    want = np.array([min(t) for t in ties], dtype=np.int32)
    announce("sampler ties", len(ties))
    d = torch.from_numpy(lg).cuda()
    out = torch.empty(len(ties), dtype=torch.int32, device="cuda")
    for top_p in (1.0, 0.5):
        q3.op_sample(d, 0.0, top_p, None, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), (top_p, out.cpu().numpy(), want)
    # the engine's entry point on the same logits
    w = _toy().with_(vocab=V, n_layers=1)
    eng = q3.Engine(q3.config(w, len(ties), 4), synth.make_weights(w))
    out2 = torch.empty(len(ties), dtype=torch.int32, device="cuda")
    eng.sample(out2, 0.0, logits=d)
    eng.sync()
    eng.close()
    assert np.array_equal(out2.cpu().numpy(), want), (out2.cpu().numpy(), want)
