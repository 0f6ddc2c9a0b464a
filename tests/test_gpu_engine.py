"""End-to-end teacher-forced parity of the engine against the live oracle (GPU)."""
import numpy as np
import pytest

import synth
from e2e import failures, run_continuous, run_ragged, run_single

pytestmark = pytest.mark.gpu


def _report(stats):
    worst = max(stats, key=lambda s: s.rel)
    print(f"steps={len(stats)} worst rel-L2={worst.rel:.2e} (step {worst.step}) "
          f"max-abs={max(s.max_abs for s in stats):.2e}")


def test_toy_fp32_prefill_and_greedy_decode():
    """Toy workload: 2 layers, fp32 weights and cache, 5-token prompt, 8 greedy steps."""
    w = synth.workload("toy")
    stats = run_single(w, w.prompt_len, w.decode_steps)
    _report(stats)
    assert not failures(stats), failures(stats)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_toy_bf16_matrix_core_prefill(path):
    """bf16 weights and cache, 512-token prompt: rows 0..510 take the matrix-core prefill
    path, the last row and the decode steps the float32 decode path -- one launch per
    operation (path 1) or the persistent decode kernel (path 2)."""
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    stats = run_single(w, 512, 16, decode_path=path)
    _report(stats)
    assert not failures(stats), failures(stats)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_toy_bf16_long_context_decode(path):
    """Decode past one 256-slot attention chunk: the persistent kernel switches to its
    split-K attention with a combine phase."""
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    stats = run_single(w, 250, 20, decode_path=path)
    _report(stats)
    assert not failures(stats), failures(stats)


def test_toy_fp32_rejects_persistent_path():
    from decoder_only_amd import q3
    w = synth.workload("toy").with_(n_layers=1)
    eng = q3.Engine(q3.config(w, 1, 8), synth.make_weights(w))
    with pytest.raises(q3.Q3Error) as e:
        eng.set_decode_path(2)                               # fp32 weights: not supported
    assert e.value.code == -7
    eng.close()


def test_engine_capacity_and_token_errors():
    import torch
    from decoder_only_amd import q3
    w = synth.workload("toy").with_(n_layers=1, vocab=512)
    eng = q3.Engine(q3.config(w, 2, 8), synth.make_weights(w))
    toks = torch.arange(9, dtype=torch.int32, device="cuda")
    with pytest.raises(q3.Q3Error) as e:
        eng.prefill(0, toks)                                 # 9 > max_seq 8
    assert e.value.code == -4
    eng.prefill(0, toks[:8])
    assert eng.seq_len(0) == 8 and eng.seq_len(1) == 0
    with pytest.raises(q3.Q3Error) as e:
        eng.decode_step(toks[:1])                            # slot 0 is full
    assert e.value.code == -4
    eng.reset(0)
    assert eng.seq_len(0) == 0
    bad = torch.tensor([700], dtype=torch.int32, device="cuda")
    eng.prefill(1, bad)
    with pytest.raises(q3.Q3Error) as e:
        eng.sync()
    assert e.value.code == -3
    eng.sync()                                               # the sticky word was cleared
    eng.close()


@pytest.mark.parametrize("path,lens", [
    (2, (5, 17, 100)),            # persistent kernel, every row on the short path
    (3, (5, 40, 300)),            # persistent kernel, split-K attention with one short row
    (3, (1990, 2100)),            # split-K: the shorter row has more chunks (32 of 64 keys) than the longer (17 of 128)
    (1, (5, 40, 300)),            # one launch per operation
    (0, (5, 9, 33, 64, 100, 130, 170, 200, 230, 260, 290, 301)),   # 12 rows: matrix-core batch path
])
def test_toy_bf16_ragged_batch(path, lens):
    """Rows of different cache lengths in one decode step (each row attends its own
    length; the batch paths take the longest row's launch shape)."""
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    stats = run_ragged(w, list(lens), 6, decode_path=path)
    _report(stats)
    assert not failures(stats), failures(stats)[:5]


@pytest.mark.parametrize("path,scale", [(1, 1), (2, 1), (3, 1), (3, 40)])
def test_toy_bf16_continuous_batching(path, scale):
    """Sequences retired and admitted between decode steps, prompts prefilled in two calls
    (the second into a non-empty cache), each slot checked against its own oracle run;
    scale 40: prompts of 80 to 440 tokens on the matrix-core prefill path."""
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    stats = run_continuous(w, 8, decode_path=path, scale=scale)
    _report(stats)
    assert len(stats) == 3 + 1 + 8 * 3
    assert not failures(stats), failures(stats)[:5]


@pytest.mark.parametrize("path", [1, 3])
def test_nonfinite_weight_raises_numeric_error(path):
    """A +inf in one O-projection row makes the residual non-finite: both decode paths
    must report non-finite logits (the persistent kernel carries the O-projection sum as
    fixed-point words, where a non-finite contribution marks the sum as NaN)."""
    import torch
    from decoder_only_amd import q3
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16", n_layers=1)
    ws = dict(synth.make_weights(w))
    name = "model.layers.0.self_attn.o_proj.weight"
    wo = ws[name].copy()
    wo[0, :] = 0x7F80                                        # bf16 +inf
    ws[name] = wo
    eng = q3.Engine(q3.config(w, 1, 16), ws)
    eng.set_decode_path(path)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(q3.Q3Error) as e:
        eng.prefill(0, torch.from_numpy(synth.prompt_tokens(w, 3)).cuda())
        eng.sample(tok, 0.0)
        for _ in range(2):
            eng.decode_step(tok)
            eng.sample(tok, 0.0)
        eng.sync()
    assert e.value.code == -8
    eng.close()


@pytest.mark.parametrize("path", [1, 3])
@pytest.mark.parametrize("name", ["model.layers.0.self_attn.o_proj.weight", "model.layers.0.mlp.down_proj.weight"])
def test_nonfinite_projection_in_decode(path, name):
    """The same through the decode step alone (no prefill, so nothing else can report it
    first): a +inf row in the O projection or in the down projection -- the two sums the
    persistent kernel carries as fixed-point words -- must surface as non-finite logits."""
    import torch
    from decoder_only_amd import q3
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16", n_layers=1)
    ws = dict(synth.make_weights(w))
    wt = ws[name].copy()
    wt[0, :] = 0x7F80                                        # bf16 +inf
    ws[name] = wt
    eng = q3.Engine(q3.config(w, 1, 16), ws)
    eng.set_decode_path(path)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(q3.Q3Error) as e:
        eng.decode_step(tok)
        eng.sample(tok, 0.0)
        eng.sync()
    assert e.value.code == -8
    eng.close()


@pytest.mark.parametrize("path", [0, 3])
def test_toy_bf16_short_prompts_in_causal_chunks(path):
    """Prompts under 16 tokens run through the persistent kernel in causal chunks of up to 4
    rows (row b of a chunk attends the chunk's earlier rows from shared memory and the
    cache), the LM head only in the last chunk. Prompts of 1..15 tokens into an empty
    cache and after earlier tokens (230 + 10 fills the 240-slot short instance exactly;
    231 + 10 goes row by row), each followed by 3 decode steps that read every cache entry
    the chunks wrote; logits against the oracle run of the whole token sequence."""
    import torch
    from decoder_only_amd import q3
    import oracle
    from e2e import compare, failures
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    weights = synth.make_weights(w)
    model = oracle.Model(oracle.Config.from_workload(w), weights)
    eng = q3.Engine(q3.config(w, 1, 260), weights)
    eng.set_decode_path(path)
    logits = torch.empty(1, w.vocab, dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    stats = []
    cases = [(0, n) for n in (1, 2, 3, 4, 5, 8, 9, 15)] + [(7, 6), (3, 13), (230, 10), (231, 10)]
    for t0, n in cases:
        base = synth.prompt_tokens(w, t0, seq=1) if t0 else np.zeros(0, np.int32)
        new = synth.prompt_tokens(w, n, seq=2)
        eng.reset(0)
        if t0:
            eng.prefill(0, torch.from_numpy(base).cuda())
        eng.prefill(0, torch.from_numpy(new).cuda(), logits)
        eng.sample(tok, 0.0)
        cache = model.new_cache(260)
        ref = model.forward(np.concatenate([base, new]), cache, 0)
        for step in range(4):
            eng.sync()
            stats.append(compare(step, 1000 * t0 + n, logits[0].cpu().numpy(), ref))
            if step == 3:
                break
            nxt = int(np.argmax(ref))
            eng.decode_step(torch.tensor([nxt], dtype=torch.int32, device="cuda"), None, logits)
            ref = model.forward([nxt], cache, t0 + n + step)
        assert eng.seq_len(0) == t0 + n + 3
    eng.close()
    _report(stats)
    assert not failures(stats), failures(stats)[:5]
