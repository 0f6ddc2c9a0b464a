"""Prefix reuse (q3_kv_fork): a prompt prefix shared by several sequences is prefilled
once, handed to other sequence slots (their page tables point at its cache pages; the
page holding the prefix's last tokens is copied by the first sequence that appends into
it), and each continues with its own suffix (a chunked prefill into the non-empty cache:
row i of the suffix sees slots j <= t0 + i), then all of them decode together. Every
sequence must match the oracle run of its whole prompt from scratch (logits within
max-abs 2e-2 and relative L2 1e-3, same greedy token), and a sequence whose prefix was
recomputed instead of forked must give bit-identical logits to its forked twin (pages and
copies are exact and the cache depends on nothing after the prefix, Step 5)."""
import numpy as np
import pytest

import oracle
import synth
from e2e import compare, failures
from gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", [0, 1])
def test_prefix_fork_then_own_suffixes(path):
    import torch
    from decoder_only_amd import q3
    w = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")
    weights = synth.make_weights(w)
    model = oracle.Model(oracle.Config.from_workload(w), weights)
    P = 300                                         # prefix: the matrix-core prefill path
    prefix = synth.prompt_tokens(w, P)
    suffixes = [synth.prompt_tokens(w, n, seq=10 + s) for s, n in enumerate((7, 1, 40, 200))]
    S = len(suffixes)
    announce("prefix fork", P, [len(x) for x in suffixes], "path", path)
    eng = q3.Engine(q3.config(w, S + 1, 600), weights)
    eng.set_decode_path(path)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    eng.prefill(0, dev(prefix))
    for s in range(1, S):
        eng.kv_fork(0, s, P)
        assert eng.seq_len(s) == P
    eng.prefill(S, dev(prefix))                     # the same prefix recomputed, no fork
    logits = torch.empty(S + 1, w.vocab, dtype=torch.float32, device="cuda")
    for s in range(S):
        eng.prefill(s, dev(suffixes[s]), logits[s])
    eng.prefill(S, dev(suffixes[1]), logits[S])
    with pytest.raises(q3.Q3Error):
        eng.kv_fork(1, 1, 10)                       # source and destination must differ
    with pytest.raises(q3.Q3Error):
        eng.kv_fork(1, 2, P + 2)                    # beyond the source's length (P + 1)
    eng.sync()
    got = logits.cpu().numpy()
    assert np.array_equal(got[1], got[S]), "forked prefix differs from the recomputed one"

    caches, refs = [], []
    for s in range(S):
        c = model.new_cache(600)
        refs.append(model.forward(np.concatenate([prefix, suffixes[s]]), c, 0))
        caches.append(c)
    stats = [compare(0, s, got[s], refs[s]) for s in range(S)]
    toks = np.array([int(np.argmax(r)) for r in refs], dtype=np.int32)
    out = torch.empty(S, dtype=torch.int32, device="cuda")
    for t in range(1, 7):                           # the four sequences decode together
        eng.decode_step(dev(toks), None, logits[:S])
        eng.sample(out, 0.0)
        eng.sync()
        got = logits[:S].cpu().numpy()
        for s in range(S):
            ref = model.forward([int(toks[s])], caches[s], P + len(suffixes[s]) + t - 1)
            stats.append(compare(t, s, got[s], ref))
            toks[s] = int(np.argmax(ref))
    eng.close()
    worst = max(stats, key=lambda x: x.rel)
    print(f"{len(stats)} rows; worst rel-L2 {worst.rel:.2e} (step {worst.step}, seq {worst.row})")
    assert not failures(stats), failures(stats)[:5]
