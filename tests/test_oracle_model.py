"""Whole-model pins of the oracle (CPU only).

* library special case: the transformers Qwen3 implementation (float64, CPU,
  eager attention) with the same weights -- pins the composition (block order,
  residuals, QK-norm before RoPE and per head, GQA map, tied head, SwiGLU);
  run with non-unit RMSNorm weights so a dropped or swapped norm weight shows;
* invariants: KV-cached decode equals full recomputation; causal prefix
  invariance; batched independent rows equal single-sequence runs, and the
  batched decode (``forward_batch``, the oracle of the batched workload) equals the
  pinned single-sequence ``forward`` row by row.
"""
import numpy as np
import pytest

import oracle
import synth


def _toy(kv_bf16=False, layers=2, vocab=8192):
    w = synth.workload("toy").with_(n_layers=layers, vocab=vocab)
    cfg = oracle.Config.from_workload(w)
    cfg = oracle.Config(**{**cfg.__dict__, "kv_bf16": kv_bf16})
    return w, cfg


def _random_norm_weights(weights, seed=0):
    rng = np.random.default_rng(seed)
    out = dict(weights)
    for name, a in weights.items():
        if name.endswith("norm.weight"):
            out[name] = (1 + 0.1 * rng.standard_normal(a.shape)).astype(np.float32)
    return out


def _hf_logits(w, weights, ids):
    torch = pytest.importorskip("torch")
    tf = pytest.importorskip("transformers")
    cfg = tf.Qwen3Config(
        vocab_size=w.vocab, hidden_size=w.hidden, intermediate_size=w.ffn,
        num_hidden_layers=w.n_layers, num_attention_heads=w.n_heads,
        num_key_value_heads=w.n_kv_heads, head_dim=w.head_dim, rms_norm_eps=w.rms_eps,
        rope_parameters={"rope_type": "default", "rope_theta": w.rope_theta},
        tie_word_embeddings=True, max_position_embeddings=4096, attention_bias=False,
        attn_implementation="eager")
    model = tf.Qwen3ForCausalLM(cfg).double().eval()
    sd = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in weights.items()}
    missing, unexpected = model.load_state_dict(sd, strict=False)
    assert not unexpected
    assert set(missing) <= {"lm_head.weight"}
    model.tie_weights()
    assert torch.equal(model.lm_head.weight, model.model.embed_tokens.weight)
    with torch.no_grad():
        out = model(input_ids=torch.tensor([list(ids)]), use_cache=False)
    return out.logits[0].numpy()


def test_model_matches_transformers_qwen3():
    w, cfg = _toy(kv_bf16=False)
    weights = _random_norm_weights(synth.make_weights(w), seed=1)
    ids = synth.prompt_tokens(w, 9)
    ref = _hf_logits(w, weights, ids)
    model = oracle.Model(cfg, weights)
    got = model.forward(ids, model.new_cache(16), 0, all_logits=True)
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    assert err <= 2e-4 * scale, (err, scale)
    assert np.array_equal(np.argmax(got, -1), np.argmax(ref, -1))


def test_model_kv_cache_equals_recompute():
    w, cfg = _toy(kv_bf16=False)
    model = oracle.Model(cfg, _random_norm_weights(synth.make_weights(w), seed=2))
    ids = synth.prompt_tokens(w, 12)
    cache = model.new_cache(16)
    model.forward(ids[:5], cache, 0)
    for t in range(5, 12):
        step = model.forward(ids[t:t + 1], cache, t)
        full = model.forward(ids[:t + 1], model.new_cache(16), 0)
        assert np.allclose(step, full, rtol=1e-4, atol=2e-5), t


def test_model_kv_cache_equals_recompute_bf16_cache():
    w, cfg = _toy(kv_bf16=True)
    model = oracle.Model(cfg, synth.make_weights(w))
    ids = synth.prompt_tokens(w, 8)
    cache = model.new_cache(8)
    model.forward(ids[:4], cache, 0)
    for t in range(4, 8):
        step = model.forward(ids[t:t + 1], cache, t)
        full = model.forward(ids[:t + 1], model.new_cache(8), 0)
        # both round K/V to bf16; inputs to the rounding agree to ~1e-6, so
        # rare 1-ulp bf16 flips bound the difference
        assert np.allclose(step, full, rtol=1e-3, atol=2e-3), t
        assert np.linalg.norm(step - full) <= 1e-3 * np.linalg.norm(full)


def test_model_is_causal():
    w, cfg = _toy(kv_bf16=True)
    model = oracle.Model(cfg, synth.make_weights(w))
    ids = synth.prompt_tokens(w, 10)
    a = model.forward(ids, model.new_cache(10), 0, all_logits=True)
    ids2 = ids.copy()
    ids2[6:] = (ids2[6:] + 17) % w.vocab
    b = model.forward(ids2, model.new_cache(10), 0, all_logits=True)
    assert np.allclose(a[:6], b[:6], rtol=1e-5, atol=1e-6)
    assert not np.allclose(a[6:], b[6:], atol=1e-3)


def test_model_batch_rows_are_independent():
    w, cfg = _toy(kv_bf16=True)
    model = oracle.Model(cfg, synth.make_weights(w))
    prompts = [synth.prompt_tokens(w, 3 + b, seq=b) for b in range(3)]
    caches, singles = [], []
    for p in prompts:
        c = model.new_cache(12)
        model.forward(p, c, 0)
        caches.append(c)
        c2 = model.new_cache(12)
        model.forward(p, c2, 0)
        singles.append(c2)
    nxt = np.array([11, 222, 3333])
    pos = np.array([len(p) for p in prompts]) + np.array([0, 100, 7])  # positions need not equal lengths
    batch = model.forward_batch(nxt, caches, pos)
    for b in range(3):
        one = model.forward_batch(nxt[b:b + 1], [singles[b]], pos[b:b + 1])[0]
        assert np.allclose(batch[b], one, rtol=1e-5, atol=1e-5)
    assert all(c.length == len(p) + 1 for c, p in zip(caches, prompts))


def test_embedding_row_and_tied_head():
    # with zero blocks the model is embedding -> final norm -> tied head:
    # logits[t] = rmsnorm(E[id]) . E[t]
    w, cfg = _toy(kv_bf16=False, layers=1, vocab=512)
    weights = synth.make_weights(w)
    model = oracle.Model(oracle.Config(**{**cfg.__dict__, "n_layers": 0}), weights)
    E = weights["model.embed_tokens.weight"].astype(np.float64)
    tok = 77
    got = model.forward([tok], model.new_cache(1), 0)
    h = E[tok] / np.sqrt(np.mean(E[tok] ** 2) + 1e-6)
    assert np.allclose(got, E @ h, rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("kv_bf16", [False, True])
def test_forward_batch_equals_forward_per_sequence(kv_bf16):
    """forward_batch writes its own block loop; pin it to forward() (pinned above against
    the transformers model) on identical caches. Non-unit norm weights (a dropped or
    swapped norm weight shows) and positions unequal to the cache lengths (a position
    taken from the length, or from another row, shows)."""
    w, cfg = _toy(kv_bf16=kv_bf16)
    weights = _random_norm_weights(synth.make_weights(w), seed=5)
    model = oracle.Model(cfg, weights)
    prompts = [synth.prompt_tokens(w, n, seq=b) for b, n in enumerate((4, 7, 2, 5))]
    nxt = np.array([5, 4000, 123, 8191])
    pos = np.array([len(p) for p in prompts]) + np.array([3, 0, 250, 41])
    batch_caches, single_caches = [], []
    for p in prompts:
        for lst in (batch_caches, single_caches):
            c = model.new_cache(16)
            model.forward(p, c, 0)
            lst.append(c)
    got = model.forward_batch(nxt, batch_caches, pos)
    for b in range(len(prompts)):
        want = model.forward([int(nxt[b])], single_caches[b], int(pos[b]))
        rel = np.linalg.norm(got[b] - want) / np.linalg.norm(want)
        # fp32 cache: summation order only (~1e-6); bf16 cache: plus rare 1-ulp rounding flips
        # of K/V entries (one ulp is 2^-6 at magnitudes in [2, 4))
        assert rel <= (1e-5 if not kv_bf16 else 1e-3), (b, rel)
        n = batch_caches[b].length
        for a, c in ((batch_caches[b].K, single_caches[b].K), (batch_caches[b].V, single_caches[b].V)):
            assert np.allclose(a[:, :, :n], c[:, :, :n], rtol=0, atol=2e-5 if not kv_bf16 else 2.0 ** -6)
        assert batch_caches[b].length == single_caches[b].length
    # the same rows with the positions of two rows swapped must differ (positions reach RoPE)
    swapped = pos.copy()
    swapped[[0, 2]] = swapped[[2, 0]]
    caches2 = []
    for p in prompts:
        c = model.new_cache(16)
        model.forward(p, c, 0)
        caches2.append(c)
    other = model.forward_batch(nxt, caches2, swapped)
    assert np.linalg.norm(other[0] - got[0]) > 1e-3 * np.linalg.norm(got[0])
