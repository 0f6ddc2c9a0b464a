"""Paged KV cache: pages of 256 token slots (every layer and kv head) drawn from one pool
shared by all sequence slots, and a page table per sequence. Step 5 of "Inside an LLM"
defines a sequence's cache as its keys and values in slot order; where those slots sit in
memory is not part of the method, so:

* scrambled pages: after a reset the pool hands pages out in another order, so a
  sequence's table is not monotonic; every row still meets the oracle bar, and its logits
  are bit-identical to an engine whose pages are in order (same launches);
* continuous batching with a pool smaller than max_batch * max_seq: a sequence retires
  (q3_reset) and a new prompt takes its slot between decode steps of the others; running
  out of pages is Q3_ERR_CAPACITY and changes nothing; every row meets the oracle bar;
* fork: shared pages are not copied; the first append into a shared page copies it
  (free-page count), and the forked rows match the oracle and each other bit for bit;
* import / export through the pages is an exact round trip, and importing a shorter cache
  returns the pages beyond it.
Bar per row and step: logits max-abs 2e-2, relative L2 1e-3, identical argmax."""
import numpy as np
import pytest

import oracle
import synth
from e2e import compare, failures
from gpu_util import announce

pytestmark = pytest.mark.gpu

W = synth.workload("toy").with_(weight_dtype="bf16", kv_dtype="bf16")


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class _Ref:
    """One sequence of the oracle, fed the same tokens as an engine slot."""

    def __init__(self, model, prompt, cap):
        self.cache = model.new_cache(cap)
        self.model = model
        self.logits = model.forward(prompt, self.cache, 0)
        self.pos = len(prompt)

    def next_token(self):
        return int(np.argmax(self.logits))

    def step(self, tok):
        self.logits = self.model.forward([tok], self.cache, self.pos)
        self.pos += 1


def _decode(eng, refs, rows, logits, stats, step):
    """One decode step of slots 0 .. rows-1 with each oracle row's argmax token."""
    toks = np.array([r.next_token() for r in refs[:rows]], dtype=np.int32)
    eng.decode_step(_dev(toks), None, logits[:rows])
    for b in range(rows):
        refs[b].step(int(toks[b]))
    eng.sync()
    got = logits[:rows].cpu().numpy()
    for b in range(rows):
        stats.append(compare(step, b, got[b], refs[b].logits))
    return got


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", [0, 1])
def test_scrambled_pages_match_ordered_pages(path):
    """Path 0: the persistent kernel (split-K instance past 240 slots); 1: one launch per
    operation. Sequence 0's pages come out 2, 1, 0 and then 5 (it crosses slot 768)."""
    import torch
    from decoder_only_amd import q3
    weights = synth.make_weights(W)
    model = oracle.Model(oracle.Config.from_workload(W), weights)
    first = synth.prompt_tokens(W, 600, seq=1)
    prompts = [synth.prompt_tokens(W, 700, seq=2), synth.prompt_tokens(W, 300, seq=3)]
    announce("paging scrambled", path)
    steps = 71
    eng = q3.Engine(q3.config(W, 2, 1024), weights)
    eng.set_decode_path(path)
    logits = torch.empty(2, W.vocab, dtype=torch.float32, device="cuda")
    eng.prefill(0, _dev(first))                      # pages 0, 1, 2
    eng.prefill(1, _dev(prompts[1]), logits[1])      # pages 3, 4
    eng.reset(0)
    assert eng.kv_free_pages() == 8 - 2
    eng.prefill(0, _dev(prompts[0]), logits[0])      # pages 2, 1, 0
    eng.sync()
    refs = [_Ref(model, p, 1024) for p in prompts]
    seen = [logits.cpu().numpy()]
    stats = [compare(0, b, seen[0][b], refs[b].logits) for b in range(2)]
    fed = []
    for t in range(1, steps + 1):
        fed.append(np.array([r.next_token() for r in refs], dtype=np.int32))
        seen.append(_decode(eng, refs, 2, logits, stats, t))
    assert eng.kv_free_pages() == 8 - 6
    eng.close()
    assert not failures(stats), failures(stats)[:5]

    eng = q3.Engine(q3.config(W, 2, 1024), weights)  # the same launches, pages in order
    eng.set_decode_path(path)
    eng.prefill(1, _dev(prompts[1]), logits[1])
    eng.prefill(0, _dev(prompts[0]), logits[0])
    eng.sync()
    assert np.array_equal(logits.cpu().numpy(), seen[0])
    for t in range(1, steps + 1):
        eng.decode_step(_dev(fed[t - 1]), None, logits)
        eng.sync()
        assert np.array_equal(logits.cpu().numpy(), seen[t]), f"step {t}"
    eng.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", [0, 1])
def test_continuous_batching_in_a_small_pool(path):
    """Three slots, a pool of 5 pages (max_seq 1024 would need 12): slot 2 runs out of pages
    at slot 256, slot 0 retires, a new prompt takes slot 0, decoding goes on."""
    import torch
    from decoder_only_amd import q3
    weights = synth.make_weights(W)
    model = oracle.Model(oracle.Config.from_workload(W), weights)
    prompts = [synth.prompt_tokens(W, n, seq=20 + i) for i, n in enumerate((300, 254, 250))]
    announce("paging continuous batching", path)
    eng = q3.Engine(q3.config(W, 3, 1024, kv_pages=5), weights)
    eng.set_decode_path(path)
    logits = torch.empty(3, W.vocab, dtype=torch.float32, device="cuda")
    for b, p in enumerate(prompts):
        eng.prefill(b, _dev(p), logits[b])
    assert eng.kv_free_pages() == 1
    eng.sync()
    refs = [_Ref(model, p, 1024) for p in prompts]
    got = logits.cpu().numpy()
    stats = [compare(0, b, got[b], refs[b].logits) for b in range(3)]
    for t in range(1, 7):         # slot 1 takes the last page at slot 256 (step 3)
        _decode(eng, refs, 3, logits, stats, t)
    assert eng.kv_free_pages() == 0
    lens = [eng.seq_len(b) for b in range(3)]
    assert lens == [306, 260, 256]
    toks = _dev(np.array([r.next_token() for r in refs], dtype=np.int32))
    with pytest.raises(q3.Q3Error) as e:
        eng.decode_step(toks, None, logits)   # slot 2 would need a page at slot 256
    assert e.value.code == -4
    assert [eng.seq_len(b) for b in range(3)] == lens and eng.kv_free_pages() == 0
    with pytest.raises(q3.Q3Error) as e:
        eng.prefill(0, _dev(synth.prompt_tokens(W, 300, seq=30)))   # slots 306 .. 605 need a third page
    assert e.value.code == -4 and eng.seq_len(0) == 306
    eng.reset(0)                  # slot 0 retires: its two pages go back
    assert eng.kv_free_pages() == 2
    new = synth.prompt_tokens(W, 40, seq=31)
    eng.prefill(0, _dev(new), logits[0])
    eng.sync()
    refs[0] = _Ref(model, new, 1024)
    stats.append(compare(7, 0, logits[0].cpu().numpy(), refs[0].logits))
    for t in range(7, 12):
        _decode(eng, refs, 3, logits, stats, t)
    assert eng.kv_free_pages() == 0
    eng.close()
    worst = max(stats, key=lambda x: x.rel)
    print(f"{len(stats)} rows; worst rel-L2 {worst.rel:.2e}")
    assert not failures(stats), failures(stats)[:5]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", [0, 1])
def test_fork_shares_pages_and_copies_on_write(path):
    import torch
    from decoder_only_amd import q3
    weights = synth.make_weights(W)
    model = oracle.Model(oracle.Config.from_workload(W), weights)
    prompt = synth.prompt_tokens(W, 600, seq=40)
    announce("paging fork", path)
    eng = q3.Engine(q3.config(W, 3, 1024), weights)
    eng.set_decode_path(path)
    eng.prefill(0, _dev(prompt))
    assert eng.kv_free_pages() == 12 - 3
    eng.kv_fork(0, 1, 600)
    eng.kv_fork(0, 2, 300)
    assert eng.kv_free_pages() == 12 - 3          # nothing copied
    refs = []
    for n in (600, 600, 300):
        refs.append(_Ref(model, prompt[:n], 1024))
    # step 1: every row appends to a shared page; slot 0 copies page 2 (held by 0 and 1),
    # slot 2 copies page 1 (held by all three); slot 1 then holds page 2 alone
    logits = torch.empty(3, W.vocab, dtype=torch.float32, device="cuda")
    stats = []
    got = _decode(eng, refs, 3, logits, stats, 1)
    assert eng.kv_free_pages() == 12 - 5
    assert np.array_equal(got[0], got[1])          # same cache, token and position
    eng.reset(1)                                   # page 2 (slot 1's alone) goes back
    assert eng.kv_free_pages() == 12 - 4
    refs[1] = _Ref(model, synth.prompt_tokens(W, 20, seq=41), 1024)
    eng.prefill(1, _dev(synth.prompt_tokens(W, 20, seq=41)))
    for t in range(2, 6):
        _decode(eng, refs, 3, logits, stats, t)
    eng.close()
    assert not failures(stats), failures(stats)[:5]


def test_import_export_round_trip_through_pages():
    import torch
    from decoder_only_amd import q3
    w = W.with_(n_layers=2, vocab=512)
    weights = synth.make_weights(w)
    announce("paging import/export")
    eng = q3.Engine(q3.config(w, 2, 1024), weights)
    eng.prefill(0, _dev(synth.prompt_tokens(w, 300, seq=50)))   # slot 0 holds pages 0, 1
    gen = torch.Generator(device="cuda").manual_seed(5)
    kv = torch.randn(2, 2, w.n_kv_heads, 700, w.head_dim, generator=gen, device="cuda").bfloat16()
    for layer in range(2):
        eng.kv_import(1, layer, kv[layer, 0].contiguous(), kv[layer, 1].contiguous(), 700)
    assert eng.kv_free_pages() == 8 - 5 and eng.seq_len(1) == 700
    L = q3.load_library()
    for layer in range(2):
        k = torch.empty(w.n_kv_heads, 700, w.head_dim, dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        assert L.q3_kv_export(eng._h, 1, layer, k.data_ptr(), v.data_ptr(), 700) == 0   # device buffers
        assert torch.equal(k, kv[layer, 0]) and torch.equal(v, kv[layer, 1])
        kh, vh = eng.kv_export(1, layer, 123)                                        # host, a prefix
        assert np.array_equal(kh, kv[layer, 0, :, :123].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        assert np.array_equal(vh, kv[layer, 1, :, :123].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    for layer in range(2):         # a shorter cache: the pages beyond it go back
        eng.kv_import(1, layer, kv[layer, 0, :, :100].contiguous(), kv[layer, 1, :, :100].contiguous(), 100)
    assert eng.kv_free_pages() == 8 - 3 and eng.seq_len(1) == 100
    kh, vh = eng.kv_export(1, 1, 100)
    assert np.array_equal(kh, kv[1, 0, :, :100].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(vh, kv[1, 1, :, :100].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    with pytest.raises(q3.Q3Error) as e:
        eng.kv_export(1, 0, 101)
    assert e.value.code == -1
    eng.close()
