"""Teacher-forced end-to-end comparison of the engine with the oracle (test infrastructure).

The oracle's own token is fed to both sides at every step, so a single near-tie in
the argmax cannot make the two runs diverge. Per step and row the comparison reports
max-abs and relative-L2 logit error, whether the greedy pick agrees (the oracle's argmax,
or a token whose oracle logit is within near_tie() of it: logits fixed only to a
tolerance cannot order two tokens closer than that), and the oracle's top-2 logit gap.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

import oracle
import synth
from gpu_util import announce, rel_l2

MAX_ABS = 2e-2
REL_L2 = 1e-3


@dataclasses.dataclass
class StepStat:
    step: int
    row: int
    max_abs: float
    rel: float
    argmax_ok: bool
    gap: float


def top2_gap(l: np.ndarray) -> float:
    t = np.partition(l.astype(np.float64), -2)[-2:]
    return float(abs(t[1] - t[0]))


def near_tie(ref: np.ndarray) -> float:
    """Greedy picks within this much of the oracle's largest logit are all correct: twice
    the per-element deviation that the relative-L2 bar allows on average (REL_L2 times the
    row's rms logit). Above it the engine must pick the oracle's argmax."""
    return 2.0 * REL_L2 * float(np.sqrt(np.mean(np.square(ref.astype(np.float64)))))


def compare(step: int, row: int, got: np.ndarray, ref: np.ndarray) -> StepStat:
    ga, ra = int(np.argmax(got)), int(np.argmax(ref))
    ok = ga == ra or float(ref[ra]) - float(ref[ga]) < near_tie(ref)
    return StepStat(step, row, float(np.abs(got - ref).max()), rel_l2(got, ref), ok, top2_gap(ref))


def failures(stats: List[StepStat], greedy: bool = True) -> List[StepStat]:
    """Steps outside the logits bar; with greedy decoding the argmax must agree as well
    (with sampling the argmax is not a decision of the method: the sampled tokens are
    checked separately)."""
    return [s for s in stats
            if s.max_abs > MAX_ABS or s.rel > REL_L2 or (greedy and not s.argmax_ok)]


@dataclasses.dataclass
class SamplerStat:
    step: int
    oracle_token: int
    gpu_token: int          # engine's sampler on the oracle's logits
    own_token: int          # engine's sampler on its own logits (reported, not gated)
    margin: float


def run_single(w: synth.Workload, prompt_len: int, steps: int, weights=None,
               sampler_stats: List[SamplerStat] | None = None, decode_path: int = 0,
               int8: bool = False, int4: bool = False) -> List[StepStat]:
    """Prefill a seeded prompt, then `steps` decode steps, batch 1, teacher-forced with the
    oracle's tokens (greedy at temperature 0, else drawn with the workload's uniforms).
    With sampling, the engine's sampler is also run on the oracle's own logits and must
    return the oracle's token whenever the decision margin exceeds 1e-9. int8: the engine
    quantises the weights at load (weight-only int8) and the oracle runs the model with
    the same quantised weights (oracle.quant); int4 likewise with the 4-bit rule."""
    import torch
    from decoder_only_amd import q3
    from oracle import quant

    weights = synth.make_weights(w) if weights is None else weights
    max_seq = prompt_len + steps + 1
    qbits = 8 if int8 else 4 if int4 else 0
    model = oracle.Model(oracle.Config.from_workload(w), quant.quantized_weights(weights, qbits) if qbits else weights)
    cache = model.new_cache(max_seq)
    announce("e2e", w.name, w.n_layers, w.vocab, w.weight_dtype, prompt_len, steps, f"int{qbits}" if qbits else "")
    eng = q3.Engine(q3.config(w, 1, max_seq, int8=int8, int4=int4), weights)
    eng.set_decode_path(decode_path)
    prompt = synth.prompt_tokens(w, prompt_len)
    T, p = float(np.float32(w.temperature)), float(np.float32(w.top_p))
    us = synth.uniforms(w, steps + 1)
    u_dev = torch.from_numpy(us).cuda()
    ref = model.forward(prompt, cache, 0)
    logits = torch.empty(1, w.vocab, dtype=torch.float32, device="cuda")
    ref_dev = torch.empty(1, w.vocab, dtype=torch.float32, device="cuda")
    eng.prefill(0, torch.from_numpy(prompt).cuda(), logits)
    stats = []
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    chk = torch.empty(1, dtype=torch.int32, device="cuda")
    for step in range(steps + 1):
        eng.sync()
        stats.append(compare(step, 0, logits[0].cpu().numpy(), ref))
        if T == 0:
            nxt = int(np.argmax(ref))
        else:
            nxt = oracle.sample(ref, T, p, float(us[step]))
            if sampler_stats is not None:
                eng.sample(chk, T, p, u_dev[step:step + 1], logits=logits)
                own = int(chk.item())
                ref_dev.copy_(torch.from_numpy(ref).view(1, -1))
                eng.sample(chk, T, p, u_dev[step:step + 1], logits=ref_dev)
                sampler_stats.append(SamplerStat(step, nxt, int(chk.item()), own,
                                                 oracle.sample_margin(ref, T, p, float(us[step]))))
        if step == steps:
            break
        ref = model.forward([nxt], cache, prompt_len + step)
        tok.fill_(nxt)
        eng.decode_step(tok, None, logits)
    eng.close()
    return stats


def run_ragged(w: synth.Workload, prompt_lens: List[int], steps: int, decode_path: int = 0,
               qbits: int = 0) -> List[StepStat]:
    """Sequences of different lengths decoded together: sequence b is prefilled with a
    seeded prompt of prompt_lens[b] tokens, then `steps` batched decode steps (row b =
    sequence b, greedy, teacher-forced with each row's oracle token). qbits 8 / 4: the
    engine quantises the weights at load and the oracle runs the same quantised weights."""
    import torch
    from decoder_only_amd import q3
    from oracle import quant

    weights = synth.make_weights(w)
    B = len(prompt_lens)
    max_seq = max(prompt_lens) + steps + 1
    model = oracle.Model(oracle.Config.from_workload(w), quant.quantized_weights(weights, qbits) if qbits else weights)
    announce("e2e ragged", w.name, w.weight_dtype, prompt_lens, steps, decode_path, f"int{qbits}" if qbits else "")
    eng = q3.Engine(q3.config(w, B, max_seq, int8=qbits == 8, int4=qbits == 4), weights)
    eng.set_decode_path(decode_path)
    caches, refs = [], []
    for b, n in enumerate(prompt_lens):
        prompt = synth.prompt_tokens(w, n, seq=b)
        cache = model.new_cache(max_seq)
        refs.append(model.forward(prompt, cache, 0))
        caches.append(cache)
        eng.prefill(b, torch.from_numpy(prompt).cuda())
    logits = torch.empty(B, w.vocab, dtype=torch.float32, device="cuda")
    toks = torch.empty(B, dtype=torch.int32, device="cuda")
    stats = []
    for step in range(steps):
        nxt = [int(np.argmax(r)) for r in refs]
        toks.copy_(torch.tensor(nxt, dtype=torch.int32))
        eng.decode_step(toks, None, logits)
        refs = [model.forward([nxt[b]], caches[b], prompt_lens[b] + step) for b in range(B)]
        eng.sync()
        got = logits.cpu().numpy()
        stats += [compare(step, b, got[b], refs[b]) for b in range(B)]
    eng.close()
    return stats


def run_continuous(w: synth.Workload, steps: int, decode_path: int = 0, scale: int = 1) -> List[StepStat]:
    """Continuous batching on three sequence slots decoded together (greedy, teacher-forced):
    slot 0 holds a 7-token prompt; slot 2 an 11-token prompt prefilled in two calls (4 then
    7 tokens, the second one into a non-empty cache); slot 1 a 3-token prompt that is
    retired after 3 decode steps (q3_reset), its slot then admitting a new 5-token prompt,
    again prefilled in two calls (2 + 3), while the other slots keep decoding. Every slot's
    logits -- after each prefill and at every step -- are compared with an oracle run of
    that sequence alone, its prompt in one call. `scale` multiplies every prompt length and
    split point (at 40 and more, the prompts take the matrix-core prefill path, the second
    call of a split one attending to the first call's cache)."""
    import torch
    from decoder_only_amd import q3

    weights = synth.make_weights(w)
    B, retire_at = 3, 3
    max_seq = 11 * scale + steps + 1
    model = oracle.Model(oracle.Config.from_workload(w), weights)
    announce("e2e continuous", w.name, w.weight_dtype, steps, decode_path)
    eng = q3.Engine(q3.config(w, B, max_seq), weights)
    eng.set_decode_path(decode_path)
    one = torch.empty(1, w.vocab, dtype=torch.float32, device="cuda")
    stats: List[StepStat] = []

    def admit(slot: int, prompt: np.ndarray, split: int, tag: int):
        cache = model.new_cache(max_seq)
        ref = model.forward(prompt, cache, 0)
        parts = [prompt] if split == 0 else [prompt[:split], prompt[split:]]
        for part in parts:
            eng.prefill(slot, torch.from_numpy(np.ascontiguousarray(part)).cuda(), one)
        eng.sync()
        assert eng.seq_len(slot) == len(prompt)
        stats.append(compare(tag, slot, one[0].cpu().numpy(), ref))
        return cache, ref, len(prompt)

    k = scale
    state = [admit(0, synth.prompt_tokens(w, 7 * k, seq=0), 0, -1),
             admit(1, synth.prompt_tokens(w, 3 * k, seq=1), 0, -1),
             admit(2, synth.prompt_tokens(w, 11 * k, seq=2), 4 * k, -1)]
    logits = torch.empty(B, w.vocab, dtype=torch.float32, device="cuda")
    toks = torch.empty(B, dtype=torch.int32, device="cuda")
    for step in range(steps):
        if step == retire_at:
            eng.reset(1)
            assert eng.seq_len(1) == 0
            state[1] = admit(1, synth.prompt_tokens(w, 5 * k, seq=3), 2 * k, step)
        nxt = [int(np.argmax(ref)) for _, ref, _ in state]
        toks.copy_(torch.tensor(nxt, dtype=torch.int32))
        eng.decode_step(toks, None, logits)
        for b in range(B):
            cache, _, pos = state[b]
            state[b] = (cache, model.forward([nxt[b]], cache, pos), pos + 1)
        eng.sync()
        got = logits.cpu().numpy()
        stats += [compare(step, b, got[b], state[b][1]) for b in range(B)]
    eng.close()
    return stats
