#!/usr/bin/env python3
"""Write stored oracle outputs for workloads too long to run the oracle inside a GPU test.

Calls only oracle/ (the CPU reference) and synth/ (seeded inputs). Usage:
    python tests/golden/make_goldens.py prefill32k [--steps N]

Output: tests/golden/<workload>.npz with, per step s (s = 0 is the prefill's last row,
s >= 1 the decode steps), under teacher forcing with the oracle's own sampled tokens:
  tokens[s]       token sampled from step s's logits (fed to step s + 1)
  u[s]            the uniform that drove that draw
  margin[s]       sampler decision margin (oracle.sample_margin)
  argmax[s], gap[s], norm[s]    argmax, top-2 logit gap, L2 norm of the logits
  top_ids[s], top_vals[s]       the 32 largest logits
  probe_vals[s]   logits at the fixed ids probe_ids (seeded, shared by all steps)
and the whole logit row at the steps full_steps (step 0, the last step and N_FULL seeded
steps in between): full_logits[i] belongs to step full_steps[i] (full_logits0 = step 0).
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

N_TOP = 32
N_PROBE = 256
N_FULL = 10


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--steps", type=int, default=None, help="decode steps (default: the workload's)")
    args = ap.parse_args()
    w = synth.workload(args.workload)
    steps = w.decode_steps if args.steps is None else args.steps
    t0 = time.time()
    weights = synth.make_weights(w)
    model = oracle.Model(oracle.Config.from_workload(w), weights)
    del weights
    cache = model.new_cache(w.prompt_len + steps + 1)
    prompt = synth.prompt_tokens(w)
    us = synth.uniforms(w, steps + 1)
    T = float(np.float32(w.temperature))
    p = float(np.float32(w.top_p))
    probe_ids = np.sort(np.random.default_rng([w.seed, 7]).choice(w.vocab, N_PROBE, replace=False))
    inner = np.random.default_rng([w.seed, 8]).choice(np.arange(1, steps), min(N_FULL, max(0, steps - 1)),
                                                      replace=False)
    full_steps = np.unique(np.concatenate([[0, steps], inner])).astype(np.int32)
    full_rows = []
    print(f"[{time.time() - t0:.0f}s] prefill {len(prompt)}", flush=True)
    logits = model.forward(prompt, cache, 0)
    rec = {k: [] for k in ("tokens", "u", "margin", "argmax", "gap", "norm", "top_ids", "top_vals", "probe_vals")}
    full0 = logits.copy()
    for s in range(steps + 1):
        u = float(us[s])
        tok = oracle.sample(logits, T, p, u)
        order = np.argsort(-logits, kind="stable")[:N_TOP]
        srt = np.sort(logits.astype(np.float64))
        rec["tokens"].append(tok)
        rec["u"].append(us[s])
        rec["margin"].append(oracle.sample_margin(logits, T, p, u))
        rec["argmax"].append(int(np.argmax(logits)))
        rec["gap"].append(float(srt[-1] - srt[-2]))
        rec["norm"].append(float(np.linalg.norm(logits.astype(np.float64))))
        rec["top_ids"].append(order.astype(np.int32))
        rec["top_vals"].append(logits[order])
        rec["probe_vals"].append(logits[probe_ids])
        if s in full_steps:
            full_rows.append(logits.copy())
        if s == steps:
            break
        logits = model.forward([tok], cache, len(prompt) + s)
        if s % 16 == 0:
            print(f"[{time.time() - t0:.0f}s] step {s + 1}/{steps}", flush=True)
    out = os.path.join(HERE, f"{w.name}.npz")
    np.savez_compressed(
        out, workload=w.name, temperature=np.float32(w.temperature), top_p=np.float32(w.top_p),
        prompt_len=len(prompt), probe_ids=probe_ids.astype(np.int32), full_logits0=full0,
        full_steps=full_steps, full_logits=np.stack(full_rows),
        tokens=np.array(rec["tokens"], np.int32), u=np.array(rec["u"], np.float32),
        margin=np.array(rec["margin"]), argmax=np.array(rec["argmax"], np.int32),
        gap=np.array(rec["gap"]), norm=np.array(rec["norm"]), top_ids=np.stack(rec["top_ids"]),
        top_vals=np.stack(rec["top_vals"]), probe_vals=np.stack(rec["probe_vals"]))
    print(f"[{time.time() - t0:.0f}s] wrote {out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
