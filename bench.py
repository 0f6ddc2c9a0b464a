#!/usr/bin/env python3
"""Throughput of the q3 engine on one MI355X: Qwen3-0.6B-shaped decoder, synthetic data.

Main line (`value`): decode tokens/s at batch 1 on the Qwen3-0.6B shape (28 layers,
bf16 weights and KV cache, random-init weights ~N(0, 0.02), tied vocab 151936). One
bench step is one whole generation: prefill a 5-token random prompt, then 128 greedy
decode steps, each followed by on-device sampling whose token feeds the next step.
value = 128 * steps / (wall time of the timed steps).

Also reported (one JSON line, under "extras"): the 2048-token prompt's prefill tokens/s and
its 256 sampled decode steps, batch-64 decode tokens/s with 4096 pre-filled KV slots per
sequence, the 32768-token prefill (GEMM and attention TFLOP/s) and its 512 sampled decode
steps, each with its roofline fraction; a 262,136-token prefill and decode at ~262K cached
slots; the bs1 workload on weight-only int8 and int4 weights; the roofline of the dominant kernel (event-timed on the engine's stream), and the CPU
oracle on this host (a bounded sample of decode steps and one 2048-token prefill).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-extras", action="store_true", help="skip the prefill and batch-64 lines")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 32768-token workload's engine and the 262K-context engine")
    ap.add_argument("--cooperative", action="store_true",
                    help="dispatch the persistent decode kernel as a cooperative launch (the engine's "
                         "default); by default the bench, which has the GPU to itself, uses an "
                         "ordinary launch: every workgroup is resident at once either way, and the "
                         "ordinary dispatch starts ~13 us sooner per step")
    ap.add_argument("--plain-launch", action="store_true", help="(the default; kept for old command lines)")
    ap.add_argument("--prefill-only-extras", action="store_true",
                    help="of the extra lines run only the 2048-token prefill (counter passes over its kernels)")
    ap.add_argument("--one-launch-mode", action="store_true",
                    help="skip the bs1 line under the other launch mode (profiling runs keep to ordinary launches)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain streaming kernel (torch.neg) over MIB MiB of float32, three "
                         "times: a known-size reference for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); "
              "the engine is single-GPU and has no multi-GPU path", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from decoder_only_amd import q3

    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration << 18, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    w = synth.workload("bs1_short")
    t = time.time()
    weights = synth.make_weights(w)
    log(f"weights generated in {time.time() - t:.1f}s")
    max_batch, max_seq = 64, 4168      # batch-64 line: 4096 pre-filled + 2 warm-up + 64 timed + 2 profiled steps
    eng = q3.Engine(q3.config(w, max_batch, max_seq), weights)
    if not args.cooperative:
        eng.set_decode_path(3)
    log("engine loaded")

    prompt = torch.from_numpy(synth.prompt_tokens(w)).cuda()
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    n_dec = w.decode_steps

    def generation():
        eng.reset(0)
        eng.prefill(0, prompt)
        eng.sample(tok, 0.0)
        for _ in range(n_dec):
            eng.decode_step(tok)
            eng.sample(tok, 0.0)

    for _ in range(args.warmup):
        generation()
    eng.sync()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        generation()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eng.sync()
    elapsed = t1 - t0
    value = n_dec * args.steps / elapsed
    ms_per_step = 1000.0 * elapsed / args.steps
    log(f"bs1 decode: {value:.1f} tok/s, {ms_per_step:.2f} ms per generation")
    # the same generations with the other launch mode of the persistent kernel, for comparison
    launch_mode = "cooperative" if args.cooperative else "ordinary"
    other_mode = "ordinary" if args.cooperative else "cooperative"
    other = None
    if not args.one_launch_mode:
        eng.set_decode_path(0 if not args.cooperative else 3)
        generation()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            generation()
        torch.cuda.synchronize()
        other = n_dec * args.steps / (time.perf_counter() - t0)
        eng.set_decode_path(3 if not args.cooperative else 0)
        log(f"bs1 decode with the {other_mode} launch: {other:.1f} tok/s")

    # Roofline of the dominant kernel, event-timed on the engine's stream over a second pass
    # of the same steps. With the persistent decode kernel (one launch per decode step) that
    # kernel is the whole step; otherwise it is the decode GEMV family (most bytes per step).
    eng.profile_begin(q3.PROF_DECODE_STEP)
    for _ in range(args.steps):
        generation()
    step = eng.profile_end()
    eng.profile_begin(q3.PROF_GEMV)
    for _ in range(args.steps):
        generation()
    gemv = eng.profile_end()
    step_gbs = step["bytes"] / (step["ms"] / 1e3) / 1e9
    step_us = 1e3 * step["ms"] / step["launches"]
    extras = {"decode_step_us": round(step_us, 2), "decode_step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
              "bs1_launch": launch_mode}
    if other is not None:
        extras[f"bs1_decode_tok_s_{other_mode}_launch"] = round(other, 2)
    if gemv["launches"] == 0:
        roofline = {"kernel": "k_decode_mega (persistent decode step: all layers, LM head, argmax)",
                    "bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                    "traffic": stored_traffic("k_decode_mega_bs1_traffic.md", MEGA_SOURCES),
                    "avg_launch_us": round(step_us, 3),
                    "bytes_per_launch": round(step["bytes"] / step["launches"])}
    else:
        gemv_gbs = gemv["bytes"] / (gemv["ms"] / 1e3) / 1e9
        roofline = {"kernel": "decode GEMV (q/k/v, o, gate/up, down)", "bound": "hbm",
                    "achieved": round(gemv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gemv_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                    "avg_launch_us": round(1e3 * gemv["ms"] / gemv["launches"], 3),
                    "bytes_per_launch": round(gemv["bytes"] / gemv["launches"])}
    log(f"decode step {step_us:.1f} us ({step_gbs:.0f} GB/s algorithmic, {100 * step_gbs / HBM_PEAK_GBS:.1f}% of HBM)")

    if not args.no_extras:
        try:
            extras.update(prefill_line(eng, w, q3, torch, synth))
        except Exception as ex:  # the main line is still reported
            extras["prefill_error"] = repr(ex)
    if not args.no_extras and not args.prefill_only_extras:
        try:
            extras.update(c3_decode_line(eng, q3, torch, synth))
        except Exception as ex:
            extras["c3_error"] = repr(ex)
        try:
            extras.update(bs64_line(eng, w, q3, torch, synth, max_seq))
        except Exception as ex:
            extras["bs64_error"] = repr(ex)
        try:
            extras.update(quant_line(weights, q3, torch, synth, args.steps, 8))
        except Exception as ex:
            extras["int8_error"] = repr(ex)
        try:
            extras.update(quant_line(weights, q3, torch, synth, args.steps, 4))
        except Exception as ex:
            extras["int4_error"] = repr(ex)

    cpu = None
    if not args.no_cpu:
        try:
            cpu = cpu_baseline(w, weights, args.cpu_seconds)
        except Exception as ex:
            cpu = {"error": repr(ex)}
    eng.close()
    if not args.no_extras and not args.no_long and not args.prefill_only_extras:
        try:
            extras.update(c5_lines(weights, q3, torch, synth))
        except Exception as ex:
            extras["c5_error"] = repr(ex)
        try:
            extras.update(ctx262k_lines(weights, q3, torch, synth))
        except Exception as ex:
            extras["ctx262k_error"] = repr(ex)

    out = {
        "metric": "decode tok/s (bs1, bs64) + prefill tok/s, Qwen3-0.6B shape; % of roofline",
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights/KV, f32 activations",
        "data": "synthetic: random-init weights N(0,0.02), uniform random token ids",
        "config": {"workload": "Qwen3-0.6B shape, batch 1, 5-token prompt + 128 greedy decode steps "
                               "(one step = one generation)",
                   "layers": w.n_layers, "hidden": w.hidden, "heads": f"{w.n_heads}q/{w.n_kv_heads}kv",
                   "vocab": w.vocab, "global_batch": 1, "seq_len": w.prompt_len + w.decode_steps,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)
    return 0


def prefill_line(eng, w, q3, torch, synth):
    """2048-token prompt prefill (the long-prompt workload), timed alone."""
    n = 2048
    toks = torch.from_numpy(synth.prompt_tokens(w.with_(seed=1003), n)).cuda()
    for _ in range(2):
        eng.reset(0)
        eng.prefill(0, toks)
    eng.sync()
    reps = 5
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        eng.reset(0)
        eng.prefill(0, toks)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    eng.reset(0)
    eng.profile_begin(q3.PROF_GEMM)
    eng.prefill(0, toks)
    g = eng.profile_end()
    eng.reset(0)
    eng.profile_begin(q3.PROF_ATTN_PREFILL)
    eng.prefill(0, toks)
    a = eng.profile_end()
    eng.reset(0)
    gt = g["flops"] / (g["ms"] / 1e3) / 1e12
    at = a["flops"] / (a["ms"] / 1e3) / 1e12
    log(f"prefill {n}: {n / dt:.0f} tok/s; GEMM {gt:.0f} TFLOP/s; attention {at:.0f} TFLOP/s")
    return {"prefill2048_tok_s": round(n / dt, 1), "prefill2048_ms": round(1e3 * dt, 3),
            "prefill_gemm_tflops": round(gt, 1), "prefill_gemm_frac": round(gt / BF16_PEAK_TFLOPS, 4),
            "prefill_attn_tflops": round(at, 1)}


def decode_loop(eng, q3, torch, tok, steps, temperature, top_p, u):
    """steps x [decode step + sampling] from the engine's current state; returns (seconds,
    HIP-event-timed persistent-kernel profile of the same steps)."""
    torch.cuda.synchronize()
    eng.profile_begin(q3.PROF_DECODE_STEP)
    t0 = time.perf_counter()
    for i in range(steps):
        eng.decode_step(tok)
        eng.sample(tok, temperature, top_p, None if u is None else u[i + 1:i + 2])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return dt, eng.profile_end()


def c3_decode_line(eng, q3, torch, synth):
    """The 2048-token workload's decode: prefill the 2048-token prompt, then its 256 steps
    sampled at T = 0.7, p = 0.9 with the workload's uniforms (2049..2304 cached slots)."""
    wl = synth.workload("prefill2k")
    toks = torch.from_numpy(synth.prompt_tokens(wl)).cuda()
    u = torch.from_numpy(synth.uniforms(wl)).cuda()
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    res = None
    for _ in range(2):                                  # warm-up, then the timed run
        eng.reset(0)
        eng.prefill(0, toks)
        eng.sample(tok, wl.temperature, wl.top_p, u[0:1])
        res = decode_loop(eng, q3, torch, tok, wl.decode_steps, wl.temperature, wl.top_p, u)
    eng.reset(0)
    dt, prof = res
    gbs = prof["bytes"] / (prof["ms"] / 1e3) / 1e9
    log(f"2048-token workload decode: {wl.decode_steps / dt:.0f} tok/s; step kernel {gbs:.0f} GB/s")
    return {"c3_decode_tok_s": round(wl.decode_steps / dt, 1),
            "c3_decode_step_us": round(1e3 * prof["ms"] / max(1, prof["launches"]), 2),
            "c3_decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def c5_lines(weights, q3, torch, synth):
    """The long-context workload on an engine of its own (1 sequence, 33,281 slots): the
    32768-token prefill (tok/s, GEMM and attention TFLOP/s), then its 512 decode steps
    sampled at T = 1.0, p = 0.95 (32769..33280 cached slots). Weights: the bs1 workload's
    synthetic tensors (the timing does not depend on their values)."""
    wl = synth.workload("prefill32k")
    eng = q3.Engine(q3.config(wl, 1, wl.prompt_len + wl.decode_steps + 1), weights)
    try:
        toks = torch.from_numpy(synth.prompt_tokens(wl)).cuda()
        u = torch.from_numpy(synth.uniforms(wl)).cuda()
        tok = torch.empty(1, dtype=torch.int32, device="cuda")
        eng.prefill(0, toks)                            # warm-up
        eng.sync()
        eng.reset(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eng.prefill(0, toks)
        torch.cuda.synchronize()
        tp = time.perf_counter() - t0
        eng.reset(0)
        eng.profile_begin(q3.PROF_GEMM)
        eng.prefill(0, toks)
        g = eng.profile_end()
        eng.reset(0)
        eng.profile_begin(q3.PROF_ATTN_PREFILL)
        eng.prefill(0, toks)
        a = eng.profile_end()
        eng.sample(tok, wl.temperature, wl.top_p, u[0:1])
        dt, prof = decode_loop(eng, q3, torch, tok, wl.decode_steps, wl.temperature, wl.top_p, u)
        eng.sync()
    finally:
        eng.close()
    n = wl.prompt_len
    gt = g["flops"] / (g["ms"] / 1e3) / 1e12
    at = a["flops"] / (a["ms"] / 1e3) / 1e12
    gbs = prof["bytes"] / (prof["ms"] / 1e3) / 1e9
    log(f"prefill {n}: {n / tp:.0f} tok/s; GEMM {gt:.0f} TFLOP/s; attention {at:.0f} TFLOP/s; "
        f"decode {wl.decode_steps / dt:.0f} tok/s, step kernel {gbs:.0f} GB/s")
    return {"prefill32k_tok_s": round(n / tp, 1), "prefill32k_ms": round(1e3 * tp, 2),
            "prefill32k_gemm_tflops": round(gt, 1), "prefill32k_gemm_frac": round(gt / BF16_PEAK_TFLOPS, 4),
            "prefill32k_attn_tflops": round(at, 1),
            "c5_decode_tok_s": round(wl.decode_steps / dt, 1),
            "c5_decode_step_us": round(1e3 * prof["ms"] / max(1, prof["launches"]), 2),
            "c5_decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def quant_line(weights, q3, torch, synth, steps, bits):
    """The bs1 workload (5-token prompt, 128 greedy steps per generation) on an engine whose
    weights are quantised to int8 (bits = 8: one byte per weight) or int4 (bits = 4: half a
    byte) at load, plus a float scale per row: decode tok/s over whole generations, and the
    persistent kernel's HBM fraction against the quantised step's algorithmic bytes."""
    w = synth.workload("bs1_short")
    eng = q3.Engine(q3.config(w, 1, w.max_seq + 1, int8=bits == 8, int4=bits == 4), weights)
    try:
        eng.set_decode_path(3)
        prompt = torch.from_numpy(synth.prompt_tokens(w)).cuda()
        tok = torch.empty(1, dtype=torch.int32, device="cuda")

        def generation():
            eng.reset(0)
            eng.prefill(0, prompt)
            eng.sample(tok, 0.0)
            for _ in range(w.decode_steps):
                eng.decode_step(tok)
                eng.sample(tok, 0.0)

        generation()
        eng.sync()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            generation()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        eng.profile_begin(q3.PROF_DECODE_STEP)
        for _ in range(steps):
            generation()
        prof = eng.profile_end()
        eng.sync()
    finally:
        eng.close()
    gbs = prof["bytes"] / (prof["ms"] / 1e3) / 1e9
    us = 1e3 * prof["ms"] / prof["launches"]
    k = f"int{bits}"
    log(f"{k} bs1 decode: {w.decode_steps * steps / dt:.0f} tok/s; step {us:.1f} us "
        f"({prof['bytes'] / prof['launches'] / 1e9:.3f} GB, {gbs:.0f} GB/s)")
    return {f"{k}_bs1_decode_tok_s": round(w.decode_steps * steps / dt, 2), f"{k}_decode_step_us": round(us, 2),
            f"{k}_step_bytes": round(prof["bytes"] / prof["launches"]),
            f"{k}_decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def ctx262k_lines(weights, q3, torch, synth):
    """Context toward 262K on an engine of its own (1 sequence, 262,160 slots; weights of the
    bs1 workload): a prefill of 262,136 seeded random tokens timed once (the kernels are warm
    from the 32768-token line), then 8 greedy decode steps at 262,139 .. 262,146 cached
    slots (after 2 untimed ones) with the persistent kernel's HBM fraction."""
    w = synth.workload("bs1_short")
    n = 262136
    eng = q3.Engine(q3.config(w, 1, 262160), weights)
    try:
        eng.set_decode_path(3)
        toks = torch.from_numpy(synth.prompt_tokens(w.with_(seed=1006), n)).cuda()
        tok = torch.empty(1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eng.prefill(0, toks)
        torch.cuda.synchronize()
        tp = time.perf_counter() - t0
        eng.sample(tok, 0.0)
        for _ in range(2):
            eng.decode_step(tok)
            eng.sample(tok, 0.0)
        eng.sync()
        dt, prof = decode_loop(eng, q3, torch, tok, 8, 0.0, 1.0, None)
        eng.sync()
    finally:
        eng.close()
    flops = 2.0 * (n - 1) * 440401920 + 512.0 * 16 * 27 * (n - 1) * n / 2.0   # GEMMs + 27 layers' causal attention
    gbs = prof["bytes"] / (prof["ms"] / 1e3) / 1e9
    log(f"prefill {n}: {n / tp:.0f} tok/s ({flops / tp / 1e12:.0f} TFLOP/s); decode at 262K slots "
        f"{8 / dt:.1f} tok/s, step kernel {gbs:.0f} GB/s")
    return {"prefill262k_tok_s": round(n / tp, 1), "prefill262k_s": round(tp, 2),
            "prefill262k_tflops": round(flops / tp / 1e12, 1),
            "ctx262k_decode_tok_s": round(8 / dt, 2),
            "ctx262k_decode_step_us": round(1e3 * prof["ms"] / max(1, prof["launches"]), 1),
            "ctx262k_decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bs64_line(eng, w, q3, torch, synth, max_seq):
    """64 sequences with 4096 pre-filled K/V slots each (synthetic N(0,1) bf16), 64 greedy
    steps timed (after two untimed ones: 4099 .. 4162 cached slots)."""
    B, T0, steps = 64, 4096, 64
    gen = torch.Generator(device="cuda").manual_seed(1004)
    for b in range(B):
        for layer in range(w.n_layers):
            kv = torch.randn(2, w.n_kv_heads, T0, w.head_dim, generator=gen, device="cuda").bfloat16()
            eng.kv_import(b, layer, kv[0].contiguous(), kv[1].contiguous(), T0)
    toks = torch.from_numpy(synth.batch_first_tokens(w.with_(seed=1004, batch=B))).cuda()
    # two untimed warm-up steps (the batch path's kernels load on first use), then the
    # workload's 64 greedy steps at 4099 .. 4162 cached slots
    for _ in range(2):
        eng.decode_step(toks)
        eng.sample(toks, 0.0)
    eng.sync()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        eng.decode_step(toks)
        eng.sample(toks, 0.0)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    eng.profile_begin(q3.PROF_ATTN_DECODE)
    eng.decode_step(toks)
    eng.sample(toks, 0.0)
    a = eng.profile_end()
    eng.profile_begin(q3.PROF_DECODE_STEP)              # the whole step, all its kernels
    eng.decode_step(toks)
    eng.sample(toks, 0.0)
    st = eng.profile_end()
    for b in range(B):
        eng.reset(b)
    ag = a["bytes"] / (a["ms"] / 1e3) / 1e9
    sg = st["bytes"] / (st["ms"] / 1e3) / 1e9
    log(f"bs64 decode: {B * steps / dt:.0f} tok/s; attention {ag:.0f} GB/s; whole step {sg:.0f} GB/s")
    return {"bs64_decode_tok_s": round(B * steps / dt, 1), "bs64_step_ms": round(1e3 * dt / steps, 3),
            "bs64_attn_gbs": round(ag, 1), "bs64_attn_hbm_frac": round(ag / HBM_PEAK_GBS, 4),
            "bs64_step_hbm_frac": round(sg / HBM_PEAK_GBS, 4)}


def stored_traffic(md_name, sources):
    """HBM bytes per launch of a kernel as recorded under profiles/ from two hardware-counter
    passes (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads for a
    plain streaming kernel of known size. None when the record is missing or was taken on
    other kernel sources than the ones in this tree."""
    h = hashlib.sha256()
    try:
        for rel in sources:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        with open(os.path.join(ROOT, "profiles", md_name)) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"kernel sources sha256: `([0-9a-f]{64})`", text)
    t = re.search(r"HBM traffic per launch: `(\d+)` bytes", text)
    if not m or not t or m.group(1) != h.hexdigest():
        return None
    return int(t.group(1))


MEGA_SOURCES = ("decoder_only_amd/csrc/decode_mega.hip", "decoder_only_amd/csrc/decode_mega.h",
                "decoder_only_amd/csrc/kv_layout.h", "decoder_only_amd/csrc/common.h")


def host_cpu():
    """CPU model, physical cores and logical CPUs this process may use."""
    cpus = sorted(os.sched_getaffinity(0))
    model, cores = "unknown", set()
    try:
        info, cur = {}, {}
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    if "processor" in cur:
                        info[int(cur["processor"])] = cur
                    cur = {}
                    continue
                k, _, v = line.partition(":")
                cur[k.strip()] = v.strip()
        if "processor" in cur:
            info[int(cur["processor"])] = cur
        for c in cpus:
            d = info.get(c, {})
            model = d.get("model name", model)
            cores.add((d.get("physical id", "0"), d.get("core id", str(c))))
    except OSError:
        pass
    return model, len(cores) or len(cpus), len(cpus)


def cpu_baseline(w, weights, budget_s):
    """The oracle (NumPy) on this host: greedy decode steps of the bs1 workload until the
    budget is spent, and one 2048-token prefill of the long-prompt workload's shape."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    model_name, phys, logical = host_cpu()
    model = oracle.Model(oracle.Config.from_workload(w), weights)
    prompt = synth.prompt_tokens(w)
    # whole generations (5-token prefill untimed, then the greedy decode steps, timed),
    # repeated until the budget is spent; a generation may stop early at the budget
    n, dt, gens = 0, 0.0, 0
    while dt < budget_s:
        cache = model.new_cache(w.max_seq)
        logits = model.forward(prompt, cache, 0)
        gens += 1
        for i in range(w.decode_steps):
            t0 = time.perf_counter()
            logits = model.forward([int(np.argmax(logits))], cache, w.prompt_len + i)
            dt += time.perf_counter() - t0
            n += 1
            if dt >= budget_s:
                break
    long_prompt = synth.prompt_tokens(w.with_(seed=1003), 2048)
    t0 = time.perf_counter()
    model.forward(long_prompt, model.new_cache(2048), 0)
    tp = time.perf_counter() - t0
    log(f"oracle: {n / dt:.2f} tok/s over {n} steps in {gens} generations; 2048-token prefill {tp:.1f} s "
        f"({threads} BLAS threads; {phys} physical cores, {logical} logical CPUs; {model_name})")
    return {"value": round(n / dt, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"batch-1 Qwen3-0.6B shape: {n} greedy decode steps over {gens} generations of "
                      f"the workload (5-token prompt, up to {w.decode_steps} steps each; {dt:.1f} s of decode)",
            "cpu_model": model_name, "physical_cores": phys, "logical_cpus": logical,
            "prefill2048_s": round(tp, 2), "prefill2048_tok_s": round(2048 / tp, 1),
            "decode_s_per_step": round(dt / n, 4)}


if __name__ == "__main__":
    sys.exit(main())
