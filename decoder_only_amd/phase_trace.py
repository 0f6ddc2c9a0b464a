"""Phase timeline of one persistent decode step (Qwen3-0.6B shape, synthetic weights).

    python -m decoder_only_amd.phase_trace [--ctx 70] [--batch 1]

Prefills `ctx` seeded prompt tokens per row, runs a few greedy decode steps, then one
traced step: thread 0 of workgroups 0 and 255 records the 100 MHz real-time counter at
every phase boundary of the persistent kernel (q3_profile_trace). Prints, per layer, the
mean / min / max of each segment in microseconds. The segment names hold for the
short-context instance (up to 240 visible slots); the split-K instances mark the same
points, with the partial merge inside "B: attention".
"""
import argparse

import numpy as np

NAMES = ["A: norm", "A: QKV dot+put", "hop QKV", "B: prep", "B: attention", "B: oproj+put", "hop P",
         "C: sum x'", "C: norm", "C: GU+put", "hop A", "D: down+put", "hop X"]
MARKS = 400   # the kernel keeps at most this many marks per traced workgroup


def main() -> None:
    import torch

    import synth
    from decoder_only_amd import q3

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--ctx", type=int, default=70, help="prompt tokens per row before the traced step")
    ap.add_argument("--batch", type=int, default=1, help="rows decoded together (1..4)")
    args = ap.parse_args()
    ctx, B = args.ctx, args.batch
    w = synth.workload("bs1_short")
    eng = q3.Engine(q3.config(w, B, max(4160, ctx + 64)), synth.make_weights(w))
    prompt = torch.from_numpy(synth.prompt_tokens(w, ctx)).cuda()
    for b in range(B):
        eng.prefill(b, prompt)
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    eng.sample(tok, 0.0)
    for _ in range(5):
        eng.decode_step(tok)
        eng.sample(tok, 0.0)
    buf = torch.zeros(2, MARKS, dtype=torch.int64, device="cuda")
    eng.profile_trace(buf)
    eng.decode_step(tok)
    eng.sample(tok, 0.0)
    eng.sync()
    eng.profile_trace(None)
    marks = buf.cpu().numpy()
    L = w.n_layers
    for row, name in [(0, "workgroup 0"), (1, "workgroup 255")]:
        v = marks[row][marks[row] > 0]
        d = np.diff(v) * 10 / 1000.0   # 100 MHz ticks -> us
        print(f"{name}: {ctx} cached slots, batch {B}: {(v[-1] - v[0]) * 10 / 1000.0:.1f} us over {len(v)} marks")
        print(f"  start -> layer-0 input {d[0]:.2f} us; LM head {d[-1]:.2f} us")
        K = (len(d) - 2) // L
        names = NAMES if K == len(NAMES) else [f"segment {i}" for i in range(K)]
        lay = d[1:1 + K * L].reshape(L, K)
        for k, nm in enumerate(names):
            print(f"  {nm:16s} mean {lay[:, k].mean():6.2f}  min {lay[:, k].min():6.2f}  max {lay[:, k].max():6.2f}")
        print(f"  per layer {lay.sum(1).mean():.2f} us")
    eng.close()


if __name__ == "__main__":
    main()
