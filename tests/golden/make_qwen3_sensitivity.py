"""Rounding sensitivity of the Qwen3-1.7B-shaped forward, from the oracle alone.

Writes tests/golden/qwen3_oracle_fp32_sensitivity.txt: for the 16 sequences of the
2-prompt x 8-response subset of the recompute workload (seeded weights and ids of
``synth``), the logprobs of the fp64 oracle against the same oracle with every linear
layer's dot products accumulated in fp32 instead of fp64 (the inputs are bf16 values,
exact in fp32, so only the accumulation precision changes; the outputs are rounded to
bf16 at the same storage points).  A GPU forward accumulates its GEMMs in fp32, so this
is how far a correct fp32-accumulating implementation can sit from the fp64 oracle on
this random-init 28-layer model; the end-to-end GPU tolerance of the Qwen3-shaped
parity test is set from it.  For the shortest sequence it also records, per layer, the
relative RMS gap of the residual stream and the MLP output between the two runs.

Nothing here comes from the HIP path: only ``oracle`` and ``synth`` are imported.

    python tests/golden/make_qwen3_sensitivity.py [--seqs N]
"""
from __future__ import annotations

import argparse
import contextlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle import ops  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "qwen3_oracle_fp32_sensitivity.txt")


def linear_f32(x, w):
    """x . w^T with fp32 operands and fp32 accumulation (BLAS sgemm), widened to fp64."""
    return (np.asarray(x, np.float32) @ np.asarray(w, np.float32).T).astype(np.float64)


@contextlib.contextmanager
def fp32_accumulation():
    saved = ops.linear
    ops.linear = linear_f32
    try:
        yield
    finally:
        ops.linear = saved


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seqs", type=int, default=16)
    args = ap.parse_args()
    cfg = synth.QWEN3_1P7B
    weights = synth.make_weights(cfg)
    seqs = synth.rl_sequences(cfg, n_prompts=2, n_responses=8)
    W = om.Weights({k: synth.bf16_bits(v) for k, v in weights.items()}, cache=False)
    order = sorted(range(len(seqs)), key=lambda i: seqs[i].length)[: args.seqs]
    lines = []
    worst_max = worst_mean = 0.0
    for n, i in enumerate(order):
        s = seqs[i]
        t0 = time.perf_counter()
        dump64, dump32 = ([], []) if n == 0 else (None, None)
        ref = om.sequence_logprobs(cfg, W, s.tokens, s.prompt_len, dump=dump64)
        with fp32_accumulation():
            alt = om.sequence_logprobs(cfg, W, s.tokens, s.prompt_len, dump=dump32)
        d = np.abs(alt.astype(np.float64) - ref.astype(np.float64))
        worst_max, worst_mean = max(worst_max, float(d.max())), max(worst_mean, float(d.mean()))
        line = (f"seq {i:2d} L={s.length:3d} scored={s.n_scored:3d} "
                f"max={d.max():.4e} mean={d.mean():.4e}")
        lines.append(line)
        print(line, f"({time.perf_counter() - t0:.0f} s)", flush=True)
        if n == 0:
            for l, (a, b) in enumerate(zip(dump32, dump64)):
                lines.append(f"  layer {l:2d} rel_rms r={rel(a['r'], b['r']):.4e} m={rel(a['m'], b['m']):.4e}")
    lines.append(f"worst over sequences: max={worst_max:.4e} mean={worst_mean:.4e}")
    with open(OUT, "w") as f:
        f.write("# fp64 oracle vs the same oracle with fp32-accumulating linear layers\n")
        f.write("# Qwen3-1.7B-shaped, random init (synth seeds), 2 prompts x 8 responses\n")
        f.write(f"# command: python tests/golden/make_qwen3_sensitivity.py --seqs {args.seqs}\n")
        f.write("\n".join(lines) + "\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
