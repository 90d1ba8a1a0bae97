#!/usr/bin/env python3
"""Throughput of the batch-invariant logprob recompute on one MI355X.

One step = the training-side recompute of every valid response token of a
GRPO-style batch: 128 prompts x 8 responses on a Qwen3-1.7B-shaped dense
decoder (28 layers, hidden 2048, 16 q / 8 kv heads of 128, MLP 6144, vocab
151936, tied embeddings), random-init bf16 weights, synthetic token ids
(prompt lengths U[80, 250], response lengths U[100, 400]).  Sequences are packed
into varlen calls of at most 16384 tokens; each call is one
bci_forward_logprobs (all kernels of the path: embedding, 28 x [add+RMSNorm,
QKV GEMM, RoPE + KV write, attention, O GEMM, add+RMSNorm, gate_up GEMM with
SiLU*up, down GEMM], final norm, lm_head + log-softmax + gather).

Reported on one JSON line: scored tokens/s, the roofline of the dominant
kernel (the gate_up GEMM, timed live with HIP events on its own stream), the
acceptance statistics of a bounded rollout-vs-recompute comparison (must be
exactly 0), and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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
sys.path.insert(0, ROOT)

def gate_up_traffic():
    """HBM bytes of one gate_up launch at M = 16384 from the committed counter profile
    (FETCH_SIZE + WRITE_SIZE, calibrated on a 1 GiB copy), or None when the GEMM source
    has changed since the counters were taken."""
    prof = os.path.join(ROOT, "profiles", "gate_up_gemm_hbm_counters.md")
    src = os.path.join(ROOT, "bitwise_consistent_rl_amd", "csrc", "gemm.hip")
    try:
        text = open(prof).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    m = re.search(r"traffic-record: gemm\.hip sha256=([0-9a-f]{64}) bytes_per_launch=(\d+) m=(\d+)", text)
    if not m or m.group(1) != digest:
        return None
    return {"bytes_per_launch": int(m.group(2)), "m": int(m.group(3))}


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
# attention segment (keys) of the Qwen3-shaped model's numeric contract: contexts of
# this workload stay below 1024 tokens, so every row's KV walk is one segment (the plain
# online softmax, no segment merges) in prefill, recompute and decode alike
QWEN_SEG_KEYS = 1024


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    """Threads the host BLAS may use: the job's CPU share (OMP_NUM_THREADS) if set."""
    try:
        return max(1, int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1))
    except ValueError:
        return os.cpu_count() or 1


def _best_of(fn, reps=3):
    best = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        best = min(best, time.perf_counter() - t0)
    return best


def cpu_baseline(cfg, weights, seqs, budget_s: float = 12.0):
    """The oracle, as it stands, timed on the host on bounded samples (fp64, NumPy BLAS).

    Headline: the shortest of the first 8 recompute sequences, then further sequences of
    the workload in order while the elapsed time stays under ``budget_s`` (scored tokens/s,
    all the job's cores).  Beside it, best of 3 with all cores and with one core, the
    other workloads' oracle on small cases: the tiny decoder's whole workload, the lm_head
    log-softmax at M = 64, the MoE layer at T = 1 and the FP8-cache decode attention of one
    query over 8192 keys."""
    import numpy as np
    import synth
    from oracle import model as om
    from oracle import ops
    from threadpoolctl import threadpool_limits
    cores = _blas_threads()
    first = min(seqs[:8], key=lambda q: q.length)
    W = om.Weights({k: synth.bf16_bits(v) for k, v in weights.items()}, cache=False)
    done, scored, dt = [], 0, 0.0
    with threadpool_limits(limits=cores):
        for s in [first] + [q for q in seqs if q is not first]:
            t0 = time.perf_counter()
            om.sequence_logprobs(cfg, W, s.tokens, s.prompt_len)
            dt += time.perf_counter() - t0
            done.append(s)
            scored += s.n_scored
            # stop when another sequence of this length would overrun the budget
            if dt * (len(done) + 1) / len(done) > budget_s:
                break

    # the other workloads, on small seeded cases
    tiny = synth.TINY
    tw = om.Weights({k: synth.bf16_bits(v) for k, v in synth.make_weights(tiny).items()})
    tseqs = synth.tiny_sequences(tiny)
    t_scored = sum(q.n_scored for q in tseqs)
    hs, lw, lids = synth.lmhead_inputs(64)
    hs64, lbits = synth.bf16_bits(hs).astype(np.uint16), synth.bf16_bits(lw)
    from oracle.codecs import bf16_decode
    hs64 = bf16_decode(hs64)
    moe_w = {k: synth.bf16_bits(v) for k, v in synth.moe_weights().items()}
    mh = bf16_decode(synth.bf16_bits(synth.normal_bf16((1, synth.MOE.hidden), index=50)))
    mz = synth.router_logits_quantised(1, seed=11)
    q, k, v = synth.fp8_attention_inputs(32, 4, 128, 8192)
    qd = bf16_decode(synth.bf16_bits(q))[-1:]
    kc, ks = ops.kv_quantise(bf16_decode(synth.bf16_bits(k)))
    vc, vs = ops.kv_quantise(bf16_decode(synth.bf16_bits(v)))

    def c1():
        for q_ in tseqs:
            om.sequence_logprobs(tiny, tw, q_.tokens, q_.prompt_len)

    def c3():
        ops.logprobs(hs64, lbits, lids)

    def c4():
        ids = ops.topk_ties(mz, synth.MOE.top_k)
        ops.moe_layer(mh, ids, ops.topk_weights(mz, ids), moe_w["wgu"], moe_w["wd"], moe_w["swgu"],
                      moe_w["swd"], synth.MOE.expert_intermediate)

    def c5():
        K = ops.kv_dequantise(kc, ks)
        V = ops.kv_dequantise(vc, vs)
        ops.causal_gqa_attention(qd, K, V, [8191])

    others = {}
    for name, fn, units, unit in (
            ("tiny_decoder_whole_workload", c1, t_scored, "scored tokens/s"),
            ("lmhead_logsoftmax_M64", c3, 64, "rows/s"),
            ("moe_layer_T1", c4, 1, "tokens/s"),
            ("fp8_decode_attention_8192_keys_B1", c5, 1, "decode steps/s")):
        row = {"unit": unit}
        for label, n in (("all_cores", cores), ("one_core", 1)):
            with threadpool_limits(limits=n):
                row[label] = round(units / _best_of(fn), 3)
        others[name] = row
    return {"value": round(scored / dt, 3), "unit": "scored tokens/s", "cores": int(cores),
            "kind": "oracle", "host_cpu": _host_cpu(),
            "sample": f"{len(done)} sequences of the workload (L = "
                      f"{', '.join(str(q.length) for q in done)}; {scored} scored tokens), "
                      f"fp64 NumPy forward, {dt:.1f} s, {cores} BLAS threads",
            "other_workloads_best_of_3": others}


def micro(args, cfg):
    """The gate_up GEMM alone (M = 16384 tokens of one packed call, N = 2 x 6144,
    K = 2048, SiLU*up epilogue), then a plain 1 GiB device copy whose bytes are known,
    for calibrating the HBM byte counters.  --micro-data zeros runs it on all-zero
    operands (same instructions and cycles, far less switching power, so the clock
    stays near its maximum); --micro gate_up_hipblaslt times the vendor library's GEMM
    (torch.matmul, plain bf16 output, not batch-invariant) on the same operands as a
    reference rate.  With many --steps the rate is the steady, power-limited one."""
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    from bitwise_consistent_rl_amd import engine
    M, N, K = args.max_tokens, 2 * cfg.intermediate, cfg.hidden
    mc = abi.ModelConfig()
    for k, v in dict(n_layers=1, hidden=K, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                     head_dim=cfg.head_dim, intermediate=cfg.intermediate, vocab=128,
                     rms_eps=1e-6, rope_theta=1e6, kv_block_tokens=64, max_tokens_per_call=64,
                     max_seqs_per_call=1, max_scored_per_call=1, max_position=64).items():
        setattr(mc, k, v)
    ctx = abi.bci_create(mc, 0)
    a, w = synth.gemm_inputs(M, N, K, index=90)
    a, w = a.cuda(), w.cuda()
    if args.micro_data == "zeros":
        a.zero_()
        w.zero_()
    c = torch.empty(M, N // 2, dtype=torch.bfloat16, device="cuda")
    if args.micro == "gate_up_hipblaslt":
        cf = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        run = lambda: torch.matmul(a, w.t(), out=cf)  # noqa: E731
    else:
        run = lambda: abi.bci_op_gemm_bf16(ctx, a, w, c, M, N, K, abi.BCI_EPI_SILU_MUL)  # noqa: E731
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")   # 1 GiB
    dst = torch.empty_like(src)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    flops = 2.0 * M * N * K
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    abi.bci_destroy(ctx)
    print(json.dumps({"micro": args.micro, "data": args.micro_data, "M": M, "N": N, "K": K,
                      "avg_ms": round(ms, 4),
                      "tflops": round(flops / ms / 1e9, 1),
                      "frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                      "algorithmic_bytes": (M * K + N * K + M * N // 2) * 2,
                      "copy_bytes": 2 * (1 << 30)}), flush=True)


def micro_attention(args, cfg):
    """The attention op alone on one packed recompute call: sequences of the seeded workload
    from position 0 up to --max-tokens tokens, the model's heads, bf16 KV cache written by
    the RoPE + KV-write op from N(0,1) q/k/v rows, 1024-key segments (every position in the
    first: the one-segment schedule).  Prints us per launch (HIP events, --steps launches)."""
    import numpy as np
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    mc = abi.ModelConfig()
    for k, v in dict(n_layers=1, hidden=cfg.hidden, n_q_heads=nq, n_kv_heads=nkv, head_dim=d,
                     intermediate=cfg.intermediate, vocab=128, rms_eps=1e-6, rope_theta=1e6,
                     kv_dtype=abi.BCI_KV_BF16, kv_block_tokens=64, attn_segment_keys=QWEN_SEG_KEYS,
                     max_tokens_per_call=args.max_tokens, max_seqs_per_call=64, max_scored_per_call=1,
                     max_position=1024, mode=abi.BCI_MODE_INVARIANT, attn_split_mode=0).items():
        setattr(mc, k, v)
    ctx = abi.bci_create(mc, 0)
    seqs = synth.rl_sequences(cfg, n_prompts=8, n_responses=8)
    lengths, tot = [], 0
    for sq in seqs:
        if tot + sq.length > args.max_tokens:
            break
        lengths.append(sq.length)
        tot += sq.length
    nb = sum((L + 63) // 64 for L in lengths)
    kc = torch.zeros((1, nb, nkv, 64, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    abi.bci_bind_kv_cache(ctx, kc, vc, None, None, nb)
    blocks, nxt = [], 0
    for L in lengths:
        blocks.append(list(range(nxt, nxt + (L + 63) // 64)))
        nxt += (L + 63) // 64
    maxb = max(len(b) for b in blocks)
    bt = np.array([b + [0] * (maxb - len(b)) for b in blocks], np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    abi.bci_set_batch(ctx, np.zeros(T, np.int32), cu, np.zeros(len(lengths), np.int32), bt, [], [])
    qkv = synth.normal_bf16((T, (nq + 2 * nkv) * d), index=44).cuda()
    q = torch.empty(T, nq * d, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    abi.bci_op_rope_kv_write(ctx, qkv, q, 0)
    for _ in range(3):
        abi.bci_op_attention(ctx, q, 0, o)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        abi.bci_op_attention(ctx, q, 0, o)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / args.steps
    abi.bci_destroy(ctx)
    print(json.dumps({"micro": "attention", "tokens": T, "sequences": len(lengths), "avg_us": round(us, 2)}),
          flush=True)


def decode_bench(args, cfg):
    """Decode steps alone, for a kernel trace: sequences of the Qwen3-shaped workload are
    prefilled to their response midpoint, then `--steps` decode steps (one new token and
    its logprob per sequence) run at B = 1 and B = 64, each timed with HIP events."""
    import numpy as np
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    from bitwise_consistent_rl_amd import engine
    weights = synth.make_weights(cfg)
    seqs = synth.rl_sequences(cfg, n_prompts=8, n_responses=8)
    m = engine.Model(cfg, weights, max_tokens=8192, max_seqs=128, max_scored=8192,
                     max_position=1024, seg_keys=QWEN_SEG_KEYS)
    cache = m.new_cache(64 * 11 + 16)
    m.bind_cache(cache)
    steps, graph_steps, graph_equal = {}, {}, {}
    for B in (1, 64):
        sub = seqs[:B]
        mids = [s.prompt_len + s.n_scored // 2 for s in sub]
        blocks = [list(range(i * 11, i * 11 + 11)) for i in range(B)]
        for g0 in range(0, B, 16):                       # prefill, <= 16 sequences per call
            g = range(g0, min(B, g0 + 16))
            engine.run_call(m, engine.CallPlan(
                np.concatenate([sub[i].tokens[:mids[i]] for i in g]).astype(np.int32),
                np.concatenate([[0], np.cumsum([mids[i] for i in g])]).astype(np.int32),
                np.zeros(len(g), np.int32), np.array([blocks[i] for i in g], np.int32),
                np.zeros(0, np.int32), np.zeros(0, np.int32), []))
        abi.bci_set_batch(m.ctx, np.array([s.tokens[mid] for s, mid in zip(sub, mids)], np.int32),
                          np.arange(B + 1, dtype=np.int32), np.array(mids, np.int32),
                          np.array(blocks, np.int32), np.arange(B, dtype=np.int32),
                          np.array([s.tokens[mid + 1] for s, mid in zip(sub, mids)], np.int32))
        out = torch.empty(B, dtype=torch.float32, device="cuda")
        for _ in range(3):
            abi.bci_forward_logprobs(m.ctx, out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            abi.bci_forward_logprobs(m.ctx, out)
        e1.record()
        torch.cuda.synchronize()
        steps[str(B)] = round(e0.elapsed_time(e1) / args.steps, 3)
        log(f"decode B = {B}: {steps[str(B)]} ms per step")
        # the same step replayed from a captured HIP graph (block table padded to the
        # context's width, as the graphed rollout pads it); the bits must not change
        width = -(-m.max_position // engine.KV_BLOCK)
        abi.bci_set_batch(m.ctx, np.array([s.tokens[mid] for s, mid in zip(sub, mids)], np.int32),
                          np.arange(B + 1, dtype=np.int32), np.array(mids, np.int32),
                          np.array([b + [0] * (width - len(b)) for b in blocks], np.int32),
                          np.arange(B, dtype=np.int32),
                          np.array([s.tokens[mid + 1] for s, mid in zip(sub, mids)], np.int32))
        gout = torch.empty(B, dtype=torch.float32, device="cuda")
        for _ in range(3):
            abi.bci_forward_logprobs_graph(m.ctx, gout)
        e0.record()
        for _ in range(args.steps):
            abi.bci_forward_logprobs_graph(m.ctx, gout)
        e1.record()
        torch.cuda.synchronize()
        graph_steps[str(B)] = round(e0.elapsed_time(e1) / args.steps, 3)
        graph_equal[str(B)] = bool(torch.equal(gout.view(torch.int32), out.view(torch.int32)))
        log(f"decode B = {B}, graph replay: {graph_steps[str(B)]} ms per step, "
            f"bitwise equal to eager: {graph_equal[str(B)]}")
    m.close()
    weight_bytes = sum(v.numel() for v in weights.values()) * 2
    print(json.dumps({"workload": "qwen3-1.7b-shaped decode steps", "decode_step_ms": steps,
                      "decode_step_ms_graph": graph_steps, "graph_step_bitwise_equal": graph_equal,
                      "steps": args.steps,
                      "weight_streaming_floor_ms": round(weight_bytes / (PEAK_HBM_GBS * 1e6), 3)}),
          flush=True)


def rollout_bench(args, cfg):
    """Rollout side of the Qwen3-shaped workload, invariant vs non-invariant mode.

    (1) Continuous batching of the first 128 sequences (16 prompts x 8 responses): each
    step runs every active sequence's prompt (once) or next response token, and takes
    the logprob of each response token as it is "sampled".  Wall-clock scored tokens/s,
    host scheduling included, the same for both modes.  (2) One decode step (one new
    token per sequence at its response midpoint) for B = 1, 16, 64, 128, timed with HIP
    events.  The non-invariant mode splits small-M GEMMs over K with atomics and sizes
    attention segments per call; its results are not batch-invariant."""
    import numpy as np
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    from bitwise_consistent_rl_amd import engine
    weights = synth.make_weights(cfg)
    seqs = synth.rl_sequences(cfg, n_prompts=16, n_responses=8)
    results = {}
    graph_steps, graph_equal, graph_rollout = {}, {}, {}
    for mode in ("invariant", "fast"):
        m = engine.Model(cfg, weights, max_tokens=8192, max_seqs=128, max_scored=8192,
                         max_position=1024, seg_keys=QWEN_SEG_KEYS, mode=mode)
        cache = m.new_cache(128 * 11 + 16)
        engine.rollout(m, seqs[:8], cache, cap=8)           # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lp = engine.rollout(m, seqs, cache, cap=128)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        scored = sum(len(x) for x in lp)
        steps = {}
        for B in (1, 16, 64, 128):
            sub = seqs[:B]
            m.bind_cache(cache)
            # prefill each sequence up to its response midpoint, then time one decode step
            mids = [s.prompt_len + s.n_scored // 2 for s in sub]
            blocks = [list(range(i * 11, i * 11 + 11)) for i in range(B)]
            for g0 in range(0, B, 16):                       # prefill, <= 16 sequences per call
                g = range(g0, min(B, g0 + 16))
                plan = engine.CallPlan(np.concatenate([sub[i].tokens[:mids[i]] for i in g]).astype(np.int32),
                                       np.concatenate([[0], np.cumsum([mids[i] for i in g])]).astype(np.int32),
                                       np.zeros(len(g), np.int32), np.array([blocks[i] for i in g], np.int32),
                                       np.zeros(0, np.int32), np.zeros(0, np.int32), [])
                engine.run_call(m, plan)
            dec = engine.CallPlan(np.array([s.tokens[mid] for s, mid in zip(sub, mids)], np.int32),
                                  np.arange(B + 1, dtype=np.int32), np.array(mids, np.int32),
                                  np.array(blocks, np.int32), np.arange(B, dtype=np.int32),
                                  np.array([s.tokens[mid + 1] for s, mid in zip(sub, mids)], np.int32), [])
            out = torch.empty(B, dtype=torch.float32, device="cuda")
            abi.bci_set_batch(m.ctx, dec.tokens, dec.cu_q, dec.pos0, dec.block_table, dec.score_rows,
                              dec.score_ids)
            for _ in range(3):
                abi.bci_forward_logprobs(m.ctx, out)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                abi.bci_forward_logprobs(m.ctx, out)
            e1.record()
            torch.cuda.synchronize()
            steps[B] = e0.elapsed_time(e1) / 10
            if mode == "invariant":
                # the same step replayed from a captured HIP graph (block table padded to
                # the context's width, as the graphed rollout does); bits must not change
                width = -(-m.max_position // engine.KV_BLOCK)
                gbt = np.array([b + [0] * (width - len(b)) for b in blocks], np.int32)
                abi.bci_set_batch(m.ctx, dec.tokens, dec.cu_q, dec.pos0, gbt, dec.score_rows,
                                  dec.score_ids)
                gout = torch.empty(B, dtype=torch.float32, device="cuda")
                for _ in range(3):
                    abi.bci_forward_logprobs_graph(m.ctx, gout)
                e0.record()
                for _ in range(10):
                    abi.bci_forward_logprobs_graph(m.ctx, gout)
                e1.record()
                torch.cuda.synchronize()
                graph_steps[B] = e0.elapsed_time(e1) / 10
                graph_equal[B] = bool(torch.equal(gout.view(torch.int32), out.view(torch.int32)))
        results[mode] = dict(lp=lp, tokens_per_s=scored / dt, seconds=dt, scored=scored, steps=steps)
        if mode == "invariant":
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            lp_g = engine.rollout(m, seqs, cache, cap=128, graph=True)
            torch.cuda.synchronize()
            graph_rollout = {"tokens_per_s": round(scored / (time.perf_counter() - t0), 1),
                             "bitwise_equal_to_eager": all(a.tobytes() == b.tobytes()
                                                           for a, b in zip(lp_g, lp))}
        m.close()
        del cache
        torch.cuda.empty_cache()
    inv, fast = results["invariant"], results["fast"]
    stats = engine.acceptance(fast["lp"], inv["lp"])
    weight_bytes = sum(v.numel() for v in weights.values()) * 2

    # (3) rollout throughput at each batch cap in both modes (the same host scheduler,
    # eager launches), and one invariant run with a random cap (1..256) per step; every
    # invariant run's logprobs must equal the recompute's bit for bit
    seqs_all = synth.rl_sequences(cfg, n_prompts=32, n_responses=8)
    cap_plan = ((1, 2), (8, 16), (32, 64), (128, 128), (256, 256))
    caps = {}
    for mode in ("fast", "invariant"):
        m = engine.Model(cfg, weights, max_tokens=8192, max_seqs=256, max_scored=8192,
                         max_position=1024, seg_keys=QWEN_SEG_KEYS, mode=mode)
        cache = m.new_cache(256 * 11 + 16)
        rec = engine.recompute(m, seqs_all, cache)
        engine.rollout(m, seqs_all[:8], cache, cap=8)           # warm-up
        for cap, n in cap_plan:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            lp = engine.rollout(m, seqs_all[:n], cache, cap=cap)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            row = caps.setdefault(str(cap), {"sequences": n})
            row[f"{mode}_tokens_per_s"] = round(sum(len(x) for x in lp) / dt, 1)
            if mode == "invariant":
                row["bitwise_equal_to_recompute"] = all(a.tobytes() == b.tobytes()
                                                        for a, b in zip(lp, rec[:n]))
                row["invariant_over_fast"] = round(row["invariant_tokens_per_s"] / row["fast_tokens_per_s"], 4)
            log(f"rollout cap {cap} ({mode}): {row}")
        if mode == "fast":
            m.close()
            del cache
            torch.cuda.empty_cache()
    rng = np.random.default_rng(9012)
    lp = engine.rollout(m, seqs_all, cache, cap=256,
                        cap_schedule=lambda step: int(rng.integers(1, 257)))
    random_cap_equal = all(a.tobytes() == b.tobytes() for a, b in zip(lp, rec))
    m.close()
    del cache
    torch.cuda.empty_cache()
    print(json.dumps({
        "workload": "qwen3-1.7b-shaped rollout, 16 prompts x 8 responses, continuous batching cap 128",
        "scored_tokens": inv["scored"],
        "invariant_tokens_per_s": round(inv["tokens_per_s"], 1),
        "fast_tokens_per_s": round(fast["tokens_per_s"], 1),
        "invariant_over_fast": round(inv["tokens_per_s"] / fast["tokens_per_s"], 4),
        "decode_step_ms": {"invariant": {str(b): round(v, 3) for b, v in inv["steps"].items()},
                           "fast": {str(b): round(v, 3) for b, v in fast["steps"].items()}},
        "decode_roofline_ms": round(weight_bytes / (PEAK_HBM_GBS * 1e6), 3),
        "decode_step_ms_graph": {str(b): round(v, 3) for b, v in graph_steps.items()},
        "graph_step_bitwise_equal": graph_equal,
        "graph_rollout_cap128": graph_rollout,
        "fast_vs_invariant_logprobs": stats,
        "rollout_by_cap": caps,
        "random_cap_bitwise_equal_to_recompute": random_cap_equal}), flush=True)


def longctx(args):
    """FP8-KV attention at 8K / 32K / 57K context (32 q / 4 kv heads of 128, e4m3 cache
    with per-token-per-head scales, KV segments of 1024 keys).  For each context: a
    decode step (one new query per sequence) at B = 1, 4, 16, 64 with the other
    sequences' lengths uniform in [C/2, C], and a chunked prefill (chunk 2048) of one
    sequence.  Decode is HBM-bound: 1056 B of K/V codes and scales per context token
    (2 x 4 heads x (128 + 4) B) plus 16 KiB of q and o per sequence."""
    import numpy as np
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    NQ, NKV, D, SEG = 32, 4, 128, 1024
    width = (NQ + 2 * NKV) * D
    rng = np.random.default_rng(5678)
    qkv = synth.normal_bf16((57344 + 64 * 131, width), index=60).cuda()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for C in (8192, 32768, 57344):
        lengths = [C] + [int(x) for x in rng.integers(C // 2, C + 1, size=63)]
        mc = abi.ModelConfig()
        for k, v in dict(n_layers=1, hidden=512, n_q_heads=NQ, n_kv_heads=NKV, head_dim=D,
                         intermediate=512, vocab=128, rms_eps=1e-6, rope_theta=1e6,
                         kv_dtype=abi.BCI_KV_FP8_E4M3, kv_block_tokens=64, attn_segment_keys=SEG,
                         max_tokens_per_call=8192, max_seqs_per_call=64, max_scored_per_call=1,
                         max_position=C + 64).items():
            setattr(mc, k, v)
        ctx = abi.bci_create(mc, 0)
        blocks, nxt = [], 0
        for L in lengths:
            blocks.append(list(range(nxt, nxt + (L + 63) // 64)))
            nxt += (L + 63) // 64
        shape = (1, nxt, NKV, 64, D)
        k = torch.empty(shape, dtype=torch.uint8, device="cuda")
        v = torch.empty_like(k)
        ks = torch.empty(shape[:-1], device="cuda")
        vs = torch.empty_like(ks)
        abi.bci_bind_kv_cache(ctx, k, v, ks, vs, nxt)
        maxb = max(len(b) for b in blocks)

        def batch(chunks):
            T = sum(n for _, _, n in chunks)
            cu = np.concatenate([[0], np.cumsum([n for _, _, n in chunks])]).astype(np.int32)
            bt = np.array([blocks[s] + [0] * (maxb - len(blocks[s])) for s, _, _ in chunks], np.int32)
            abi.bci_set_batch(ctx, np.zeros(T, np.int32), cu,
                              np.array([p for _, p, _ in chunks], np.int32), bt, [], [])
        # fill every sequence's cache (positions 0 .. L-2) through the FP8 writer
        qbuf = torch.empty(8192, NQ * D, dtype=torch.bfloat16, device="cuda")
        for sq, L in enumerate(lengths):
            for s0 in range(0, L - 1, 8192):
                n = min(8192, L - 1 - s0)
                batch([(sq, s0, n)])
                abi.bci_op_rope_kv_write(ctx, qkv[sq * 131 + s0: sq * 131 + s0 + n].contiguous(), qbuf, 0)
        torch.cuda.synchronize()
        log(f"context {C}: caches filled")
        for B in (1, 4, 16, 64):
            seqs = list(range(B))
            rows = torch.cat([qkv[s * 131 + lengths[s] - 1: s * 131 + lengths[s]] for s in seqs]).contiguous()
            q = torch.empty(B, NQ * D, dtype=torch.bfloat16, device="cuda")
            o = torch.empty_like(q)
            batch([(s, lengths[s] - 1, 1) for s in seqs])
            abi.bci_op_rope_kv_write(ctx, rows, q, 0)
            for _ in range(3):
                abi.bci_op_attention(ctx, q, 0, o)
            e0, e1 = ev(), ev()
            reps = 20
            e0.record()
            for _ in range(reps):
                abi.bci_op_attention(ctx, q, 0, o)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            ctx_tokens = sum(lengths[s] for s in seqs)
            nbytes = ctx_tokens * 1056 + B * 16384
            print(json.dumps({"workload": "fp8-kv long-context decode step", "context": C, "batch": B,
                              "context_tokens": ctx_tokens, "us_per_step": round(us, 2),
                              "tokens_per_s": round(B / us * 1e6, 1),
                              "roofline": {"bound": "hbm", "achieved": round(nbytes / us / 1e3, 1),
                                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                           "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}}),
                  flush=True)
        # chunked prefill of sequence 0 (chunk 2048), attention included
        q = torch.empty(2048, NQ * D, dtype=torch.bfloat16, device="cuda")
        o = torch.empty_like(q)
        e0, e1 = ev(), ev()
        e0.record()
        for s0 in range(0, C, 2048):
            batch([(0, s0, 2048)])
            abi.bci_op_rope_kv_write(ctx, qkv[s0: s0 + 2048].contiguous(), q, 0)
            abi.bci_op_attention(ctx, q, 0, o)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        flops = 4.0 * NQ * D * C * (C + 1) / 2
        print(json.dumps({"workload": "fp8-kv chunked prefill (2048)", "context": C, "ms": round(ms, 2),
                          "roofline": {"bound": "mfma", "achieved": round(flops / ms / 1e9, 1),
                                       "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}}), flush=True)
        abi.bci_destroy(ctx)
        del k, v, ks, vs


def sparse_bench(args):
    """Sparse attention over a Top-K selected set on the FP8 path (32 q / 4 kv heads of
    128, e4m3 cache; indexer of 64 heads x 128 with an e4m3 index cache; K = 2048).
    Decode steps at B = 1, 16, 64 with sequence 0 at 57344 tokens and the others uniform
    in [8192, 57344]; each kernel of the step timed alone with HIP events on the launch
    stream.  Then a chunked prefill (chunk 2048) of the last 2048 positions of a 32768-token
    sequence.  Algorithmic bytes / flops per unit:
      index scores   per (query, key): 132 B of index-key codes + scale read (decode: every
                     query has its own sequence; prefill: the chunk's queries share the
                     keys, read once), 4 B score written; 2 x 64 x 128 = 16384 flop
      top-K          per (query, key): 4 B score read; per query 4 x 2048 B written
      sparse attn    per (query, selected key): 4 kv heads x 2 x (128 + 4) B of K/V codes
                     and scales; 4 x 32 x 128 = 16384 flop; per query 16 KiB of q and o."""
    import numpy as np
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    NQ, NKV, D, HI, DI, K = 32, 4, 128, 64, 128, 2048
    width = (NQ + 2 * NKV) * D
    C = 57344
    rng = np.random.default_rng(5678)
    lengths = [C] + [int(x) for x in rng.integers(8192, C + 1, size=63)]
    n_rows = 63 * 131 + C + 64
    qkv = synth.normal_bf16((n_rows, width), index=60).cuda()
    _, _, kidx = synth.sparse_index_inputs(0, n_rows, HI, DI, exact=False, index=61)
    kidx = kidx.cuda()
    qi_all, w_all, _ = synth.sparse_index_inputs(2048, 0, HI, DI, exact=False, index=62)
    qi_all, w_all = qi_all.cuda(), torch.from_numpy(w_all).cuda()
    mc = abi.ModelConfig()
    for k, v in dict(n_layers=1, hidden=512, n_q_heads=NQ, n_kv_heads=NKV, head_dim=D,
                     intermediate=512, vocab=128, rms_eps=1e-6, rope_theta=1e6,
                     kv_dtype=abi.BCI_KV_FP8_E4M3, kv_block_tokens=64, attn_segment_keys=1024,
                     max_tokens_per_call=8192, max_seqs_per_call=64, max_scored_per_call=1,
                     max_position=C + 64).items():
        setattr(mc, k, v)
    ctx = abi.bci_create(mc, 0)
    blocks, nxt = [], 0
    for L in lengths:
        blocks.append(list(range(nxt, nxt + (L + 63) // 64)))
        nxt += (L + 63) // 64
    shape = (1, nxt, NKV, 64, D)
    kc = torch.empty(shape, dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    ks = torch.empty(shape[:-1], device="cuda")
    vs = torch.empty_like(ks)
    ic = torch.empty(nxt, 64, DI, dtype=torch.uint8, device="cuda")
    isc = torch.empty(nxt, 64, device="cuda")
    abi.bci_bind_kv_cache(ctx, kc, vc, ks, vs, nxt)
    maxb = max(len(b) for b in blocks)
    stride = C + 64

    def batch(chunks):
        T = sum(n for _, _, n in chunks)
        cu = np.concatenate([[0], np.cumsum([n for _, _, n in chunks])]).astype(np.int32)
        bt = np.array([blocks[s] + [0] * (maxb - len(blocks[s])) for s, _, _ in chunks], np.int32)
        abi.bci_set_batch(ctx, np.zeros(T, np.int32), cu,
                          np.array([p for _, p, _ in chunks], np.int32), bt, [], [])

    qbuf = torch.empty(8192, NQ * D, dtype=torch.bfloat16, device="cuda")
    for sq, L in enumerate(lengths):
        for s0 in range(0, L - 1, 8192):
            n = min(8192, L - 1 - s0)
            batch([(sq, s0, n)])
            r = slice(sq * 131 + s0, sq * 131 + s0 + n)
            abi.bci_op_rope_kv_write(ctx, qkv[r].contiguous(), qbuf, 0)
            abi.bci_op_index_key_write(ctx, kidx[r].contiguous(), DI, ic, isc, nxt)
    torch.cuda.synchronize()
    log("sparse: caches filled")
    scores = torch.empty(2048, stride, device="cuda")
    sel = torch.empty(2048, K, dtype=torch.int32, device="cuda")
    q = torch.empty(2048, NQ * D, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)

    def report(name, B, keys, us, flops, nbytes, extra=None):
        t_f, t_b = flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
        bound = "mfma" if t_f > t_b else "hbm"
        rec = {"workload": "sparse attention, FP8 KV, K = 2048", "kernel": name, "batch": B,
               "keys_scored": keys, "us": round(us, 2), "bound": bound,
               "achieved": round(flops / us / 1e6, 1) if bound == "mfma" else round(nbytes / us / 1e3, 1),
               "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
               "frac_of_roofline": round(max(t_f, t_b) / (us * 1e-6), 4)}
        rec.update(extra or {})
        print(json.dumps(rec), flush=True)

    for B in (1, 16, 64):
        seqs = list(range(B))
        chunks = [(s, lengths[s] - 1, 1) for s in seqs]
        batch(chunks)
        rows = torch.cat([qkv[s * 131 + lengths[s] - 1: s * 131 + lengths[s]] for s in seqs]).contiguous()
        krows = torch.cat([kidx[s * 131 + lengths[s] - 1: s * 131 + lengths[s]] for s in seqs]).contiguous()
        qi, wi = qi_all[:B].contiguous(), w_all[:B].contiguous()
        qB, oB, sB, selB = q[:B], o[:B], scores[:B], sel[:B]
        keys = sum(lengths[s] for s in seqs)
        t_rope = _time_ms(lambda: abi.bci_op_rope_kv_write(ctx, rows, qB, 0), reps=20) * 1e3
        t_ikw = _time_ms(lambda: abi.bci_op_index_key_write(ctx, krows, DI, ic, isc, nxt), reps=20) * 1e3
        t_sc = _time_ms(lambda: abi.bci_op_index_scores(ctx, qi, wi, HI, DI, ic, isc, nxt, sB, stride),
                        reps=20) * 1e3
        t_tk = _time_ms(lambda: abi.bci_op_sparse_topk(ctx, sB, stride, K, selB), reps=20) * 1e3
        t_at = _time_ms(lambda: abi.bci_op_sparse_attention(ctx, qB, 0, selB, K, oB), reps=20) * 1e3
        report("index_scores", B, keys, t_sc, 16384.0 * keys, 136.0 * keys + B * (HI * DI * 2 + HI * 4))
        report("sparse_topk", B, keys, t_tk, 0.0, 4.0 * keys + 4.0 * K * B)
        report("sparse_attention", B, keys, t_at, 16384.0 * K * B, NKV * 2 * (D + 4) * K * B + 16384.0 * B)
        step = t_rope + t_ikw + t_sc + t_tk + t_at
        print(json.dumps({"workload": "sparse attention decode step, FP8 KV, K = 2048", "batch": B,
                          "context_tokens": keys, "us_per_step": round(step, 2),
                          "us": {"rope_kv_write": round(t_rope, 2), "index_key_write": round(t_ikw, 2),
                                 "index_scores": round(t_sc, 2), "sparse_topk": round(t_tk, 2),
                                 "sparse_attention": round(t_at, 2)},
                          "tokens_per_s": round(B / step * 1e6, 1)}), flush=True)

    # chunked prefill: the last 2048 positions of a 32768-token context (sequence 1 of the
    # fill is at least 8192 long; use sequence 0's cache, positions 30720 .. 32767)
    P0, n = 32768 - 2048, 2048
    batch([(0, P0, n)])
    qi, wi = qi_all[:n].contiguous(), w_all[:n].contiguous()
    r = slice(P0, P0 + n)
    abi.bci_op_rope_kv_write(ctx, qkv[r].contiguous(), q, 0)
    keys = sum(P0 + i + 1 for i in range(n))
    t_sc = _time_ms(lambda: abi.bci_op_index_scores(ctx, qi, wi, HI, DI, ic, isc, nxt, scores, stride),
                    reps=3, warm=1) * 1e3
    t_tk = _time_ms(lambda: abi.bci_op_sparse_topk(ctx, scores, stride, K, sel), reps=3, warm=1) * 1e3
    t_at = _time_ms(lambda: abi.bci_op_sparse_attention(ctx, q, 0, sel, K, o), reps=3, warm=1) * 1e3
    # the chunk's queries share one sequence's index keys: read once, scores written per query
    report("index_scores", n, keys, t_sc, 16384.0 * keys,
           132.0 * (P0 + n) + 4.0 * keys + n * (HI * DI * 2 + HI * 4), {"phase": "chunked prefill"})
    report("sparse_topk", n, keys, t_tk, 0.0, 4.0 * keys + 4.0 * K * n, {"phase": "chunked prefill"})
    report("sparse_attention", n, keys, t_at, 16384.0 * K * n, NKV * 2 * (D + 4) * K * n + 16384.0 * n,
           {"phase": "chunked prefill"})
    abi.bci_destroy(ctx)


def ssd_bench(args):
    """Chunked state-space layer (Mamba-2-style; 128 heads x 64, 8 groups, state 128, chunks
    of 64): a prefill call of 4 sequences x 4096 positions, and decode steps at B = 1, 16,
    64 with every sequence 1000 positions in (the state, and a partly filled chunk, read
    back).  Algorithmic work per (token, head): 2 x 64 x 128 (inter) + 2 x 64 x 128 (the
    scores against the chunk) + 2 x 64 x 64 (their product with x) + 2 x 64 x 128 (the
    chunk state, per position) = 57344 FLOP; bytes per token: x 16 KiB + B and C 4 KiB + dt
    512 B read, y 16 KiB written; decode also reads each (sequence, head) state once
    (32 KiB fp32)."""
    import numpy as np
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    H, G, N, P = 128, 8, 128, 64
    cfg = abi.SsdConfig()
    for k, v in dict(n_heads=H, head_dim=P, d_state=N, n_groups=G, max_tokens_per_call=16384,
                     max_seqs_per_call=64).items():
        setattr(cfg, k, v)
    ctx = abi.bci_ssd_create(cfg, 0)
    n_slots = 64
    state = torch.zeros(n_slots, H, P, N, device="cuda")
    cbuf = torch.zeros(abi.bci_ssd_slot_bytes(ctx, 1) * n_slots, dtype=torch.uint8, device="cuda")
    d = synth.ssd_inputs(16384, H, P, N, G, index=30)
    x, B, C = d["x"].cuda(), d["B"].cuda(), d["C"].cuda()
    dt = torch.from_numpy(d["dt"]).cuda()
    A, D = torch.from_numpy(d["A"]).cuda(), torch.from_numpy(d["D"]).cuda()
    y = torch.empty_like(x)
    flop_tok, byte_tok = 57344.0 * H, 16384 + 4096 + 512 + 16384

    def report(name, T, us, extra_bytes=0.0):
        flops, nbytes = flop_tok * T, byte_tok * T + extra_bytes
        t_f, t_b = flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
        bound = "mfma" if t_f > t_b else "hbm"
        print(json.dumps({"workload": "state-space layer, 128 heads x 64, state 128, chunk 64",
                          "phase": name, "tokens": T, "us": round(us, 2),
                          "tokens_per_s": round(T / us * 1e6, 1), "bound": bound,
                          "achieved": round(flops / us / 1e6, 1) if bound == "mfma"
                          else round(nbytes / us / 1e3, 1),
                          "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                          "frac_of_roofline": round(max(t_f, t_b) / (us * 1e-6), 4)}), flush=True)

    # prefill: 4 sequences x 4096 positions in one call (slots 0..3)
    cu = np.arange(0, 16385, 4096, dtype=np.int32)

    def prefill():
        abi.bci_ssd_set_batch(ctx, cu, [0, 0, 0, 0], [0, 1, 2, 3])
        abi.bci_ssd_forward(ctx, x, dt, A, B, C, D, state, cbuf, n_slots, y)
    report("prefill 4 x 4096", 16384, _time_ms(prefill, reps=5, warm=2) * 1e3)
    # decode: every slot holds 1000 positions (prefilled in calls of 16 sequences)
    for s0 in range(0, 64, 16):
        abi.bci_ssd_set_batch(ctx, np.arange(0, 16 * 1000 + 1, 1000, dtype=np.int32), [0] * 16,
                              list(range(s0, s0 + 16)))
        abi.bci_ssd_forward(ctx, x, dt, A, B, C, D, state, cbuf, n_slots, y)
    torch.cuda.synchronize()
    for Bn in (1, 16, 64):
        cud = np.arange(Bn + 1, dtype=np.int32)
        xs, dts, Bs, Cs = x[:Bn].contiguous(), dt[:Bn].contiguous(), B[:Bn].contiguous(), C[:Bn].contiguous()
        ys = y[:Bn]

        def step():
            # position 1000 again each time: the same work per step (the chunk is not
            # completed, so the slots' states are not changed)
            abi.bci_ssd_set_batch(ctx, cud, [1000] * Bn, list(range(Bn)))
            abi.bci_ssd_forward(ctx, xs, dts, A, Bs, Cs, D, state, cbuf, n_slots, ys)
        report(f"decode B = {Bn}", Bn, _time_ms(step, reps=20) * 1e3, extra_bytes=Bn * H * P * N * 4.0)
    abi.bci_ssd_destroy(ctx)


def backward_bench(args):
    """Backward pieces at the Qwen3-shaped widths: the SiLU-gated MLP (H 2048, I 6144) over
    4096 tokens, add+RMSNorm over 4096 x 2048, and the lm_head logprob (V 151936) over 512
    scored rows.  Algorithmic work: MLP 3 x 2 x (2 x M x H x 2I ... ) -- the forward
    recompute of gate/up and the activation (2 GEMMs) plus four gradient GEMMs:
    2 M H 2I (gu) + 2 M H 2I (act) + 2 M I H x 2 (dact, dwd) + 2 M 2I H x 2 (dh, dwgu);
    lm_head: 2 M V H x 3 (z, dhf, dE); RMSNorm: 10 B per element (r, dh, dr_in read, dr
    written, r and dh read again for dg)."""
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    from bitwise_consistent_rl_amd import backward as bw
    H, I, V = 2048, 6144, 151936
    mc = abi.ModelConfig()
    for k, v in dict(n_layers=1, hidden=H, n_q_heads=16, n_kv_heads=8, head_dim=128, intermediate=I,
                     vocab=V, rms_eps=1e-6, rope_theta=1e6, kv_block_tokens=64, attn_segment_keys=2048,
                     max_tokens_per_call=4096, max_seqs_per_call=1, max_scored_per_call=512,
                     max_position=64).items():
        setattr(mc, k, v)
    ctx = abi.bci_create(mc, 0)

    def report(name, ms, flops=0.0, nbytes=0.0):
        t_f, t_b = flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
        bound = "mfma" if t_f > t_b else "hbm"
        print(json.dumps({"workload": "backward pieces (Qwen3-shaped widths)", "op": name,
                          "ms": round(ms, 3), "bound": bound,
                          "achieved": round(flops / ms / 1e9, 1) if bound == "mfma"
                          else round(nbytes / ms / 1e6, 1),
                          "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                          "frac_of_roofline": round(max(t_f, t_b) / (ms * 1e-3), 4)}), flush=True)

    M = 4096
    h = synth.normal_bf16((M, H), index=66).cuda()
    wgu = synth.normal_bf16((2 * I, H), index=67, scale=0.02).cuda()
    wd = synth.normal_bf16((H, I), index=68, scale=0.02).cuda()
    dout = synth.normal_bf16((M, H), index=69).cuda()
    ms = _time_ms(lambda: bw.mlp_backward(ctx, h, wgu, wd, dout, I), reps=5, warm=2)
    report("SiLU-MLP backward, 4096 tokens", ms, flops=2.0 * M * H * 2 * I * 2 + 2.0 * M * I * H * 2
           + 2.0 * M * 2 * I * H * 2)
    g = (synth.normal_bf16((H,), index=61, scale=0.1).float() + 1.0).to(torch.bfloat16).cuda()
    ms = _time_ms(lambda: bw.add_rmsnorm_backward(ctx, h, g, dout, 1e-6, dout), reps=10)
    report("add+RMSNorm backward, 4096 x 2048", ms, nbytes=10.0 * M * H)
    Ms = 512
    hs, w, ids = synth.lmhead_inputs(Ms, hidden=H, vocab=V)
    hf, emb = hs.cuda(), w.cuda()
    gids = torch.from_numpy(ids.astype("int32")).cuda()
    gg = torch.ones(Ms, device="cuda")
    embT = bw.transpose(ctx, emb, ld=V)
    ms = _time_ms(lambda: bw.logprob_backward(ctx, hf, emb, gids, gg, embT=embT), reps=3, warm=1)
    report("lm_head logprob backward, 512 rows", ms, flops=2.0 * Ms * V * H * 3)
    # attention backward, one 4096-token sequence, 16 q / 8 kv heads of 128: five products
    # of the causal half (S, dP, dV, dQ, dK) = 5 x 2 x nq x d x L^2 / 2 FLOP
    L, NQ, NKV, D = 4096, 16, 8, 128
    q = synth.normal_bf16((L, NQ * D), index=72).cuda()
    kk = synth.normal_bf16((L, NKV * D), index=73).cuda()
    vv = synth.normal_bf16((L, NKV * D), index=74).cuda()
    o = synth.normal_bf16((L, NQ * D), index=75).cuda()
    do = synth.normal_bf16((L, NQ * D), index=76).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(kk), torch.empty_like(vv)
    ws = torch.empty(2 * 4 * kk.numel(), dtype=torch.float32, device="cuda")   # row parts of dK/dV
    ms = _time_ms(lambda: abi.bci_op_attention_backward(ctx, q, kk, vv, o, do, L, dq, dk, dv, ws), reps=5)
    report("attention backward, 4096 tokens, 16/8 heads of 128", ms, flops=5.0 * NQ * D * L * L)
    abi.bci_destroy(ctx)


def _time_ms(fn, reps=10, warm=3):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def lmhead_bench(args):
    """lm_head + log-softmax + gather alone (config 3): hidden [M, 2048] N(0,1), W
    [151936, 2048] N(0,0.02), ids uniform; M in {1, 7, 64, 512, 4096, 8192}.  Roofline
    time max(622.33 MFLOP x M / 2.5 PF/s, (622.33 MB + 4104 B x M) / 8 TB/s)."""
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    H, V = 2048, 151936
    mc = abi.ModelConfig()
    for k, v in dict(n_layers=1, hidden=H, n_q_heads=16, n_kv_heads=8, head_dim=128,
                     intermediate=6144, vocab=V, rms_eps=1e-6, rope_theta=1e6, kv_block_tokens=64,
                     attn_segment_keys=2048, max_tokens_per_call=8192, max_seqs_per_call=1,
                     max_scored_per_call=8192, max_position=64).items():
        setattr(mc, k, v)
    ctx = abi.bci_create(mc, 0)
    hs, w, ids = synth.lmhead_inputs(8192)
    ghs, gw = hs.cuda(), w.cuda()
    gids = torch.from_numpy(ids).cuda()
    lp = torch.empty(8192, dtype=torch.float32, device="cuda")
    for M in (1, 7, 64, 512, 4096, 8192):
        a = ghs[:M].contiguous()
        ms = _time_ms(lambda: abi.bci_op_lmhead_logprob(ctx, a, gw, gids, M, H, V, lp))
        flops, nbytes = 622.33e6 * M, 622.33e6 + 4104.0 * M
        t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
        bound = "mfma" if flops / (PEAK_BF16_TFLOPS * 1e12) > nbytes / (PEAK_HBM_GBS * 1e9) else "hbm"
        print(json.dumps({"workload": "lm_head + log-softmax + gather (config 3)", "M": M,
                          "us": round(ms * 1e3, 2), "bound": bound,
                          "achieved": round(flops / ms / 1e9, 1) if bound == "mfma"
                          else round(nbytes / ms / 1e6, 1),
                          "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                          "frac_of_roofline": round(t_roof / (ms * 1e-3), 4)}), flush=True)
    abi.bci_destroy(ctx)


def moe_bench(args):
    """MoE layer alone (config 4): router GEMM (fp32 logits), top-6 with lowest-index
    ties, stable permutation, grouped expert GEMMs + shared expert, FP32 slot-order
    combine; h [T, 4096] N(0,1), T in {1, 64, 512, 2048, 8192}.  Roofline time
    max(264.77 MFLOP x T / 2.5 PF/s, ((distinct experts + 1) x 37.75 MB + 16.4 KB x T)
    / 8 TB/s)."""
    import numpy as np
    import torch
    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    cfg = synth.MOE
    H, E = cfg.hidden, cfg.n_experts
    mc = abi.ModelConfig()
    for k, v in dict(n_layers=1, hidden=H, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     intermediate=cfg.expert_intermediate, vocab=128, rms_eps=1e-6, rope_theta=1e6,
                     kv_block_tokens=64, attn_segment_keys=2048, max_tokens_per_call=8192,
                     max_seqs_per_call=8, max_scored_per_call=8, max_position=64,
                     n_experts=E, top_k=cfg.top_k, expert_intermediate=cfg.expert_intermediate,
                     n_shared_experts=1).items():
        setattr(mc, k, v)
    ctx = abi.bci_create(mc, 0)
    log("generating MoE weights")
    g = {k: v.cuda() for k, v in synth.moe_weights(cfg).items()}
    h_all = synth.normal_bf16((8192, H), index=50).cuda()
    z = torch.empty(8192, E, dtype=torch.float32, device="cuda")
    ids = torch.empty(8192, cfg.top_k, dtype=torch.int32, device="cuda")
    wt = torch.empty(8192, cfg.top_k, dtype=torch.float32, device="cuda")
    out = torch.empty(8192, H, dtype=torch.bfloat16, device="cuda")
    expert_bytes = (2 * cfg.expert_intermediate * H + H * cfg.expert_intermediate) * 2
    for T in (1, 64, 512, 2048, 8192):
        h = h_all[:T].contiguous()

        def step():
            abi.bci_op_gemm_bf16(ctx, h, g["wr"], z, T, E, H, abi.BCI_EPI_F32)
            abi.bci_op_moe_topk(ctx, z, T, ids, wt)
            abi.bci_op_moe_forward(ctx, h, ids, wt, T, g["wgu"], g["wd"], g["swgu"], g["swd"], out)
        ms = _time_ms(step)
        touched = len(np.unique(ids[:T].cpu().numpy()))
        flops = 264.77e6 * T
        nbytes = (touched + 1) * expert_bytes + 16.4e3 * T
        t_f, t_b = flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
        bound = "mfma" if t_f > t_b else "hbm"
        print(json.dumps({"workload": "MoE layer (config 4)", "T": T, "experts_touched": touched,
                          "us": round(ms * 1e3, 2), "bound": bound,
                          "achieved": round(flops / ms / 1e9, 1) if bound == "mfma"
                          else round(nbytes / ms / 1e6, 1),
                          "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                          "frac_of_roofline": round(max(t_f, t_b) / (ms * 1e-3), 4)}), flush=True)
    abi.bci_destroy(ctx)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--prompts", type=int, default=128)
    ap.add_argument("--responses", type=int, default=8)
    ap.add_argument("--max-tokens", type=int, default=16384)
    ap.add_argument("--accept-seqs", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fast", action="store_true",
                    help="skip timing the non-invariant mode on the recompute's calls")
    ap.add_argument("--mode", choices=["invariant", "fast"], default="invariant",
                    help="the recompute's timed pass in the invariant (default) or the "
                         "non-invariant mode (for profiling the latter alone)")
    ap.add_argument("--micro", choices=["gate_up", "gate_up_hipblaslt", "attention"], default=None,
                    help="time one kernel alone at the workload's shape (for counter runs)")
    ap.add_argument("--micro-data", choices=["random", "zeros"], default="random")
    ap.add_argument("--workload", choices=["recompute", "longctx", "rollout", "decode", "lmhead", "moe",
                                           "sparse", "ssd", "backward"],
                    default="recompute",
                    help="longctx: FP8-KV long-context attention (decode steps, chunked prefill); "
                         "rollout: continuous-batching decode, invariant vs non-invariant mode; "
                         "lmhead: the lm_head log-softmax alone at M = 1 .. 8192; "
                         "moe: the MoE layer alone at T = 1 .. 8192")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every sequence is independent, so N GPUs would "
              "each run their own share with no exchange; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from bitwise_consistent_rl_amd import _abi as abi
    from bitwise_consistent_rl_amd import engine

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = synth.QWEN3_1P7B
    if args.micro == "attention":
        return micro_attention(args, cfg)
    if args.micro:
        return micro(args, cfg)
    if args.workload == "longctx":
        return longctx(args)
    if args.workload == "rollout":
        return rollout_bench(args, cfg)
    if args.workload == "decode":
        return decode_bench(args, cfg)
    if args.workload == "lmhead":
        return lmhead_bench(args)
    if args.workload == "sparse":
        return sparse_bench(args)
    if args.workload == "ssd":
        return ssd_bench(args)
    if args.workload == "backward":
        return backward_bench(args)
    if args.workload == "moe":
        return moe_bench(args)
    log("generating weights and workload")
    weights = synth.make_weights(cfg)
    seqs = synth.rl_sequences(cfg, n_prompts=args.prompts, n_responses=args.responses)
    scored = sum(s.n_scored for s in seqs)
    processed = sum(s.length - 1 for s in seqs)
    n_blocks = args.max_tokens // 64 + 64
    model = engine.Model(cfg, weights, kv_dtype="bf16", max_tokens=args.max_tokens, max_seqs=64,
                         max_scored=args.max_tokens, max_position=1024, seg_keys=QWEN_SEG_KEYS,
                         mode=args.mode)
    cache = model.new_cache(n_blocks)
    model.bind_cache(cache)
    calls = engine.plan_recompute(seqs, range(len(seqs)), args.max_tokens, 64, args.max_tokens,
                                  n_blocks)
    lp_all = torch.empty(scored, dtype=torch.float32, device="cuda")
    offs = np.cumsum([0] + [len(p.score_rows) for p, _ in calls])
    stream = torch.cuda.current_stream()
    log(f"{len(seqs)} sequences, {processed} processed / {scored} scored tokens, {len(calls)} calls")

    def step(m=None):
        ctx = (m or model).ctx
        for (plan, _), o in zip(calls, offs[:-1]):
            abi.bci_set_batch(ctx, plan.tokens, plan.cu_q, plan.pos0, plan.block_table,
                              plan.score_rows, plan.score_ids, stream)
            abi.bci_forward_logprobs(ctx, lp_all[o:o + len(plan.score_rows)], stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    first = lp_all.clone()
    torch.cuda.synchronize()
    # one event pair per gate_up launch of the timed region: calls x layers x steps
    expect_launches = len(calls) * cfg.n_layers * args.steps
    abi.bci_profile_begin(model.ctx, expect_launches)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gu_ms, gu_launches, gu_rows, gu_dropped = abi.bci_profile_end(model.ctx)
    log(f"timed {args.steps} steps: {dt:.3f} s")
    if args.mode == "invariant":
        assert torch.equal(first.view(torch.int32), lp_all.view(torch.int32)), "run-to-run bits differ"
    assert gu_launches == expect_launches and gu_dropped == 0, (gu_launches, gu_dropped, expect_launches)
    assert gu_rows == args.steps * cfg.n_layers * sum(len(p.tokens) for p, _ in calls), gu_rows

    # gate_up GEMM: 2 * M * (2 I) * H flops per launch, M = tokens of the call; counted
    # over exactly the launches whose events were timed
    gu_flops = 2.0 * gu_rows * 2 * cfg.intermediate * cfg.hidden
    achieved = gu_flops / (gu_ms * 1e-3) / 1e12 if gu_ms > 0 else 0.0
    ms_per_step = dt * 1e3 / args.steps

    # whole-step algorithmic work: the projections' flops per processed token, causal
    # attention's 4 d n_q flops per (query, key <= query) pair, the lm_head per scored row
    lin = 2.0 * cfg.n_layers * cfg.hidden * (cfg.qkv_rows + cfg.hidden + 2 * cfg.intermediate
                                             + cfg.intermediate)
    attn = sum(2.0 * 2 * cfg.n_layers * cfg.n_q_heads * cfg.head_dim * (t + 1)
               for s in seqs for t in range(s.length - 1))
    head = 2.0 * cfg.hidden * cfg.vocab * scored
    step_flops = lin * processed + attn + head

    # acceptance on a bounded subset: rollout (continuous batching, decode) vs recompute
    sub = seqs[: args.accept_seqs]
    log(f"acceptance: rollout of {len(sub)} sequences vs recompute")
    roll_cache = model.new_cache(len(sub) * 11 + 8)
    roll = engine.rollout(model, sub, roll_cache, cap=min(64, len(sub)), prefill_chunk=None)
    rec = engine.recompute(model, sub, cache)
    acc = engine.acceptance(rec, roll)
    lp_host = first.cpu().numpy()
    # the timed step's rows for these sequences equal the standalone recompute
    if rec:
        acc["bench_rows_equal"] = bool(np.concatenate(rec).tobytes()
                                       == lp_host[: sum(len(r) for r in rec)].tobytes())
    del roll_cache

    # the non-invariant mode (per-call attention segments, split-K for 129..256-row GEMMs)
    # on the same calls with the same harness: the overhead the invariance costs here
    fast = None
    if args.steps > 0 and not args.no_fast and args.mode == "invariant":
        log("non-invariant mode on the same calls")
        fm = engine.Model(cfg, weights, kv_dtype="bf16", max_tokens=args.max_tokens, max_seqs=64,
                          max_scored=args.max_tokens, max_position=1024, seg_keys=QWEN_SEG_KEYS,
                          mode="fast")
        fcache = fm.new_cache(n_blocks)
        fm.bind_cache(fcache)
        step(fm)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(fm)
        torch.cuda.synchronize()
        fdt = time.perf_counter() - t0
        fm.close()
        del fcache
        torch.cuda.empty_cache()
        fast_value = scored / (fdt / args.steps)
        fast = {"value": round(fast_value, 1), "unit": "scored tokens/s",
                "ms_per_step": round(fdt * 1e3 / args.steps, 3),
                "invariant_over_fast": round(scored / (dt / args.steps) / fast_value, 4)}

    tr = gate_up_traffic()
    traffic = tr["bytes_per_launch"] if tr else None
    # the chip's sustained MFMA rate on random operands (power-limited clock), measured here
    log("measuring the sustained MFMA rate")
    sustained = abi.bci_measure_mfma_rate(0, True)
    out = {
        "metric": "invariant logprob-recompute tokens/sec @1 GPU, % roofline; diff/k3-KL must be 0",
        "value": round(scored / (dt / args.steps), 1),
        "unit": "scored tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-1.7b-shaped logprob recompute, 128 prompts x 8 responses",
                   "sequences": len(seqs), "processed_tokens": processed, "scored_tokens": scored,
                   "max_tokens_per_call": args.max_tokens, "calls_per_step": len(calls),
                   "kv_cache": "bf16", "mode": args.mode},
        "roofline": {"bound": "mfma", "kernel": "gate_up GEMM (SiLU*up epilogue)",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch at M = 16384 (rocprofv3 FETCH_SIZE + "
                                     "WRITE_SIZE, copy-calibrated)",
                     "launches": gu_launches, "avg_launch_us": round(gu_ms * 1e3 / max(gu_launches, 1), 2),
                     "sustained_peak": round(sustained, 1),
                     "frac_of_sustained": round(achieved / sustained, 4) if sustained > 0 else None,
                     "sustained_peak_note": "measured dense bf16 MFMA issue on pseudo-random register "
                                            "operands, all SIMDs, two waves each (bci_measure_mfma_rate)"},
        "step_roofline": {"algorithmic_tflop_per_step": round(step_flops / 1e12, 3),
                          "achieved_tflops": round(step_flops / (dt / args.steps) / 1e12, 1),
                          "frac_of_mfma_peak": round(step_flops / (dt / args.steps) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "acceptance": acc,
        "fast_mode": fast,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, weights, seqs)
    model.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
