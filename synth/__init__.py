"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no norm, no matmul, no softmax, no quantiser).
Both sides receive exactly the same arrays from here, so a parity failure
can never come from the inputs.

Shapes follow the workloads of the pages:
  * the vLLM/TorchTitan digest runs Qwen3-1.7B RL on one host (page
    "No More Train-Inference Mismatch", sections "实验环境"/"实验结果");
  * the DeepSeek-V4-Flash report uses 128 prompts x 8 responses per step
    with an FP8 KV cache (page "train-inference-consistency", sections
    "两组结果" and "让训练前向使用推理的数值");
  * Nemotron trajectories are about 57K tokens long (same page, "两组结果").

The named datasets (GSM8K, DAPO-format maths, SWE-bench Pro subset) are not
used; uniform random token ids of the same length mix stand in for them.

Weights: fp32 standard normal times 0.02, rounded to bf16 by torch's CPU
cast (a library routine), generated per tensor from
``SeedSequence([seed, tensor_index])``.  RMSNorm gains are 1.0 (a gain drawn
from N(0, 0.02) would shrink every normalised activation ~50x and flatten
all logprobs toward -ln V); ``gain_noise=True`` draws 1 + N(0, 0.02) instead
so that tests exercise the gain indexing.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Tuple

import numpy as np
import torch

SEED_WEIGHTS = 1234
SEED_INPUTS = 5678
SEED_SHUFFLE = 9012


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


# 2 layers, hidden 256, 4 q / 2 kv heads of 64, SiLU-gated MLP 768, vocab 4096.
TINY = ModelConfig("tiny-decoder", 2, 256, 4, 2, 64, 768, 4096)
# Qwen3-1.7B shape: 28 layers, hidden 2048, 16 q / 8 kv heads of 128,
# MLP 6144, vocab 151936, tied embeddings.
QWEN3_1P7B = ModelConfig("qwen3-1.7b-shaped", 28, 2048, 16, 8, 128, 6144, 151936)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str = "moe-64x1536-top6"
    hidden: int = 4096
    n_experts: int = 64
    n_shared: int = 1
    top_k: int = 6
    expert_intermediate: int = 1536


MOE = MoEConfig()


def _rng(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch CPU tensor (torch's round-to-nearest-even cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16 tensor, as numpy uint16 (CPU copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def weight_specs(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Ordered (name, shape, kind) list; kind is "normal" or "gain".

    Linear weights are row-major [out, in].  The fused QKV weight stacks the
    q heads, then the k heads, then the v heads; the fused gate_up weight
    stacks the gate rows, then the up rows.  The embedding is tied to the
    lm_head.
    """
    H, d = cfg.hidden, cfg.head_dim
    specs = [("embed", (cfg.vocab, H), "normal")]
    for layer in range(cfg.n_layers):
        p = f"layers.{layer}."
        specs += [
            (p + "attn_norm", (H,), "gain"),
            (p + "wqkv", (cfg.qkv_rows, H), "normal"),
            (p + "wo", (H, cfg.n_q_heads * d), "normal"),
            (p + "mlp_norm", (H,), "gain"),
            (p + "wgu", (2 * cfg.intermediate, H), "normal"),
            (p + "wd", (H, cfg.intermediate), "normal"),
        ]
    specs.append(("final_norm", (H,), "gain"))
    return specs


def _draw(seed: int, index: int, shape, kind: str, gain_noise: bool) -> torch.Tensor:
    rng = _rng(seed, index)
    if kind == "gain":
        if gain_noise:
            x = 1.0 + 0.02 * rng.standard_normal(shape, dtype=np.float32)
        else:
            x = np.ones(shape, dtype=np.float32)
    else:
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(0.02)
    return to_bf16(x)


def make_weights(cfg: ModelConfig, seed: int = SEED_WEIGHTS, gain_noise: bool = False,
                 threads: int = 8) -> Dict[str, torch.Tensor]:
    """All model weights as bf16 CPU tensors, keyed by the names of weight_specs."""
    specs = weight_specs(cfg)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(_draw, seed, i, shape, kind, gain_noise)
                for i, (_, shape, kind) in enumerate(specs)]
        return {name: f.result() for (name, _, _), f in zip(specs, futs)}


@dataclasses.dataclass
class Sequence:
    """One prompt+response sequence.  Position t in [prompt_len-1, L-2] scores token t+1."""
    tokens: np.ndarray  # int32 [L]
    prompt_len: int

    @property
    def length(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def n_scored(self) -> int:
        return self.length - self.prompt_len


def tiny_sequences(cfg: ModelConfig = TINY, n: int = 8, seed: int = SEED_INPUTS,
                   min_len: int = 16, max_len: int = 64) -> List[Sequence]:
    """Lengths uniform in [min_len, max_len], prompt length uniform in [1, L-1]."""
    rng = _rng(seed, 0)
    out = []
    for _ in range(n):
        L = int(rng.integers(min_len, max_len + 1))
        P = int(rng.integers(1, L))
        toks = rng.integers(0, cfg.vocab, size=L, dtype=np.int64).astype(np.int32)
        out.append(Sequence(toks, P))
    return out


def rl_sequences(cfg: ModelConfig = QWEN3_1P7B, n_prompts: int = 128, n_responses: int = 8,
                 seed: int = SEED_INPUTS, prompt_range=(80, 250), response_range=(100, 400)
                 ) -> List[Sequence]:
    """GRPO-style batch: each prompt is shared by n_responses sequences, each with its own
    response (and its own KV; no prefix sharing).  Lengths are uniform in the given ranges."""
    rng = _rng(seed, 1)
    out = []
    for _ in range(n_prompts):
        P = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
        prompt = rng.integers(0, cfg.vocab, size=P, dtype=np.int64).astype(np.int32)
        for _ in range(n_responses):
            R = int(rng.integers(response_range[0], response_range[1] + 1))
            resp = rng.integers(0, cfg.vocab, size=R, dtype=np.int64).astype(np.int32)
            out.append(Sequence(np.concatenate([prompt, resp]), P))
    return out


def shuffled(seqs: List[Sequence], seed: int = SEED_SHUFFLE, index: int = 0) -> List[int]:
    """A seeded permutation of range(len(seqs))."""
    return [int(i) for i in _rng(seed, index).permutation(len(seqs))]


# ----------------------------------------------------------------- isolated ops

def lmhead_inputs(M: int, hidden: int = 2048, vocab: int = 151936, seed: int = SEED_INPUTS
                  ) -> Tuple[torch.Tensor, torch.Tensor, np.ndarray]:
    """Hidden states N(0,1) [M, hidden] bf16, weight N(0,0.02) [vocab, hidden] bf16,
    ids uniform over the vocabulary.  Row i is the same for every M (prefix of one draw)."""
    Mmax = max(M, 8192)
    rng = _rng(seed, 3)
    hs = rng.standard_normal((Mmax, hidden), dtype=np.float32)[:M]
    ids = rng.integers(0, vocab, size=Mmax, dtype=np.int64).astype(np.int32)[:M]
    w = _rng(seed, 4).standard_normal((vocab, hidden), dtype=np.float32)
    w *= np.float32(0.02)
    return to_bf16(hs), to_bf16(w), ids


def gemm_inputs(M: int, N: int, K: int, seed: int = SEED_INPUTS, index: int = 5,
                a_scale: float = 1.0, w_scale: float = 0.02) -> Tuple[torch.Tensor, torch.Tensor]:
    rng = _rng(seed, index)
    a = rng.standard_normal((M, K), dtype=np.float32) * np.float32(a_scale)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_scale)
    return to_bf16(a), to_bf16(w)


def normal_bf16(shape, seed: int = SEED_INPUTS, index: int = 6, scale: float = 1.0) -> torch.Tensor:
    x = _rng(seed, index).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return to_bf16(x)


def moe_weights(cfg: MoEConfig = MOE, seed: int = SEED_WEIGHTS, threads: int = 8
                ) -> Dict[str, torch.Tensor]:
    """Routed experts stacked: wgu [E, 2*I, H] (gate rows then up rows), wd [E, H, I];
    shared expert: swgu [2*I, H], swd [H, I]; router wr [E, H].  All N(0, 0.02) bf16."""
    H, I, E = cfg.hidden, cfg.expert_intermediate, cfg.n_experts
    specs = [("wgu", (E, 2 * I, H)), ("wd", (E, H, I)), ("swgu", (2 * I, H)),
             ("swd", (H, I)), ("wr", (E, H))]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(_draw, seed, 100 + i, shape, "normal", False)
                for i, (_, shape) in enumerate(specs)]
        return {name: f.result() for (name, _), f in zip(specs, futs)}


def router_logits_quantised(T: int, E: int = 64, seed: int = SEED_INPUTS,
                            adversarial: bool = True) -> np.ndarray:
    """fp32 router logits that are integers in [-128, 128] divided by 64, so ties are
    frequent.  With ``adversarial`` the first rows are all-equal, and rows with a 7-way
    tie straddling rank 6 follow."""
    rng = _rng(seed, 7)
    z = rng.integers(-128, 129, size=(T, E), dtype=np.int64).astype(np.float32) / np.float32(64)
    if adversarial and T >= 1:
        z[0, :] = np.float32(0.25)
        for r in range(1, min(T, 4)):
            row = rng.integers(-128, 0, size=E, dtype=np.int64).astype(np.float32) / np.float32(64)
            hi = rng.choice(E, size=3, replace=False)
            tie = rng.choice(np.setdiff1d(np.arange(E), hi), size=7, replace=False)
            row[hi] = np.float32(1.5)
            row[tie] = np.float32(0.5)
            z[r] = row
    return z


def fp8_attention_inputs(n_q: int, n_kv: int, head_dim: int, ctx: int, seed: int = SEED_INPUTS
                         ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """q [ctx, n_q, d], k and v [ctx, n_kv, d], bf16 N(0,1) -- one long sequence."""
    rng = _rng(seed, 8)
    q = rng.standard_normal((ctx, n_q, head_dim), dtype=np.float32)
    k = rng.standard_normal((ctx, n_kv, head_dim), dtype=np.float32)
    v = rng.standard_normal((ctx, n_kv, head_dim), dtype=np.float32)
    return to_bf16(q), to_bf16(k), to_bf16(v)


def sparse_index_inputs(T: int, n_keys: int, heads: int = 64, dim: int = 128,
                        exact: bool = True, seed: int = SEED_INPUTS, index: int = 9
                        ) -> Tuple[torch.Tensor, np.ndarray, torch.Tensor]:
    """Inputs of the sparse-attention indexer: index queries q_idx [T, heads, dim] bf16,
    head weights w [T, heads] fp32 and index keys k_idx [n_keys, dim] bf16.

    exact=True draws small integers so that every score is an exactly representable
    fp32 value whatever the summation order (ties are frequent): q_idx in [-2, 2],
    k_idx in [-7, 7] with one entry of each row set to +-7 (its FP8 scale is then
    7/448 = 2^-6 and the codes are exact), w = +-2^j with j in [-2, 1].
    exact=False draws N(0, 1) queries and keys and N(0, 1)/sqrt(heads) weights."""
    rng = _rng(seed, index)
    if exact:
        q = rng.integers(-2, 3, size=(T, heads, dim)).astype(np.float32)
        k = rng.integers(-7, 8, size=(n_keys, dim)).astype(np.float32)
        if n_keys:
            col = rng.integers(0, dim, size=n_keys)
            k[np.arange(n_keys), col] = np.where(rng.random(n_keys) < 0.5, -7.0, 7.0)
        w = (np.ldexp(1.0, rng.integers(-2, 2, size=(T, heads)))
             * np.where(rng.random((T, heads)) < 0.25, -1.0, 1.0)).astype(np.float32)
    else:
        q = rng.standard_normal((T, heads, dim), dtype=np.float32)
        k = rng.standard_normal((n_keys, dim), dtype=np.float32)
        w = rng.standard_normal((T, heads), dtype=np.float32) / np.float32(np.sqrt(heads))
    return to_bf16(q), w, to_bf16(k)


def ssd_inputs(T: int, heads: int = 128, head_dim: int = 64, d_state: int = 128, groups: int = 8,
               seed: int = SEED_INPUTS, index: int = 12) -> Dict[str, object]:
    """Inputs of a Mamba-2-style state-space layer for T positions: x [T, heads, head_dim]
    bf16 N(0, 1); dt [T, heads] fp32 log-uniform in [1e-3, 1e-1] (the step after its
    softplus); A [heads] fp32 = -exp(U(0, ln 16)); B, C [T, groups, d_state] bf16 N(0, 1);
    D [heads] fp32 = 1 + 0.1 N(0, 1)."""
    rng = _rng(seed, index)
    x = rng.standard_normal((T, heads, head_dim), dtype=np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (T, heads))).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), heads))).astype(np.float32)
    B = rng.standard_normal((T, groups, d_state), dtype=np.float32)
    C = rng.standard_normal((T, groups, d_state), dtype=np.float32)
    D = (1.0 + 0.1 * rng.standard_normal(heads)).astype(np.float32)
    return dict(x=to_bf16(x), dt=dt, A=A, B=to_bf16(B), C=to_bf16(C), D=D)
