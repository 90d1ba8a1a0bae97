"""The dense decoder forward that recomputes per-token logprobs, in fp64.

Test infrastructure only.

What is computed (page "Finish RL Training Faster" digest, section
"零差异需要一个精确的比较对象"): for one sequence of prompt length P and
total length L, under fixed weights, the logprob of every valid response
token, i.e. of token t+1 given tokens 0..t for t = P-1 .. L-2.  The last
token is scored but never forwarded.  Each sequence is independent; there is
no padding.

Layer structure (page "No More Train-Inference Mismatch", section "方法细节":
SiLU MLPs and RMSNorms with added residual connections), pre-norm:

    r = E[x]                                  (layer 0 norm takes no add)
    per layer:  r, h  = AddNorm(m_prev, r, g_attn)
                q,k,v = split(bf(h Wqkv^T));  q,k = RoPE(q,k)
                (FP8 cache: k,v <- dequant(quant(k,v)) for every key)
                a     = bf(Attn(q, k, v) Wo^T)
                r, h2 = AddNorm(a, r, g_mlp)
                m     = MLP(h2)
    r, hf = AddNorm(m, r, g_final);   lp_t = log softmax(hf_t E^T)[x_{t+1}]

``forward_chunks`` takes any split of the sequence into consecutive chunks
with a KV cache carried between them; whole-sequence prefill is one chunk and
token-by-token decode is chunks of one.  ``weights`` is a mapping from the
tensor names (embed, layers.{i}.attn_norm, .wqkv, .wo, .mlp_norm, .wgu, .wd,
final_norm) to bf16 bit arrays (uint16).
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import ops
from .codecs import bf16_decode


class Weights:
    """Lazily decoded fp64 copies of bf16 weight bits (cached when ``cache``)."""

    def __init__(self, bits: Dict[str, np.ndarray], cache: bool = True):
        self.bits = bits
        self.cache = cache
        self._f64: Dict[str, np.ndarray] = {}

    def __call__(self, name: str) -> np.ndarray:
        if name in self._f64:
            return self._f64[name]
        v = bf16_decode(self.bits[name])
        if self.cache:
            self._f64[name] = v
        return v

    def raw(self, name: str) -> np.ndarray:
        return self.bits[name]


def _embed(W: Weights, ids) -> np.ndarray:
    return bf16_decode(W.raw("embed")[np.asarray(ids, dtype=np.int64)])


def decoder_layer(cfg, W: Weights, li: int, m_prev, r, pos, cache_k, cache_v,
                  kv_dtype: str = "bf16") -> dict:
    """One decoder layer for a chunk of consecutive positions ``pos``.

    m_prev: the previous layer's MLP output (None for layer 0, whose first norm
    takes no add); r: the residual entering the layer; cache_k/cache_v: this
    layer's keys/values of the positions before the chunk.  Returns the layer's
    tensors, including the updated residual ``r`` and MLP output ``m``.
    """
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    n = len(pos)
    p = f"layers.{li}."
    r, h = ops.add_rmsnorm(m_prev, r, W(p + "attn_norm"), cfg.rms_eps)
    r_mid = r
    qkv = ops.bf(ops.linear(h, W(p + "wqkv")))
    q = qkv[:, : nq * d].reshape(n, nq, d)
    k = qkv[:, nq * d: (nq + nkv) * d].reshape(n, nkv, d)
    v = qkv[:, (nq + nkv) * d:].reshape(n, nkv, d)
    q = ops.rope(q, pos, cfg.rope_theta)
    k = ops.rope(k, pos, cfg.rope_theta)
    if kv_dtype == "fp8":
        k = ops.kv_roundtrip(k)
        v = ops.kv_roundtrip(v)
    K = np.concatenate([cache_k, k], axis=0)
    V = np.concatenate([cache_v, v], axis=0)
    o = ops.causal_gqa_attention(q, K, V, pos)
    a = ops.bf(ops.linear(o.reshape(n, nq * d), W(p + "wo")))
    r, h2 = ops.add_rmsnorm(a, r, W(p + "mlp_norm"), cfg.rms_eps)
    m = ops.mlp(h2, W(p + "wgu"), W(p + "wd"), cfg.intermediate)
    return dict(layer=li, r_mid=r_mid, h=h, q=q, k=k, v=v, K=K, V=V, o=o, a=a, r=r, h2=h2, m=m)


def forward_chunks(cfg, W: Weights, tokens, chunks: List[int], kv_dtype: str = "bf16",
                   dump: Optional[list] = None) -> np.ndarray:
    """Forward positions 0 .. sum(chunks)-1 in consecutive chunks; returns the final
    normed hidden states hf (float64 on the bf16 grid) for every forwarded position.

    ``dump``, when a list, receives the per-layer dicts of ``decoder_layer``.
    """
    nkv, d = cfg.n_kv_heads, cfg.head_dim
    tokens = np.asarray(tokens)
    cache_k = [np.zeros((0, nkv, d)) for _ in range(cfg.n_layers)]
    cache_v = [np.zeros((0, nkv, d)) for _ in range(cfg.n_layers)]
    outs = []
    p0 = 0
    for n in chunks:
        pos = np.arange(p0, p0 + n)
        r = _embed(W, tokens[p0:p0 + n])
        m = None
        for li in range(cfg.n_layers):
            out = decoder_layer(cfg, W, li, m, r, pos, cache_k[li], cache_v[li], kv_dtype)
            cache_k[li], cache_v[li] = out.pop("K"), out.pop("V")
            r, m = out["r"], out["m"]
            if dump is not None:
                out["p0"] = p0
                dump.append(out)
        r, hf = ops.add_rmsnorm(m, r, W("final_norm"), cfg.rms_eps)
        outs.append(hf)
        p0 += n
    return np.concatenate(outs, axis=0)


def sequence_logprobs(cfg, W: Weights, tokens, prompt_len: int, kv_dtype: str = "bf16",
                      chunks: Optional[List[int]] = None, dump: Optional[list] = None
                      ) -> np.ndarray:
    """fp32 logprobs of tokens[prompt_len:] (one per valid response token)."""
    tokens = np.asarray(tokens)
    L = tokens.shape[0]
    T = L - 1
    if L - prompt_len <= 0:
        return np.zeros(0, dtype=np.float32)
    if chunks is None:
        chunks = [T]
    assert sum(chunks) == T
    hf = forward_chunks(cfg, W, tokens, chunks, kv_dtype, dump)
    rows = hf[prompt_len - 1: T]
    return ops.logprobs(rows, W.raw("embed"), tokens[prompt_len:])
