"""Per-operator definitions of the decoder forward, in fp64 on the CPU.

Test infrastructure only.  Nothing on the product path imports this.

The method does not change what the forward computes; it pins how every
reduction is ordered so that one row's result never depends on the batch,
the phase or the caller (page "Finish RL Training Faster" digest, sections
"零差异需要一个精确的比较对象" and "让训练前向使用推理的数值").  The oracle
therefore computes the plain mathematical definition of each operator in
fp64, rounding to bf16 exactly where the product path stores a bf16 tensor.
It does not imitate any reduction order.

Conventions: bf16 tensors travel as uint16 bit patterns; ``bf`` rounds a
float64 value to bf16 (ties to even) and returns float64.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_decode, bf16_round, e4m3_decode, e4m3_encode

bf = bf16_round
dec = bf16_decode


# --------------------------------------------------------------- add + RMSNorm

def add_rmsnorm(a, r, g, eps: float):
    """Fused residual add + RMSNorm.

    The vLLM/TorchTitan digest names RMSNorm with an added residual as one of
    the fused ops imported into the training forward (page "No More
    Train-Inference Mismatch", section "方法细节").  Reading: the residual is
    bf16; ``r <- bf(a + r)`` (skipped when ``a`` is None, the first norm of
    layer 0); ``h = bf(r * (mean(r^2) + eps)^(-1/2) * g)`` with the mean over
    the rounded residual.  All arguments are float64 arrays [rows, H] / [H].
    Returns (r, h) as float64 values on the bf16 grid.
    """
    r = np.asarray(r, dtype=np.float64)
    if a is not None:
        r = bf(np.asarray(a, dtype=np.float64) + r)
    ms = np.mean(r * r, axis=-1, keepdims=True)
    h = bf(r / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64))
    return r, h


# ------------------------------------------------------------------- linear

def linear(x, w):
    """y = x . w^T in fp64 (w row-major [out, in], as stored).  Not rounded."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def silu_mul(g, u):
    """SiLU-gated product of the MLP: bf(silu(g) * u) with g, u already bf16
    (page "No More Train-Inference Mismatch", section "方法细节", fused SiLU MLP)."""
    return bf(silu(g) * np.asarray(u, dtype=np.float64))


def mlp(h, wgu, wd, inter: int):
    """SiLU-gated MLP: g, u = bf(h W_gate^T), bf(h W_up^T); act = bf(silu(g) u);
    out = bf(act W_down^T).  The fused gate_up weight holds gate rows then up rows."""
    gu = bf(linear(h, wgu))
    act = silu_mul(gu[:, :inter], gu[:, inter:])
    return bf(linear(act, wd))


# --------------------------------------------------------------------- RoPE

def rope_tables(positions, head_dim: int, theta: float):
    """cos/sin of t * theta^(-2i/d) for i < d/2, computed in fp64 and rounded to fp32.
    Returns float64 arrays [len(positions), d/2] holding fp32 values."""
    half = head_dim // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang).astype(np.float32).astype(np.float64)
    s = np.sin(ang).astype(np.float32).astype(np.float64)
    return c, s


def rope(x, positions, theta: float):
    """Rotary embedding, half-split (NeoX) pairing (i, i + d/2), at absolute positions.
    x: float64 [T, heads, d] on the bf16 grid.  Returns bf16-grid float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    c, s = rope_tables(positions, d, theta)
    c, s = c[:, None, :], s[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return bf(np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1))


# ------------------------------------------------------------- FP8 KV cache

def kv_quantise(x):
    """Per-(token, head) e4m3 quantisation of a bf16 K or V row.

    The DeepSeek recipe keeps the KV cache in FP8 for every phase and the
    training recompute builds a private cache copy through the same FP8 round
    trip (page "Finish RL Training Faster" digest, section
    "让训练前向使用推理的数值").  The rule here is the reading for an e4m3
    cache with a per-token-per-head fp32 scale: a = max|x|;
    sigma = fp32(a / 448) (1 when a = 0); code = e4m3_rne(clamp(fp32(x/sigma), +-448)).
    The division and the scale are taken in fp32 because they decide an
    integer code.  x: float64 [..., d] on the bf16 grid.  Returns (codes uint8
    [..., d], sigma float32 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)
    sigma = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    q = x.astype(np.float32) / sigma[..., None]
    codes = e4m3_encode(np.clip(q.astype(np.float64), -448.0, 448.0))
    return codes, sigma


def kv_dequantise(codes, sigma):
    """x_hat = bf(fp32(e4m3(code)) * sigma), the product taken in fp32 (the stated
    rule of the cache format).  Returns bf16-grid float64 [..., d]."""
    v = e4m3_decode(codes).astype(np.float32)
    prod = v * np.asarray(sigma, dtype=np.float32)[..., None]
    return bf(prod.astype(np.float64))


def kv_roundtrip(x):
    return kv_dequantise(*kv_quantise(x))


# ---------------------------------------------------------------- attention

def causal_gqa_attention(q, k, v, q_pos, k_pos=None):
    """Causal grouped-query attention for one sequence, by definition.

    q: [Tq, nq, d], k/v: [Tk, nkv, d] float64 (bf16 grid); q_pos: absolute
    positions of the queries; k_pos: positions of the keys (default 0..Tk-1).
    Query head h reads kv head floor(h * nkv / nq).  s_j = q.k_j / sqrt(d)
    for k_pos_j <= q_pos; p = softmax(s); o = bf(sum_j p_j v_j).
    The pages require one attention operator for prefill, decode and the
    training recompute (page "Finish RL Training Faster" digest, sections
    "零差异需要一个精确的比较对象" and "让训练前向使用推理的数值"); the
    mathematical result is ordinary softmax attention.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, nq, d = q.shape
    Tk, nkv, _ = k.shape
    if k_pos is None:
        k_pos = np.arange(Tk)
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    grp = nq // nkv
    out = np.empty((Tq, nq, d), dtype=np.float64)
    mask = k_pos[None, :] <= q_pos[:, None]            # [Tq, Tk]
    for h in range(nq):
        g = h // grp
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p /= np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return bf(out)


# ----------------------------------------------------------------- logprobs

def logprobs(hf, emb, ids, vocab_block: int = 16384):
    """Log-probability of token ids[t] under softmax(hf[t] . E^T), in fp64.

    The compared quantity is the per-token logprob of valid response tokens
    (page "Finish RL Training Faster" digest, section "零差异需要一个精确的比较对象").
    Logits are never rounded to bf16.  ``emb`` is the bf16 bit matrix [V, H];
    it is decoded block by block to bound memory.  Returns fp32 [R].
    """
    hf = np.asarray(hf, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    V = emb.shape[0]
    R = hf.shape[0]
    zmax = np.full(R, -np.inf)
    blocks = []
    for v0 in range(0, V, vocab_block):
        z = hf @ dec(emb[v0:v0 + vocab_block]).T
        blocks.append(z)
        zmax = np.maximum(zmax, z.max(axis=1))
    ssum = np.zeros(R)
    zid = np.zeros(R)
    for b, v0 in zip(blocks, range(0, V, vocab_block)):
        ssum += np.exp(b - zmax[:, None]).sum(axis=1)
        sel = (ids >= v0) & (ids < v0 + b.shape[1])
        zid[sel] = b[sel, ids[sel] - v0]
    lse = zmax + np.log(ssum)
    return (zid - lse).astype(np.float32)


def full_logprobs(hf, emb):
    """All V logprobs per row (fp64) -- small vocabularies only (pins)."""
    z = np.asarray(hf, dtype=np.float64) @ dec(emb).T
    m = z.max(axis=1, keepdims=True)
    return z - m - np.log(np.exp(z - m).sum(axis=1, keepdims=True))


# ---------------------------------------------------------------------- MoE

def topk_ties(z, k: int):
    """Top-k experts per row ordered by (logit descending, expert index ascending).

    Discrete Top-K turns tiny numeric differences into different expert sets,
    so the tie rule must be fixed (page "Finish RL Training Faster" digest,
    section "零差异需要一个精确的比较对象"; MoE section of
    "让训练前向使用推理的数值").  Plain definition: a stable sort on the key
    (-z, index).  Returns int32 [T, k] slot lists.
    """
    z = np.asarray(z, dtype=np.float64)
    T, E = z.shape
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-z[t, e], e))
        out[t] = order[:k]
    return out


def topk_weights(z, ids):
    """Softmax over the selected logits, in fp64, in slot order."""
    z = np.asarray(z, dtype=np.float64)
    sel = np.take_along_axis(z, np.asarray(ids, dtype=np.int64), axis=1)
    e = np.exp(sel - sel[:, :1])
    return e / e.sum(axis=1, keepdims=True)


def moe_layer(h, ids, w, wgu, wd, swgu, swd, inter: int):
    """MoE block with one ungated shared expert.

    out = bf( sum_s w_s * y_{e_s} + y_shared ), where each expert output y is
    the SiLU-gated MLP of ``mlp`` (bf16 at its storage points).  The slot sum
    is the plain sum; the product path accumulates it in fp32 in slot order
    (page "Finish RL Training Faster" digest, section "让训练前向使用推理的数值":
    expert outputs return to the token's GPU and combine in FP32 in a fixed
    slot order).  h: float64 [T, H]; ids [T, k]; w [T, k]; wgu, wd: bf16 bit
    arrays [E, 2I, H], [E, H, I]; swgu, swd the shared expert.
    """
    h = np.asarray(h, dtype=np.float64)
    T, k = ids.shape
    acc = mlp(h, dec(swgu), dec(swd), inter).copy()
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        y = mlp(h[rows], dec(wgu[e]), dec(wd[e]), inter)
        acc[rows] += w[rows, slots][:, None] * y
    return bf(acc)


# ------------------------------------------------------ acceptance statistics

def acceptance_stats(lp_recompute, lp_rollout):
    """Diff statistics of the acceptance test: per valid response token
    delta = lp_recompute - lp_rollout (fp64); max|delta|, mean|delta|, std(delta)
    and the k3 estimator mean(expm1(delta) - delta) of KL, i.e. (r - 1) - log r
    with r = exp(delta).  All four must be exactly 0 (page "Finish RL Training
    Faster" digest, section "零差异需要一个精确的比较对象"; news page "A vLLM bitre
    azonosította...", section on the trainer calling the vLLM kernels)."""
    a = np.asarray(lp_recompute, dtype=np.float64)
    b = np.asarray(lp_rollout, dtype=np.float64)
    d = a - b
    if d.size == 0:
        return dict(max=0.0, mean=0.0, std=0.0, k3=0.0)
    return dict(max=float(np.max(np.abs(d))), mean=float(np.mean(np.abs(d))),
                std=float(np.std(d)), k3=float(np.mean(np.expm1(d) - d)))
